// Indexer score pass: I[t,s] = sum_h w[t,h] * max(0, qI[t,h,:] . kI[s,:]) for s < n_t.
//
// Source: "A.X-K2: a sparse-attention upgrade that costs nothing, trained
// natively in FP8", section "Sparse Gated Attention" (a lightweight indexer
// scores every cached key for each query); "A.X-K2" model card, section
// "Sparse Gated Attention (SGA)" (the indexer scores and ranks key-value
// candidates). The weighted-ReLU form is the reading this library implements.
//
// Three kernels:
//  * k_index_f32: generic fp32 path, one thread per (query, key).
//  * k_index_fp8: MI355X path for 64 index heads x 128 dims in E4M3FN, one
//    query per workgroup row of the grid (decode). Each wave keeps the
//    query's 64 x 128 index matrix in registers as four 16 x 128 MFMA A tiles
//    and streams its own range of keys through LDS (LDS-DMA, two 8 KiB tiles
//    in flight). One 16x16x128 FP8 MFMA per (head tile, 16-key tile) gives 16
//    heads x 16 keys; the ReLU and the weighted head sum run on the
//    accumulators, and lane-swap additions leave one finished score per lane,
//    stored coalesced.
//  * k_index_fp8_pf: the same arithmetic for runs of query rows of one
//    sequence (prefill): the workgroup's waves share each LDS key tile.
// k_index_f32 and k_index_fp8 can also build the level-0 histogram (top 12
// bits of the score key) the top-k select starts from, so the layer never
// re-reads the scores for it.

#include "kernels.h"

namespace sga {

namespace {

__device__ __forceinline__ void hist_flush(uint32_t *lds_hist, uint32_t *g_hist) {
  __syncthreads();
  for (int i = threadIdx.x; i < kHist0Bins; i += blockDim.x) {
    uint32_t c = lds_hist[i];
    if (c) atomicAdd(g_hist + i, c);
  }
}

__device__ __forceinline__ void hist_zero(uint32_t *lds_hist) {
  for (int i = threadIdx.x; i < kHist0Bins; i += blockDim.x) lds_hist[i] = 0u;
  __syncthreads();
}

// Query rows are grouped in runs of kPfGroup for the prefill kernel. A group is
// "shared" when all of its rows name the same sequence; the prefill kernel
// scores exactly those groups and the per-query kernel skips them.
constexpr int kPfGroup = 8;

__device__ __forceinline__ bool group_is_shared(const SeqMeta &m, int T, int g) {
  const int t0 = g * kPfGroup;
  const int t1 = min(T, t0 + kPfGroup);
  const int32_t b = m.q_seq[t0];
  bool same = true;
  for (int t = t0 + 1; t < t1; ++t) same = same && (m.q_seq[t] == b);
  return same;
}

// --------------------------------------------------------------------------
// fp32 path
// --------------------------------------------------------------------------
constexpr int kF32Block = 256;
constexpr int kF32MaxQ = 8192;  // HI * DI

__global__ __launch_bounds__(kF32Block) void k_index_f32(SeqMeta m, int k, int HI, int DI,
                                                         const float *__restrict__ q_idx,
                                                         const float *__restrict__ w,
                                                         const float *__restrict__ k_idx,
                                                         float *__restrict__ scores,
                                                         int64_t stride, TopkWs sel) {
  __shared__ float qs[kF32MaxQ];
  __shared__ float ws[64];
  __shared__ uint32_t hist[kHist0Bins];
  const bool want_hist = sel.hist0 != nullptr;
  const int t = blockIdx.y;
  int64_t start;
  const int n = query_candidates(m, t, &start);
  const int base = blockIdx.x * kF32Block;
  if (base >= n) return;
  for (int i = threadIdx.x; i < HI * DI; i += kF32Block) qs[i] = q_idx[(size_t)t * HI * DI + i];
  for (int i = threadIdx.x; i < HI; i += kF32Block) ws[i] = w[(size_t)t * HI + i];
  if (want_hist) hist_zero(hist);
  __syncthreads();
  const int s = base + threadIdx.x;
  if (s < n) {
    const float *kr = k_idx + (start + s) * (int64_t)DI;
    float acc = 0.0f;
    for (int h = 0; h < HI; ++h) {
      float d = 0.0f;
      for (int j = 0; j < DI; ++j) d = fmaf(qs[h * DI + j], kr[j], d);
      acc = fmaf(fmaxf(d, 0.0f), ws[h], acc);
    }
    acc += 0.0f;  // -0 -> +0
    scores[t * stride + s] = acc;
    if (want_hist) atomicAdd(&hist[score_key(acc) >> kHist0Shift], 1u);
  }
  if (want_hist) hist_flush(hist, sel.hist0 + (size_t)t * kHist0Bins);
}

// --------------------------------------------------------------------------
// FP8 MFMA path (HI = 64, DI = 128)
//
// Each wave streams its own contiguous range of keys. 64-key tiles (8 KiB)
// are copied global -> LDS with LDS-DMA (global_load_lds_dwordx4): every DMA
// instruction moves 1 KiB of consecutive bytes, and two tiles per wave are in
// flight. The MFMA B operand is then read from LDS in the layout the
// 16x16x128 FP8 MFMA wants. Within a 128-byte key row the 32-byte segments are
// XOR-swizzled by key so that the 16 keys read by one instruction spread over
// the LDS banks; the swizzle is applied on the DMA source side.
// --------------------------------------------------------------------------
constexpr int kIdxWaves = 4;                 // waves per workgroup
constexpr int kIdxTileKeys = 64;             // keys per DMA tile
constexpr int kIdxTileBytes = kIdxTileKeys * 128;
constexpr int kIdxDmaPerTile = kIdxTileBytes / (64 * 16);  // 8 DMA issues per lane
constexpr int kIdxBufs = 2;                  // tiles in flight per wave
constexpr size_t kIdxSmem = (size_t)kIdxWaves * kIdxBufs * kIdxTileBytes;

typedef __attribute__((address_space(3))) void lds_void;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ v4f mfma_fp8(const v8i &a, const v8i &b, const v4f &c) {
  // E4M3 x E4M3 (format code 0), unit E8M0 scales (127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// LDS atomic add without a return value, issued as inline asm so that the
// compiler does not make it wait for the wave's in-flight LDS-DMA copies
// (it cannot tell that the histogram and the DMA buffers do not overlap).
// It has no result register; later lgkmcnt waits cover its completion.
__device__ __forceinline__ void lds_add_u32(uint32_t *p, uint32_t v) {
  const uint32_t addr =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t *)p;
  asm volatile("ds_add_u32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

// Piece swizzle of key row r in LDS: the 16-byte piece q of the row is
// stored at piece q ^ key_swz(r). A ds_read_b128 of the B operand serves 16
// lanes at a time, 16 consecutive rows with one piece each; rows r and r + 1
// sit half the banks apart, and (r >> 1) & 7 spreads each row pair over all
// eight piece positions, so every 16-lane group hits 64 distinct banks.
__device__ __forceinline__ int key_swz(int r) { return (r >> 1) & 7; }

// B operand of key tile kt (keys 16 kt .. 16 kt + 15 of a 64-key LDS tile):
// key 16 kt + c16, bytes [32 kg, 32 kg + 32) of its 128-byte row.
__device__ __forceinline__ v8i load_key_operand(const unsigned char *tb, int kt, int kg, int c16) {
  const int r = kt * 16 + c16;
  const unsigned char *row = tb + r * 128;
  const v4i lo = *(const v4i *)(row + (((2 * kg) ^ key_swz(r)) << 4));
  const v4i hi = *(const v4i *)(row + (((2 * kg + 1) ^ key_swz(r)) << 4));
  return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// Weighted-ReLU head sums of kQ queries over one 64-key LDS tile: part[j][kt]
// (lane l) is the sum, over the 16 heads this lane's accumulator rows cover,
// of w[h] * max(0, qI[h] . k) for query j and key 16 kt + l % 16.
//
// On gfx950 MFMA and VALU time add up on a SIMD (measured: they do not
// overlap), so the epilogue (a max and an FMA per accumulator element) is
// kept as short as it can be; each sum is split over two accumulators so
// that consecutive FMAs do not wait on each other. The B operand is read
// per key tile, which also bounds how many MFMA results are live at once.
template <int kQ>
__device__ __forceinline__ void score_tiles(const v8i (&a)[kQ][4], const unsigned char *tb, int kg,
                                            int c16, const float (&wv)[kQ][16],
                                            float (&part)[kQ][4]) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const v8i b = load_key_operand(tb, kt, kg, c16);
#pragma unroll
    for (int j = 0; j < kQ; ++j) {
      float ev = 0.0f, od = 0.0f;
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        const v4f x = mfma_fp8(a[j][ht], b, zero);
        const float *wr = &wv[j][ht * 4];
        ev = fmaf(fmaxf(x[0], 0.0f), wr[0], ev);
        od = fmaf(fmaxf(x[1], 0.0f), wr[1], od);
        ev = fmaf(fmaxf(x[2], 0.0f), wr[2], ev);
        od = fmaf(fmaxf(x[3], 0.0f), wr[3], od);
      }
      part[j][kt] = ev + od;
    }
  }
}

__device__ __forceinline__ float add_swapped(float x, float y, bool wide) {
  // lanes of x and y exchanged across the two 32-lane halves (wide) or across
  // neighbouring 16-lane rows; the two results summed
  const auto r = wide ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false)
                      : __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Reduce-scatter of part[0..3] over the lanes l, l^16, l^32, l^48 that hold
// partial sums of the same keys: lane l returns the score of key l of the
// tile (-0 becomes +0). Lane-swap instructions of gfx950 do the exchange:
// across the halves, lane l < 32 gets part[0] (part[1]) of lanes l and l + 32
// and lane l >= 32 part[2] (part[3]) of lanes l - 32 and l; then across
// 16-lane rows, even rows keep the first sum and odd rows the second.
__device__ __forceinline__ float tile_scores(const float (&part)[4]) {
  const float k0 = add_swapped(part[0], part[2], true);
  const float k1 = add_swapped(part[1], part[3], true);
  return add_swapped(k0, k1, false) + 0.0f;
}


// Global byte offset of the 16-byte piece that lane `lane` copies with DMA
// issue i, relative to row 8 i of the tile: piece 64 i + lane of the LDS tile
// holds key row r = 8 i + lane / 8 and global piece (lane % 8) ^ key_swz(r);
// key_swz(r) only depends on the lane and on the parity of i.
__device__ __forceinline__ int key_dma_offset(int lane, int i) {
  const int r = 8 * i + (lane >> 3);
  return (lane >> 3) * 128 + (((lane & 7) ^ key_swz(r)) << 4);
}

// Issue the DMA of one 64-key tile (keys base.., clamped to n-1) into `buf`.
__device__ __forceinline__ void issue_key_tile(unsigned char *buf, const uint8_t *__restrict__ k_idx,
                                               int64_t start, int n, int base, int lane,
                                               const int (&lane_off)[2]) {
  if (base + kIdxTileKeys <= n) {
    const uint8_t *src = k_idx + (start + base) * 128;
#pragma unroll
    for (int i = 0; i < kIdxDmaPerTile; ++i)
      __builtin_amdgcn_global_load_lds(src + i * 1024 + lane_off[i & 1], (lds_void *)(buf + i * 1024),
                                       16, 0, 0);
  } else {
    // sequence tail: rows past the end repeat the last key (their scores are dropped)
#pragma unroll
    for (int i = 0; i < kIdxDmaPerTile; ++i) {
      const int r = i * 8 + (lane >> 3);
      int key = base + r;
      key = key < n ? key : n - 1;
      const uint8_t *src = k_idx + (start + key) * 128 + (lane_off[i & 1] & 127);
      __builtin_amdgcn_global_load_lds(src, (lds_void *)(buf + i * 1024), 16, 0, 0);
    }
  }
}

template <bool kHist>
__global__ __launch_bounds__(kIdxWaves * 64) void k_index_fp8(SeqMeta m, int T, int k, int iters,
                                                              int skip_shared,
                                                              const uint8_t *__restrict__ q_idx,
                                                              const float *__restrict__ w,
                                                              const uint8_t *__restrict__ k_idx,
                                                              float *__restrict__ scores,
                                                              int64_t stride, TopkWs sel) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // level-0 histogram with two 16-bit bins per word (a workgroup scores at most
  // 4 x 32 x 64 = 8192 keys, so a bin cannot overflow)
  __shared__ uint32_t hist[kHist ? kHist0Bins / 2 : 1];
  const int t = blockIdx.y;
  int64_t start;
  const int n = query_candidates(m, t, &start);
  const int wave_keys = iters * kIdxTileKeys;
  const int chunk0 = blockIdx.x * kIdxWaves * wave_keys;
  if (chunk0 >= n) return;
  if (skip_shared && group_is_shared(m, T, t / kPfGroup)) return;  // scored by k_index_fp8_pf
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kg = lane >> 4, c16 = lane & 15;

  // A tiles: head (ht*16 + c16), bytes [32*kg, 32*kg+32) of its 128-byte row
  v8i a[1][4];
  float wv[1][16];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const v4i *src = (const v4i *)(q_idx + ((size_t)t * 64 + ht * 16 + c16) * 128 + kg * 32);
    const v4i lo = src[0], hi = src[1];
    a[0][ht] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    // accumulator row r of this lane is head ht*16 + 4*kg + r
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[0][ht * 4 + r] = w[(size_t)t * 64 + ht * 16 + 4 * kg + r];
  }
  if (kHist) {
    for (int i = threadIdx.x; i < kHist0Bins / 2; i += kIdxWaves * 64) hist[i] = 0u;
    __syncthreads();
  }

  const int wbase = chunk0 + wave * wave_keys;
  const int nit = wbase < n ? min(iters, (n - wbase + kIdxTileKeys - 1) / kIdxTileKeys) : 0;
  unsigned char *mybuf = smem + (size_t)wave * kIdxBufs * kIdxTileBytes;
  const int lane_off[2] = {key_dma_offset(lane, 0), key_dma_offset(lane, 1)};
  // the q/w loads above must have landed before the DMA counting starts
  wait_vmcnt<0>();
  if (nit > 0) issue_key_tile(mybuf, k_idx, start, n, wbase, lane, lane_off);
  if (nit > 1) issue_key_tile(mybuf + kIdxTileBytes, k_idx, start, n, wbase + kIdxTileKeys, lane, lane_off);
  float *srow = scores + t * stride;
  for (int it = 0; it < nit; ++it) {
    // Outstanding vector-memory ops issued after tile `it`: the score store of
    // iteration it-1 (if any) and the DMA of tile it+1 (if any). They retire in
    // order, so waiting down to that many guarantees tile `it` has landed.
    const int later = (it > 0 ? 1 : 0) + (it + 1 < nit ? kIdxDmaPerTile : 0);
    if (later == kIdxDmaPerTile + 1) wait_vmcnt<kIdxDmaPerTile + 1>();
    else if (later == kIdxDmaPerTile) wait_vmcnt<kIdxDmaPerTile>();
    else if (later == 1) wait_vmcnt<1>();
    else wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    const unsigned char *tb = mybuf + (it & 1) * kIdxTileBytes;
    float part[1][4];
    score_tiles<1>(a, tb, kg, c16, wv, part);
    const float keep = tile_scores(part[0]);
    const int s = wbase + it * kIdxTileKeys + lane;
    // the tile buffer is free once this iteration's LDS reads completed
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    if (s < n) srow[s] = keep;
    if (it + 2 < nit)
      issue_key_tile(mybuf + (it & 1) * kIdxTileBytes, k_idx, start, n,
                     wbase + (it + 2) * kIdxTileKeys, lane, lane_off);
    if (kHist && s < n) {
      const uint32_t bin = score_key(keep) >> kHist0Shift;
      lds_add_u32(&hist[bin >> 1], (bin & 1) ? 65536u : 1u);
    }
  }
  if (kHist) {
    __syncthreads();
    uint32_t *g = sel.hist0 + (size_t)t * kHist0Bins;
    for (int i = threadIdx.x; i < kHist0Bins / 2; i += kIdxWaves * 64) {
      const uint32_t c = hist[i];
      if (c & 0xFFFFu) atomicAdd(g + 2 * i, c & 0xFFFFu);
      if (c >> 16) atomicAdd(g + 2 * i + 1, c >> 16);
    }
  }
}

// --------------------------------------------------------------------------
// Prefill: many queries of one sequence share every key tile.
//
// A workgroup owns a group of 8 query rows of one sequence (8 / kQpw waves of
// kQpw queries; each wave keeps its 64 x 128 index matrices in VGPRs) and a
// range of 8192 keys. Key tiles of 64 keys are copied once into LDS with
// LDS-DMA and reused by all 16 queries, so the pass is bound by the MFMAs and
// the ReLU/weight epilogue instead of by HBM. Three tile buffers let one
// barrier per tile both publish tile i and free the buffer that tile i + 2
// overwrites. Keys past a query's own position are neither scored nor stored.
// --------------------------------------------------------------------------
constexpr int kPfChunk = 8192;  // keys per workgroup
constexpr int kPfQpw = 1;       // queries per wave
constexpr int kPfBufs = 3;

// kQpw queries per wave, kPfGroup / kQpw waves per workgroup. MFMA and VALU
// time add up on a SIMD, so latency is hidden by wave count: the register
// budget is held to 6 waves per SIMD (3 workgroups per CU).
template <int kQpw>
__global__ __launch_bounds__(kPfGroup / kQpw * 64, 6) void k_index_fp8_pf(SeqMeta m, int T,
                                                                const uint8_t *__restrict__ q_idx,
                                                                const float *__restrict__ w,
                                                                const uint8_t *__restrict__ k_idx,
                                                                float *__restrict__ scores,
                                                                int64_t stride) {
  constexpr int kThreads = kPfGroup / kQpw * 64;
  static_assert(512 % kThreads == 0 || kThreads % 512 == 0, "a tile is 512 16-byte pieces");
  constexpr int kDmaPer = kThreads >= 512 ? 1 : 512 / kThreads;  // DMA issues per thread per tile
  // dynamic LDS: the compiler then leaves the DMA/LDS-read ordering to the
  // explicit waits below instead of draining every DMA before each read
  extern __shared__ __attribute__((aligned(16))) unsigned char tiles[];
  __shared__ int s_nmax;
  const int g = blockIdx.y;
  if (!group_is_shared(m, T, g)) return;  // left to the per-query kernel
  const int t0 = g * kPfGroup;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 4, c16 = lane & 15;
  int64_t start;
  if (tid == 0) {
    int mx = 0;
    for (int t = t0; t < min(T, t0 + kPfGroup); ++t) mx = max(mx, query_candidates(m, t, &start));
    s_nmax = mx;
  }
  __syncthreads();
  const int nmax = s_nmax;
  const int c0 = blockIdx.x * kPfChunk;
  if (c0 >= nmax) return;
  const int ntiles = (min(nmax, c0 + kPfChunk) - c0 + kIdxTileKeys - 1) / kIdxTileKeys;

  // the wave's queries (rows past T get n = 0)
  int nq[kQpw];
  v8i a[kQpw][4];
  float wv[kQpw][16];
#pragma unroll
  for (int j = 0; j < kQpw; ++j) {
    const int t = t0 + kQpw * wave + j;
    nq[j] = t < T ? query_candidates(m, t, &start) : 0;
    const int tt = t < T ? t : t0;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const v4i *src = (const v4i *)(q_idx + ((size_t)tt * 64 + ht * 16 + c16) * 128 + kg * 32);
      const v4i lo = src[0], hi = src[1];
      a[j][ht] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) wv[j][ht * 4 + r] = w[(size_t)tt * 64 + ht * 16 + 4 * kg + r];
    }
  }
  query_candidates(m, t0, &start);  // the group's sequence start
  // DMA pieces of this thread: piece p = u * kThreads + tid of the 8 KiB tile
  // holds tile row p / 8 and its swizzled 16-byte piece
  auto issue = [&](int i) {
#pragma unroll
    for (int u = 0; u < kDmaPer; ++u) {
      const int p = u * kThreads + tid;
      if (kThreads > 512 && p >= 512) break;  // wave-uniform: whole waves past the tile
      const int r = p >> 3;
      int key = c0 + i * kIdxTileKeys + r;
      key = key < nmax ? key : nmax - 1;
      const uint8_t *src = k_idx + (start + key) * 128 + (((p & 7) ^ key_swz(r)) << 4);
      __builtin_amdgcn_global_load_lds(
          src, (lds_void *)(tiles + (i % kPfBufs) * kIdxTileBytes + (u * kThreads + wave * 64) * 16),
          16, 0, 0);
    }
  };
  wait_vmcnt<0>();
  issue(0);
  if (ntiles > 1) issue(1);
  for (int i = 0; i < ntiles; ++i) {
    // Tile i has landed once at most the kDmaPer copies of tile i + 1 (issued
    // after it) are outstanding; score stores issued later only make this
    // wait longer. The barrier then publishes every wave's part of tile i and
    // certifies that all LDS reads of tile i - 1 are done, so the copy of
    // tile i + 2 may overwrite that buffer.
    if (i + 1 < ntiles) wait_vmcnt<kDmaPer>(); else wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (i + 2 < ntiles) issue(i + 2);
    const unsigned char *tb = tiles + (i % kPfBufs) * kIdxTileBytes;
    const int kbase = c0 + i * kIdxTileKeys;
    float part[kQpw][4];
    score_tiles<kQpw>(a, tb, kg, c16, wv, part);
    const int s = kbase + lane;
#pragma unroll
    for (int j = 0; j < kQpw; ++j) {
      const float keep = tile_scores(part[j]);
      if (s < nq[j]) scores[(size_t)(t0 + kQpw * wave + j) * stride + s] = keep;
    }
  }
}

}  // namespace

int index_fp8_iters(int T, int max_kv_len) {
  // aim for about eight 4-wave workgroups per CU over the whole batch
  const int64_t keys = (int64_t)T * max_kv_len;
  const int64_t per_iter = 2048LL * kIdxWaves * kIdxTileKeys;
  int64_t it = (keys + per_iter - 1) / per_iter;
  if (it < 2) it = 2;
  if (it > 32) it = 32;
  return (int)it;
}

namespace {
}  // namespace

hipError_t launch_index_f32(const SeqMeta &m, int T, int k, int HI, int DI, const float *q_idx,
                            const float *w, const float *k_idx, float *scores, int64_t stride,
                            const TopkWs *sel, hipStream_t s) {
  if (T == 0 || m.max_kv_len == 0) return hipSuccess;
  TopkWs none{};
  dim3 grid((m.max_kv_len + kF32Block - 1) / kF32Block, T);
  hipLaunchKernelGGL(k_index_f32, grid, dim3(kF32Block), 0, s, m, k, HI, DI, q_idx, w, k_idx,
                     scores, stride, sel ? *sel : none);
  return hipGetLastError();
}

hipError_t launch_index_fp8(const SeqMeta &m, int T, int k, const uint8_t *q_idx, const float *w,
                            const uint8_t *k_idx, float *scores, int64_t stride, const TopkWs *sel,
                            hipStream_t s) {
  if (T == 0 || m.max_kv_len == 0) return hipSuccess;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void *)k_index_fp8<true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kIdxSmem);
    (void)hipFuncSetAttribute((const void *)k_index_fp8<false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kIdxSmem);
    (void)hipGetLastError();
    attr = true;
  }
  // many query rows per sequence: score shared 16-row groups with the
  // query-tiled kernel, the rest with the per-query kernel
  const bool prefill = T >= 4 * kPfGroup && T >= 4 * m.num_seqs;
  const int iters = index_fp8_iters(T, m.max_kv_len);
  const int per_wg = kIdxWaves * iters * kIdxTileKeys;
  dim3 grid((m.max_kv_len + per_wg - 1) / per_wg, T);
  TopkWs none{};
  if (prefill) {
    dim3 pgrid((m.max_kv_len + kPfChunk - 1) / kPfChunk, (T + kPfGroup - 1) / kPfGroup);
    hipLaunchKernelGGL(k_index_fp8_pf<kPfQpw>, pgrid, dim3(kPfGroup / kPfQpw * 64), kPfBufs * kIdxTileBytes,
                       s, m, T, q_idx, w, k_idx, scores, stride);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_index_fp8<false>, grid, dim3(kIdxWaves * 64), kIdxSmem, s, m, T, k, iters,
                       1, q_idx, w, k_idx, scores, stride, none);
    e = hipGetLastError();
    if (e != hipSuccess || !sel) return e;
    return launch_topk_hist0(m, T, scores, stride, *sel, s);
  }
  if (sel)
    hipLaunchKernelGGL(k_index_fp8<true>, grid, dim3(kIdxWaves * 64), kIdxSmem, s, m, T, k, iters, 0,
                       q_idx, w, k_idx, scores, stride, *sel);
  else
    hipLaunchKernelGGL(k_index_fp8<false>, grid, dim3(kIdxWaves * 64), kIdxSmem, s, m, T, k, iters, 0,
                       q_idx, w, k_idx, scores, stride, none);
  return hipGetLastError();
}

}  // namespace sga
