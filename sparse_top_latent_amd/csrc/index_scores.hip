// Indexer score pass: I[t,s] = sum_h w[t,h] * max(0, qI[t,h,:] . kI[s,:]) for s < n_t.
//
// Source: "A.X-K2: a sparse-attention upgrade that costs nothing, trained
// natively in FP8", section "Sparse Gated Attention" (a cheap indexer rates
// each cached key for each query); "A.X-K2" model card, section
// "Sparse Gated Attention (SGA)" (the indexer rates and orders the cached
// candidates). The weighted-ReLU form is the reading this library implements.
//
// Three kernels (device helpers shared with the prefill kernel live in
// index_common.h):
//  * k_index_f32: generic fp32 path, one thread per (query, key).
//  * k_index_fp8: MI355X path for 64 index heads x 128 dims in E4M3FN, one
//    query per workgroup row of the grid (decode). Each wave keeps the
//    query's 64 x 128 index matrix in registers as four 16 x 128 MFMA A tiles;
//    the workgroup streams one range of keys through an LDS ring (LDS-DMA,
//    three 8 KiB tiles in flight). One 16x16x128 FP8 MFMA per (head tile,
//    16-key tile) gives 16 heads x 16 keys; the ReLU and the weighted head
//    sum run on the accumulators, and lane-swap additions leave the finished
//    score of each key in 16 lanes, stored coalesced.
//  * k_index_fp8_pf (index_prefill.hip): the same arithmetic for runs of
//    query rows of one sequence (prefill): the waves of a workgroup share
//    each LDS key tile.
// k_index_f32 and k_index_fp8 can also build the level-0 histogram (top 12
// bits of the score key) the top-k select starts from, so the layer never
// re-reads the scores for it.

#include "index_common.h"
#include "select_common.h"

namespace sga {

namespace {

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
  __shared__ uint32_t scratch[kF32Block / 64 + 1];
  const bool want_hist = sel.lists != nullptr;
  const int t = blockIdx.y;
  int64_t start;
  const int n = query_candidates(m, t, &start);
  if (want_hist && blockIdx.x == 0 && threadIdx.x == 0) sel.ncand[t] = make_int2(n, (int32_t)start);
  const int base = blockIdx.x * kF32Block;
  if (base >= n) return;
  for (int i = threadIdx.x; i < HI * DI; i += kF32Block) qs[i] = q_idx[(size_t)t * HI * DI + i];
  for (int i = threadIdx.x; i < HI; i += kF32Block) ws[i] = w[(size_t)t * HI + i];
  if (want_hist)
    for (int i = threadIdx.x; i < kHist0Bins; i += kF32Block) hist[i] = 0u;
  __syncthreads();
  const int s = base + threadIdx.x;
  if (s < n) {
    const float *kr = k_idx + kv_row(m, m.q_seq[t], start, s) * (int64_t)DI;
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
  if (want_hist) {
    __syncthreads();
    write_hist0_list<false, kF32Block>(hist, sel, t, blockIdx.x, scratch);
  }
}

// --------------------------------------------------------------------------
// FP8 MFMA path (HI = 64, DI = 128), one query per grid row (decode)
//
// The waves of a workgroup stream one contiguous key range of the query
// through a ring of kIdxRing steps in LDS; a step is kIdxStepTiles tiles of 64
// keys (8 KiB each). Every thread copies kIdxPieces 16-byte pieces of each step
// with LDS-DMA (global_load_lds_dwordx4), so kIdxRing - 1 steps are in flight
// while the workgroup computes. Within a 128-byte key row the 16-byte pieces
// are XOR-swizzled by key (applied on the DMA source side) so that the
// B-operand reads spread over the LDS banks. A step has 4 kIdxStepTiles groups
// of 16 keys; wave w scores groups w, w + kIdxWaves, .. with four 16x16x128
// MFMAs each (one per 16-head tile).
// One barrier per step both publishes the step and frees the buffer that the
// next copy overwrites.
// --------------------------------------------------------------------------
constexpr int kIdxWaves = 4;       // waves per workgroup (4 or 8)
constexpr int kKeyLoadPolicy = 2;  // nontemporal (streamed) key copies
constexpr int kIdxRing = 4;        // steps in the LDS ring
constexpr int kIdxStepTiles = 1;   // 64-key tiles per step
// The workgroup's scores collect in LDS and leave in one coalesced burst at
// its end instead of one 64-byte store per wave and tile.
constexpr bool kIdxStageScores = true;
constexpr int kIdxStepKeys = kIdxStepTiles * kIdxTileKeys;
constexpr int kIdxStepBytes = kIdxStepTiles * kIdxTileBytes;
constexpr int kIdxGroups = kIdxStepTiles * 4 / kIdxWaves;        // 16-key groups per wave and step
constexpr int kIdxPieces = kIdxStepBytes / (kIdxWaves * 64 * 16);  // DMA pieces per thread and step
static_assert(kIdxGroups >= 1 && kIdxGroups * kIdxWaves == kIdxStepTiles * 4, "groups per wave");
static_assert(kIdxPieces >= 1 && kIdxPieces * kIdxWaves * 64 * 16 == kIdxStepBytes, "pieces per thread");

// LDS atomic add without a return value, issued as inline asm so that the
// compiler does not make it wait for the in-flight LDS-DMA copies (it cannot
// tell that the histogram and the DMA buffers do not overlap). It has no
// result register; later lgkmcnt waits cover its completion.
__device__ __forceinline__ void lds_add_u32(uint32_t *p, uint32_t v) {
  const uint32_t addr =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t *)p;
  asm volatile("ds_add_u32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  // s_waitcnt needs an immediate: dispatch n = 0 .. N to a constant wait
  if constexpr (N > 0) {
    if (n >= N) {
      wait_vmcnt<N>();
      return;
    }
    wait_vmcnt_upto<N - 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}

template <bool kHist, int kR, bool kPaged>
__global__ __launch_bounds__(kIdxWaves * 64) void k_index_fp8(SeqMeta m, int T, int steps_per_wg,
                                                              const uint8_t *__restrict__ q_idx,
                                                              const float *__restrict__ w,
                                                              const uint8_t *__restrict__ k_idx,
                                                              float *__restrict__ scores,
                                                              int64_t stride, TopkWs sel) {
  constexpr int kThreads = kIdxWaves * 64;
  // dynamic LDS: the compiler then leaves the DMA/LDS-read ordering to the
  // explicit waits below instead of draining every DMA before each read
  extern __shared__ __attribute__((aligned(16))) unsigned char ring[];
  // the score stage follows the ring in the same allocation
  float *stage = (float *)(ring + kR * kIdxStepBytes);
  // level-0 histogram, one word per bin (two bins per word measured slower:
  // more same-address atomics)
  __shared__ uint32_t hist[kHist ? kHist0Bins : 1];
  __shared__ uint32_t scratch[kIdxWaves + 1];
  const int t = blockIdx.y;
  int64_t start;
  const int n = query_candidates(m, t, &start);
  if (kHist && blockIdx.x == 0 && threadIdx.x == 0) sel.ncand[t] = make_int2(n, (int32_t)start);
  const int c0 = blockIdx.x * steps_per_wg * kIdxStepKeys;
  if (c0 >= n) return;
  // paged caches: the page ids under this workgroup's keys, one per lane
  // (requested first, so that waiting for them waits for nothing else)
  PageWindow<1> win;
  if (kPaged) win.load(m, m.q_seq[t], c0, n);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform loop bounds
  const int kg = lane >> 4, c16 = lane & 15;
  const int nsteps = min(steps_per_wg, (n - c0 + kIdxStepKeys - 1) / kIdxStepKeys);
  // piece p = u * kThreads + tid of a step holds key row p / 8 of the step and
  // its swizzled 16-byte piece; rows past the sequence repeat its last key
  // (their scores are dropped)
  auto issue = [&](int i) {
    const int base = c0 + i * kIdxStepKeys;
    // paged: the step's 64 keys lie in one page (wave-uniform row); a key
    // past the sequence takes the row of its last key, as below
    const int64_t rb = kPaged ? win.row(m, base) : 0;
    const int64_t rlast = kPaged ? win.row(m, n - 1) : 0;
#pragma unroll
    for (int u = 0; u < kIdxPieces; ++u) {
      const int p = u * kThreads + tid;
      const int r = p >> 3;
      const int key = min(base + r, n - 1);
      const int64_t row = kPaged ? (base + r <= n - 1 ? rb + r : rlast) : start + key;
      const uint8_t *src = k_idx + row * 128 + (((p & 7) ^ key_swz(r)) << 4);
      __builtin_amdgcn_global_load_lds(
          src, (lds_void *)(ring + (i % kR) * kIdxStepBytes + (u * kThreads + wave * 64) * 16), 16, 0,
          kKeyLoadPolicy);
    }
  };
  // The query's 64 x 128 index matrix has the shape of a key step (64 rows of
  // 128 bytes). Every wave needs all of it (four 16 x 128 A tiles), so it is
  // copied once per workgroup into the ring's last buffer, which no key step
  // fills before the loop's first iteration, in the key steps' swizzled
  // layout, and each wave reads its A tiles from there: a quarter of the L2
  // traffic of four copies while the first steps are being fetched.
  static_assert(kIdxStepBytes == 64 * 128, "the index matrix fills one ring buffer");
  unsigned char *qbuf = ring + (kR - 1) * kIdxStepBytes;
#pragma unroll
  for (int u = 0; u < kIdxPieces; ++u) {
    const int p = u * kThreads + tid;
    const int r = p >> 3;
    const uint8_t *src = q_idx + ((size_t)t * 64 + r) * 128 + (((p & 7) ^ key_swz(r)) << 4);
    __builtin_amdgcn_global_load_lds(src, (lds_void *)(qbuf + (u * kThreads + wave * 64) * 16), 16, 0, 0);
  }
  // accumulator row r of this lane is head ht*16 + 4 kg + r
  float wv[16];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[ht * 4 + r] = w[(size_t)t * 64 + ht * 16 + 4 * kg + r];
  // The first steps are requested after the query's index matrix and weights,
  // so that only those loads are waited for before the loop (step 0 then
  // lands while the waves finish setting up). The requests are unconditional;
  // steps past nsteps read the clamped last key into ring buffers that are
  // never read, and the loop's last wait covers them.
  for (int i = 0; i < kR - 1; ++i) issue(i);
  // (cleared before the first barrier of the loop; no wave adds to it earlier)
  if (kHist)
    for (int i = tid; i < kHist0Bins; i += kThreads) hist[i] = 0u;
  wait_vmcnt<kIdxPieces * (kR - 1)>();  // the query loads have landed; from here vmcnt counts copies and stores
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();  // every wave's part of the index matrix is in LDS
  asm volatile("" ::: "memory");
  // A tiles: head ht*16 + c16, bytes [32 kg, 32 kg + 32) of its 128-byte row
  v8i a[4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) a[ht] = load_key_operand(qbuf, ht, kg, c16);
  // the reads are done before the loop's first barrier, after which step
  // kR - 1 overwrites this buffer
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
  float *srow = scores + t * stride;
  for (int i = 0; i < nsteps; ++i) {
    // step i has landed once at most the copies of the steps issued after it
    // are outstanding (score stores issued in between only lengthen the wait)
    wait_vmcnt_upto<kIdxPieces * (kR - 2)>(kIdxPieces * (min(nsteps - 1, i + kR - 2) - i));
    // (no lgkmcnt wait: this wave's B-operand reads of the buffer the next
    // copy overwrites completed before its MFMAs; only histogram atomics,
    // which touch no ring buffer, can still be in flight)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (i + kR - 1 < nsteps) issue(i + kR - 1);
    // group g of this wave: 16-key group wave + g * kIdxWaves of the step
    v8i b[kIdxGroups];
#pragma unroll
    for (int g = 0; g < kIdxGroups; ++g) {
      const int q = wave + g * kIdxWaves;
      b[g] = load_key_operand(ring + (i % kR) * kIdxStepBytes + (q >> 2) * kIdxTileBytes, q & 3, kg, c16);
    }
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    // each head sum split over two accumulators so consecutive FMAs do not wait
    float ev[kIdxGroups], od[kIdxGroups];
#pragma unroll
    for (int g = 0; g < kIdxGroups; ++g) ev[g] = od[g] = 0.0f;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
#pragma unroll
      for (int g = 0; g < kIdxGroups; ++g) {
        const v4f x = mfma_fp8(a[ht], b[g], zero);
        ev[g] = fmaf(fmaxf(x[0], 0.0f), wv[ht * 4 + 0], ev[g]);
        od[g] = fmaf(fmaxf(x[1], 0.0f), wv[ht * 4 + 1], od[g]);
        ev[g] = fmaf(fmaxf(x[2], 0.0f), wv[ht * 4 + 2], ev[g]);
        od[g] = fmaf(fmaxf(x[3], 0.0f), wv[ht * 4 + 3], od[g]);
      }
    }
#pragma unroll
    for (int g = 0; g < kIdxGroups; ++g) {
      // sum over the four lane groups that hold the same key: every lane ends
      // with the score of its key (-0 becomes +0)
      const float x = ev[g] + od[g];
      const float y = add_swapped(x, x, true);
      const float keep = add_swapped(y, y, false) + 0.0f;
      const int s = c0 + i * kIdxStepKeys + (wave + g * kIdxWaves) * 16 + lane;
      if (lane < 16 && s < n) {
        if (kIdxStageScores)
          stage[s - c0] = keep;
        else
          srow[s] = keep;
        if (kHist) {
          const uint32_t bin = score_key(keep) >> kHist0Shift;
          lds_add_u32(&hist[bin], 1u);
        }
      }
    }
  }
  if (kHist || kIdxStageScores) __syncthreads();
  if (kIdxStageScores) {
    const int nk = min(n - c0, steps_per_wg * kIdxStepKeys);
    const bool vec = ((stride | c0) & 3) == 0 && ((uintptr_t)srow & 15) == 0;  // 16-byte aligned stores
    if (vec) {
      for (int j = 4 * tid; j < nk; j += 4 * kThreads) {
        if (j + 4 <= nk)
          *(float4 *)(srow + c0 + j) = *(const float4 *)(stage + j);
        else
          for (int e = j; e < nk; ++e) srow[c0 + e] = stage[e];
      }
    } else {
      for (int j = tid; j < nk; j += kThreads) srow[c0 + j] = stage[j];
    }
  }
  if (kHist) write_hist0_list<false, kThreads>(hist, sel, t, blockIdx.x, scratch);
}

// --------------------------------------------------------------------------
// Streaming-read reference: the index kernel's copy pattern with no scoring.
// Each workgroup streams a contiguous share of 8 KiB tiles through the same
// LDS ring (LDS-DMA, nontemporal, kIdxRing steps, one barrier per step), and
// every thread reads back its 32 bytes of each tile and folds them into one
// word, written to sink[blockIdx.x] so that no copy can be dropped.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kIdxWaves * 64) void k_stream_read(const uint8_t *__restrict__ src, int64_t tiles,
                                                                 uint32_t *__restrict__ sink) {
  constexpr int kThreads = kIdxWaves * 64;
  constexpr int kPer = kIdxTileBytes / (kThreads * 16);  // copies per thread and tile
  __shared__ __attribute__((aligned(16))) unsigned char ring[kIdxRing * kIdxTileBytes];
  __shared__ uint32_t red[kIdxWaves];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t per = (tiles + gridDim.x - 1) / gridDim.x;
  const int64_t t0 = min(tiles, (int64_t)blockIdx.x * per), t1 = min(tiles, t0 + per);
  const int n = (int)(t1 - t0);
  auto issue = [&](int i) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int pc = u * kThreads + tid;
      __builtin_amdgcn_global_load_lds(src + (t0 + i) * kIdxTileBytes + pc * 16,
                                       (lds_void *)(ring + (i % kIdxRing) * kIdxTileBytes + (u * kThreads + wave * 64) * 16),
                                       16, 0, kKeyLoadPolicy);
    }
  };
  for (int i = 0; i < kIdxRing - 1 && i < n; ++i) issue(i);
  uint32_t acc = 0;
  for (int i = 0; i < n; ++i) {
    const int after = min(n - 1, i + kIdxRing - 2) - i;  // tiles issued after tile i
    wait_vmcnt_upto<kPer * (kIdxRing - 2)>(kPer * after);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (i + kIdxRing - 1 < n) issue(i + kIdxRing - 1);
    const v4i *tb = (const v4i *)(ring + (i % kIdxRing) * kIdxTileBytes);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const v4i x = tb[u * kThreads + tid];
      acc ^= (uint32_t)(x.x ^ x.y ^ x.z ^ x.w);
    }
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0): reads done before the buffer is reused
  }
  for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d, 64);
  if ((tid & 63) == 0) red[wave] = acc;
  __syncthreads();
  if (tid == 0) {
    uint32_t r = 0;
    for (int i = 0; i < kIdxWaves; ++i) r ^= red[i];
    sink[blockIdx.x] = r;
  }
}

}  // namespace

hipError_t launch_stream_read(const uint8_t *src, int64_t bytes, uint32_t *sink, hipStream_t s) {
  const int64_t tiles = bytes / kIdxTileBytes;
  if (tiles <= 0) return hipSuccess;
  const int64_t most = (int64_t)kStreamReadBlocksPerCu * device_cu_count();
  const int grid = (int)(tiles < most ? tiles : most);
  hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(kIdxWaves * 64), 0, s, src, tiles, sink);
  return hipGetLastError();
}

int index_fp8_iters(int T, int max_kv_len) {
  // a workgroup scores 4 * iters tiles of 64 keys; aim for about two
  // workgroups per CU over the whole batch (4096 keys each for 16 x 128K).
  // At most 4096 keys per workgroup: the grid is sized by max_kv_len, and
  // with sequences of mixed length most of a long grid row has work only for
  // the longest sequences, so larger workgroups would leave CUs idle.
  const int64_t keys = (int64_t)T * max_kv_len;
  const int64_t per_iter = 2048LL * kIdxTileKeys;
  int64_t it = (keys + per_iter - 1) / per_iter;
  if (it < 2) it = 2;
  if (it > 16) it = 16;
  return (int)it;
}

hipError_t launch_index_f32(const SeqMeta &m, int T, int k, int HI, int DI, const float *q_idx,
                            const float *w, const float *k_idx, float *scores, int64_t stride,
                            TopkWs *sel, hipStream_t s) {
  if (T == 0 || m.max_kv_len == 0) return hipSuccess;
  TopkWs none{};
  if (sel && (m.max_kv_len + kF32Block - 1) / kF32Block > kTopkMaxSlots) {
    // too many 256-position slots for the list merge: histogram in a separate pass
    hipLaunchKernelGGL(k_index_f32, dim3((m.max_kv_len + kF32Block - 1) / kF32Block, T), dim3(kF32Block), 0,
                       s, m, k, HI, DI, q_idx, w, k_idx, scores, stride, none);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_topk_hist0(m, T, scores, stride, sel, s);
  }
  if (sel) {
    sel->slot_keys = kF32Block;
    sel->slot_words = 4 + kF32Block;
  }
  dim3 grid((m.max_kv_len + kF32Block - 1) / kF32Block, T);
  hipLaunchKernelGGL(k_index_f32, grid, dim3(kF32Block), 0, s, m, k, HI, DI, q_idx, w, k_idx,
                     scores, stride, sel ? *sel : none);
  return hipGetLastError();
}

hipError_t launch_index_fp8(const SeqMeta &m, int T, int k, const uint8_t *q_idx, const float *w,
                            const uint8_t *k_idx, float *scores, int64_t stride, TopkWs *sel,
                            hipStream_t s) {
  if (T == 0 || m.max_kv_len == 0) return hipSuccess;
  // one-time set-up (a function-local static is initialised exactly once,
  // also when several host threads arrive together)
  static const bool attr = [] {
    // ring plus the largest score stage (64 tiles)
    const int max_smem = kIdxRing * kIdxStepBytes + (kIdxStageScores ? 64 * kIdxTileKeys * 4 : 0);
    (void)hipFuncSetAttribute((const void *)k_index_fp8<true, kIdxRing, false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, max_smem);
    (void)hipFuncSetAttribute((const void *)k_index_fp8<false, kIdxRing, false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, max_smem);
    (void)hipFuncSetAttribute((const void *)k_index_fp8<true, kIdxRing, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, max_smem);
    (void)hipFuncSetAttribute((const void *)k_index_fp8<false, kIdxRing, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, max_smem);
    (void)hipGetLastError();
    return true;
  }();
  (void)attr;
  // many query rows per sequence: the query-tiled kernel (it also scores the
  // row groups that span a sequence boundary); the level-0 histogram then
  // comes from a separate pass over the scores
  if (T >= 4 * kPfGroup && T >= 4 * m.num_seqs) {
    hipError_t e = launch_index_fp8_prefill(m, T, q_idx, w, k_idx, scores, stride, s);
    if (e != hipSuccess || !sel) return e;
    return launch_topk_hist0(m, T, scores, stride, sel, s);
  }
  // aim for about two workgroups per CU; a workgroup scores whole steps
  const int steps = index_fp8_iters(T, m.max_kv_len) * 4 / kIdxStepTiles;
  const int per_wg = steps * kIdxStepKeys;
  dim3 grid((m.max_kv_len + per_wg - 1) / per_wg, T);
  TopkWs none{};
  if (sel) {
    sel->slot_keys = per_wg;
    sel->slot_words = 4 + (per_wg < kHist0Bins ? per_wg : kHist0Bins);
  }
  const size_t smem = (size_t)kIdxRing * kIdxStepBytes + (kIdxStageScores ? (size_t)per_wg * 4 : 0);
  const dim3 block(kIdxWaves * 64);
  if (m.page_shift) {
    if (sel)
      hipLaunchKernelGGL((k_index_fp8<true, kIdxRing, true>), grid, block, smem, s, m, T, steps, q_idx, w,
                         k_idx, scores, stride, *sel);
    else
      hipLaunchKernelGGL((k_index_fp8<false, kIdxRing, true>), grid, block, smem, s, m, T, steps, q_idx, w,
                         k_idx, scores, stride, none);
  } else if (sel) {
    hipLaunchKernelGGL((k_index_fp8<true, kIdxRing, false>), grid, block, smem, s, m, T, steps, q_idx, w,
                       k_idx, scores, stride, *sel);
  } else {
    hipLaunchKernelGGL((k_index_fp8<false, kIdxRing, false>), grid, block, smem, s, m, T, steps, q_idx, w,
                       k_idx, scores, stride, none);
  }
  return hipGetLastError();
}

}  // namespace sga
