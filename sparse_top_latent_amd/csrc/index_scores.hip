// Indexer score pass: I[t,s] = sum_h w[t,h] * max(0, qI[t,h,:] . kI[s,:]) for s < n_t.
//
// Source: "A.X-K2: a sparse-attention upgrade that costs nothing, trained
// natively in FP8", section "Sparse Gated Attention" (a lightweight indexer
// scores every cached key for each query); "A.X-K2" model card, section
// "Sparse Gated Attention (SGA)" (the indexer scores and ranks key-value
// candidates). The weighted-ReLU form is the reading this library implements.
//
// Three kernels (device helpers shared with the prefill kernel live in
// index_common.h):
//  * k_index_f32: generic fp32 path, one thread per (query, key).
//  * k_index_fp8: MI355X path for 64 index heads x 128 dims in E4M3FN, one
//    query per workgroup row of the grid (decode). Each wave keeps the
//    query's 64 x 128 index matrix in registers as four 16 x 128 MFMA A tiles
//    and streams its own range of keys through LDS (LDS-DMA, two 8 KiB tiles
//    in flight). One 16x16x128 FP8 MFMA per (head tile, 16-key tile) gives 16
//    heads x 16 keys; the ReLU and the weighted head sum run on the
//    accumulators, and lane-swap additions leave one finished score per lane,
//    stored coalesced.
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
  const int base = blockIdx.x * kF32Block;
  if (base >= n) return;
  for (int i = threadIdx.x; i < HI * DI; i += kF32Block) qs[i] = q_idx[(size_t)t * HI * DI + i];
  for (int i = threadIdx.x; i < HI; i += kF32Block) ws[i] = w[(size_t)t * HI + i];
  if (want_hist)
    for (int i = threadIdx.x; i < kHist0Bins; i += kF32Block) hist[i] = 0u;
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
  if (want_hist) {
    __syncthreads();
    write_hist0_list<false>(hist, sel, t, blockIdx.x, scratch);
  }
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
constexpr int kKeyLoadPolicy = 2;            // nontemporal (streamed) key copies
constexpr int kIdxDmaPerTile = kIdxTileBytes / (64 * 16);  // 8 DMA issues per lane
constexpr int kIdxBufs = 2;                  // tiles in flight per wave
constexpr size_t kIdxSmem = (size_t)kIdxWaves * kIdxBufs * kIdxTileBytes;

// LDS atomic add without a return value, issued as inline asm so that the
// compiler does not make it wait for the wave's in-flight LDS-DMA copies
// (it cannot tell that the histogram and the DMA buffers do not overlap).
// It has no result register; later lgkmcnt waits cover its completion.
__device__ __forceinline__ void lds_add_u32(uint32_t *p, uint32_t v) {
  const uint32_t addr =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t *)p;
  asm volatile("ds_add_u32 %0, %1" ::"v"(addr), "v"(v) : "memory");
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
                                       16, 0, kKeyLoadPolicy);
  } else {
    // sequence tail: rows past the end repeat the last key (their scores are dropped)
#pragma unroll
    for (int i = 0; i < kIdxDmaPerTile; ++i) {
      const int r = i * 8 + (lane >> 3);
      int key = base + r;
      key = key < n ? key : n - 1;
      const uint8_t *src = k_idx + (start + key) * 128 + (lane_off[i & 1] & 127);
      __builtin_amdgcn_global_load_lds(src, (lds_void *)(buf + i * 1024), 16, 0, kKeyLoadPolicy);
    }
  }
}

template <bool kHist>
__global__ __launch_bounds__(kIdxWaves * 64) void k_index_fp8(SeqMeta m, int T, int k, int iters,
                                                              const uint8_t *__restrict__ q_idx,
                                                              const float *__restrict__ w,
                                                              const uint8_t *__restrict__ k_idx,
                                                              float *__restrict__ scores,
                                                              int64_t stride, TopkWs sel) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // level-0 histogram with two 16-bit bins per word (a workgroup scores at most
  // 4 x 32 x 64 = 8192 keys, so a bin cannot overflow)
  __shared__ uint32_t hist[kHist ? kHist0Bins / 2 : 1];
  __shared__ uint32_t scratch[kIdxWaves + 1];
  const int t = blockIdx.y;
  int64_t start;
  const int n = query_candidates(m, t, &start);
  const int wave_keys = iters * kIdxTileKeys;
  const int chunk0 = blockIdx.x * kIdxWaves * wave_keys;
  if (chunk0 >= n) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform loop bounds
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
    score_tiles<1>(a, [&](int kt) { return load_key_operand(tb, kt, kg, c16); }, wv, part);
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
    write_hist0_list<true>(hist, sel, t, blockIdx.x, scratch);
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
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void *)k_index_fp8<true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kIdxSmem);
    (void)hipFuncSetAttribute((const void *)k_index_fp8<false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kIdxSmem);
    (void)hipGetLastError();
    attr = true;
  }
  // many query rows per sequence: the query-tiled kernel (it also scores the
  // row groups that span a sequence boundary); the level-0 histogram then
  // comes from a separate pass over the scores
  if (T >= 4 * kPfGroup && T >= 4 * m.num_seqs) {
    hipError_t e = launch_index_fp8_prefill(m, T, q_idx, w, k_idx, scores, stride, s);
    if (e != hipSuccess || !sel) return e;
    return launch_topk_hist0(m, T, scores, stride, sel, s);
  }
  const int iters = index_fp8_iters(T, m.max_kv_len);
  const int per_wg = kIdxWaves * iters * kIdxTileKeys;
  dim3 grid((m.max_kv_len + per_wg - 1) / per_wg, T);
  TopkWs none{};
  if (sel) {
    sel->slot_keys = per_wg;
    sel->slot_words = 4 + (per_wg < kHist0Bins ? per_wg : kHist0Bins);
  }
  if (sel)
    hipLaunchKernelGGL(k_index_fp8<true>, grid, dim3(kIdxWaves * 64), kIdxSmem, s, m, T, k, iters,
                       q_idx, w, k_idx, scores, stride, *sel);
  else
    hipLaunchKernelGGL(k_index_fp8<false>, grid, dim3(kIdxWaves * 64), kIdxSmem, s, m, T, k, iters,
                       q_idx, w, k_idx, scores, stride, none);
  return hipGetLastError();
}

}  // namespace sga
