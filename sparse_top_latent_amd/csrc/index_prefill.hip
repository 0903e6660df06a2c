// Indexer score pass for runs of query rows of one sequence (prefill):
// I[t,s] = sum_h w[t,h] * max(0, qI[t,h,:] . kI[s,:]) for s < n_t, with every
// LDS key tile shared by a group of query rows.
//
// Source: "A.X-K2: a sparse-attention upgrade that costs nothing, trained
// natively in FP8", section "Sparse Gated Attention" (the indexer scores every
// cached key for each query); "A.X-K2" model card, section "Sparse Gated
// Attention (SGA)". The weighted-ReLU form is the reading this library
// implements (see index_scores.hip).

#include "index_common.h"

namespace sga {

namespace {

// --------------------------------------------------------------------------
// Prefill: many queries of one sequence share every key tile.
//
// A workgroup owns a group of 8 query rows of one sequence (8 / kQpw waves of
// kQpw queries; each wave keeps its 64 x 128 index matrices in VGPRs) and a
// range of 8192 keys. Key tiles of 64 keys are copied once into LDS with
// LDS-DMA and reused by all 8 queries, so the pass is bound by the MFMAs and
// the ReLU/weight epilogue instead of by HBM. Three tile buffers let one
// barrier per tile both publish tile i and free the buffer that tile i + 2
// overwrites. Keys past a query's own position are neither scored nor stored.
// A group whose rows span a sequence boundary is scored by the same
// workgroup, one row per wave, without sharing.
// --------------------------------------------------------------------------
// A group is "shared" when all of its rows name the same sequence.
template <int kGroup>
__device__ __forceinline__ bool group_is_shared(const SeqMeta &m, int T, int g) {
  const int t0 = g * kGroup;
  const int t1 = min(T, t0 + kGroup);
  const int32_t b = m.q_seq[t0];
  bool same = true;
  for (int t = t0 + 1; t < t1; ++t) same = same && (m.q_seq[t] == b);
  return same;
}

// Two shapes of the kernel (query rows per workgroup, keys per workgroup,
// tile buffers): prefill, 8 rows x 8,192 keys with 3 buffers, bound by the
// MFMAs; multi-query decode (a few queries per sequence, e.g. the draft
// tokens of speculative decoding), 4 rows x 2,048 keys with 4 buffers: four
// workgroups per CU for 16 x 128K (4,096 keys per workgroup: 10 % slower).
constexpr int kPfQpw = 1;       // queries per wave

// kQpw queries per wave, kPfGroup / kQpw waves per workgroup. The
// weighted-ReLU epilogue brings about as much VALU work as there is MFMA work
// and the two overlap only in part on a SIMD, so latency is hidden by wave
// count: the register budget is held to 6 waves per SIMD (3 workgroups per CU).
template <int kQpw, int kGroup, int kChunk, int kBufs, bool kPaged>
__global__ __launch_bounds__(kGroup / kQpw * 64, 6) void k_index_fp8_pf(SeqMeta m, int T,
                                                                const uint8_t *__restrict__ q_idx,
                                                                const float *__restrict__ w,
                                                                const uint8_t *__restrict__ k_idx,
                                                                float *__restrict__ scores,
                                                                int64_t stride) {
  constexpr int kThreads = kGroup / kQpw * 64;
  static_assert(kBufs == 3 || kBufs == 4, "tile buffers");
  static_assert(512 % kThreads == 0 || kThreads % 512 == 0, "a tile is 512 16-byte pieces");
  constexpr int kDmaPer = kThreads >= 512 ? 1 : 512 / kThreads;  // DMA issues per thread per tile
  // dynamic LDS: the compiler then leaves the DMA/LDS-read ordering to the
  // explicit waits below instead of draining every DMA before each read
  extern __shared__ __attribute__((aligned(16))) unsigned char tiles[];
  __shared__ int s_nmax;
  const int g = blockIdx.y;
  const bool shared = group_is_shared<kGroup>(m, T, g);  // uniform over the workgroup
  const int t0 = g * kGroup;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int kg = lane >> 4, c16 = lane & 15;
  int64_t start = 0;
  if (tid == 0) {
    int mx = 0;
    for (int t = t0; t < min(T, t0 + kGroup); ++t) mx = max(mx, query_candidates(m, t, &start));
    s_nmax = mx;
  }
  __syncthreads();
  const int nmax = s_nmax;
  const int c0 = blockIdx.x * kChunk;
  if (c0 >= nmax) return;
  const int ntiles = (min(nmax, c0 + kChunk) - c0 + kIdxTileKeys - 1) / kIdxTileKeys;

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
  if (!shared) {
    // The group's rows name several sequences (a sequence boundary falls
    // inside it): each wave scores its own rows, with the B operands read
    // straight from global memory (16 keys x 128 bytes, one coalesced 2 KiB
    // block per operand); no LDS and no barrier.
#pragma unroll
    for (int j = 0; j < kQpw; ++j) {
      const int t = t0 + kQpw * wave + j;
      int64_t st = 0;
      const int n = t < T ? query_candidates(m, t, &st) : 0;
      const int cend = min(n, c0 + kChunk);
      for (int kbase = c0; kbase < cend; kbase += kIdxTileKeys) {
        float part[1][4];
        const v8i(&aj)[1][4] = *reinterpret_cast<const v8i(*)[1][4]>(&a[j]);
        const float(&wj)[1][16] = *reinterpret_cast<const float(*)[1][16]>(&wv[j]);
        score_tiles<1>(
            aj,
            [&](int kt) {
              int key = kbase + kt * 16 + c16;
              key = key < n ? key : n - 1;
              const int64_t row = kPaged ? kv_row(m, m.q_seq[t], st, key) : st + key;
              const v4i *src = (const v4i *)(k_idx + row * 128 + kg * 32);
              const v4i lo = src[0], hi = src[1];
              return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            },
            wj, part);
        const float keep = tile_scores(part[0]);
        const int sidx = kbase + lane;
        if (sidx < n) scores[(size_t)t * stride + sidx] = keep;
      }
    }
    return;
  }
  query_candidates(m, t0, &start);  // the group's sequence start
  // paged caches: the page ids under this workgroup's keys, one per lane
  PageWindow<(kChunk / kIdxTileKeys + 63) / 64> win;
  if (kPaged) win.load(m, m.q_seq[t0], c0, nmax);
  // DMA pieces of this thread: piece p = u * kThreads + tid of the 8 KiB tile
  // holds tile row p / 8 and its swizzled 16-byte piece
  auto issue = [&](int i) {
    const int base = c0 + i * kIdxTileKeys;
    // paged: the tile's 64 keys lie in one page (wave-uniform row); a key
    // past the group's last key takes that key's row
    const int64_t rb = kPaged ? win.row(m, base) : 0;
    const int64_t rlast = kPaged ? win.row(m, nmax - 1) : 0;
#pragma unroll
    for (int u = 0; u < kDmaPer; ++u) {
      const int p = u * kThreads + tid;
      if (kThreads > 512 && p >= 512) break;  // wave-uniform: whole waves past the tile
      const int r = p >> 3;
      int key = base + r;
      key = key < nmax ? key : nmax - 1;
      const int64_t row = kPaged ? (base + r < nmax ? rb + r : rlast) : start + key;
      const uint8_t *src = k_idx + row * 128 + (((p & 7) ^ key_swz(r)) << 4);
      __builtin_amdgcn_global_load_lds(
          src, (lds_void *)(tiles + (i % kBufs) * kIdxTileBytes + (u * kThreads + wave * 64) * 16),
          16, 0, 0);
    }
  };
  wait_vmcnt<0>();
  for (int i = 0; i < kBufs - 1; ++i)
    if (i < ntiles) issue(i);
  for (int i = 0; i < ntiles; ++i) {
    // Tile i has landed once at most the kDmaPer copies of each tile issued
    // after it are outstanding; score stores issued later only make this wait
    // longer. The barrier then publishes every wave's part of tile i and
    // certifies that all LDS reads of tile i - 1 are done, so the copy of
    // tile i + kBufs - 1 may overwrite that buffer.
    const int after = min(ntiles - 1, i + kBufs - 2) - i;  // tiles issued after tile i
    if (after >= 2)
      wait_vmcnt<2 * kDmaPer>();
    else if (after == 1)
      wait_vmcnt<kDmaPer>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (i + kBufs - 1 < ntiles) issue(i + kBufs - 1);
    const unsigned char *tb = tiles + (i % kBufs) * kIdxTileBytes;
    const int kbase = c0 + i * kIdxTileKeys;
    float part[kQpw][4];
    score_tiles<kQpw>(a, [&](int kt) { return load_key_operand(tb, kt, kg, c16); }, wv, part);
    const int s = kbase + lane;
#pragma unroll
    for (int j = 0; j < kQpw; ++j) {
      const float keep = tile_scores(part[j]);
      if (s < nq[j]) scores[(size_t)(t0 + kQpw * wave + j) * stride + s] = keep;
    }
  }
}

}  // namespace

template <bool kPaged>
hipError_t launch_pf(const SeqMeta &m, int T, const uint8_t *q_idx, const float *w, const uint8_t *k_idx,
                     float *scores, int64_t stride, hipStream_t s) {
  if (T < 8 * m.num_seqs) {
    // a few queries per sequence (multi-query decode): groups of 4 rows
    dim3 grid((m.max_kv_len + 2047) / 2048, (T + 3) / 4);
    hipLaunchKernelGGL((k_index_fp8_pf<kPfQpw, 4, 2048, 4, kPaged>), grid, dim3(4 / kPfQpw * 64),
                       4 * kIdxTileBytes, s, m, T, q_idx, w, k_idx, scores, stride);
  } else {
    dim3 grid((m.max_kv_len + 8191) / 8192, (T + kPfGroup - 1) / kPfGroup);
    hipLaunchKernelGGL((k_index_fp8_pf<kPfQpw, kPfGroup, 8192, 3, kPaged>), grid,
                       dim3(kPfGroup / kPfQpw * 64), 3 * kIdxTileBytes, s, m, T, q_idx, w, k_idx, scores,
                       stride);
  }
  return hipGetLastError();
}

hipError_t launch_index_fp8_prefill(const SeqMeta &m, int T, const uint8_t *q_idx, const float *w,
                                    const uint8_t *k_idx, float *scores, int64_t stride,
                                    hipStream_t s) {
  if (m.page_shift)
    return launch_pf<true>(m, T, q_idx, w, k_idx, scores, stride, s);
  return launch_pf<false>(m, T, q_idx, w, k_idx, scores, stride, s);
}


}  // namespace sga
