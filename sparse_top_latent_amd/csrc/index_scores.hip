// Indexer score pass: I[t,s] = sum_h w[t,h] * max(0, qI[t,h,:] . kI[s,:]) for s < n_t.
//
// Source: "A.X-K2: a sparse-attention upgrade that costs nothing, trained
// natively in FP8", section "Sparse Gated Attention" (a lightweight indexer
// scores every cached key for each query); "A.X-K2" model card, section
// "Sparse Gated Attention (SGA)" (the indexer scores and ranks key-value
// candidates). The weighted-ReLU form is the reading this library implements.
//
// Two kernels:
//  * k_index_f32: generic fp32 path, one thread per (query, key).
//  * k_index_fp8: MI355X path for 64 index heads x 128 dims in E4M3FN. Each
//    wave keeps the query's 64 x 128 index matrix in registers as four 16 x 128
//    MFMA A tiles and streams 16-key B tiles straight from HBM into registers
//    (every key is used once, so no LDS staging). One 16x16x128 FP8 MFMA per
//    (head tile, key tile) gives 16 heads x 16 keys; the ReLU and the weighted
//    head sum run on the accumulators, and a 2-step cross-lane reduction leaves
//    one finished score per lane, stored coalesced.
// Both can also build the level-0 histogram (top 12 bits of the score key) the
// top-k select starts from, so the layer never re-reads the scores for it.

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

// --------------------------------------------------------------------------
// fp32 path
// --------------------------------------------------------------------------
constexpr int kF32Block = 256;
constexpr int kF32MaxQ = 8192;  // HI * DI

__global__ __launch_bounds__(kF32Block) void k_index_f32(SeqMeta m, int HI, int DI,
                                                         const float *__restrict__ q_idx,
                                                         const float *__restrict__ w,
                                                         const float *__restrict__ k_idx,
                                                         float *__restrict__ scores,
                                                         int64_t stride, uint32_t *hist0) {
  __shared__ float qs[kF32MaxQ];
  __shared__ float ws[64];
  __shared__ uint32_t hist[kHist0Bins];
  const int t = blockIdx.y;
  int64_t start;
  const int n = query_candidates(m, t, &start);
  const int base = blockIdx.x * kF32Block;
  if (base >= n) return;
  for (int i = threadIdx.x; i < HI * DI; i += kF32Block) qs[i] = q_idx[(size_t)t * HI * DI + i];
  for (int i = threadIdx.x; i < HI; i += kF32Block) ws[i] = w[(size_t)t * HI + i];
  if (hist0) hist_zero(hist);
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
    if (hist0) atomicAdd(&hist[score_key(acc) >> kHist0Shift], 1u);
  }
  if (hist0) hist_flush(hist, hist0 + (size_t)t * kHist0Bins);
}

// --------------------------------------------------------------------------
// FP8 MFMA path (HI = 64, DI = 128)
// --------------------------------------------------------------------------
constexpr int kFp8Waves = 4;
constexpr int kFp8Iters = 8;                                   // 64-key steps per wave
constexpr int kFp8Chunk = kFp8Waves * kFp8Iters * 64;          // keys per workgroup

__device__ __forceinline__ v4f mfma_fp8(const v8i &a, const v8i &b, const v4f &c) {
  // E4M3 x E4M3 (format code 0), unit E8M0 scales (127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ void load_key_tiles(v8i (&b)[4], const uint8_t *__restrict__ k_idx,
                                               int64_t start, int n, int base, int lane) {
  const int kg = lane >> 4;  // which 32-byte quarter of the 128-byte key
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    int key = base + kt * 16 + (lane & 15);
    key = key < n ? key : n - 1;
    const v4i *src = (const v4i *)(k_idx + (start + key) * 128 + kg * 32);
    v4i lo = __builtin_nontemporal_load(src);
    v4i hi = __builtin_nontemporal_load(src + 1);
    b[kt] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  }
}

template <bool kHist>
__global__ __launch_bounds__(256) void k_index_fp8(SeqMeta m, const uint8_t *__restrict__ q_idx,
                                                   const float *__restrict__ w,
                                                   const uint8_t *__restrict__ k_idx,
                                                   float *__restrict__ scores, int64_t stride,
                                                   uint32_t *hist0) {
  __shared__ uint32_t hist[kHist ? kHist0Bins : 1];
  const int t = blockIdx.y;
  int64_t start;
  const int n = query_candidates(m, t, &start);
  const int chunk0 = blockIdx.x * kFp8Chunk;
  if (chunk0 >= n) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kg = lane >> 4;

  // A tiles: head (ht*16 + lane%16), bytes [32*kg, 32*kg+32) of its 128-byte row
  v8i a[4];
  float wv[16];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const v4i *src = (const v4i *)(q_idx + ((size_t)t * 64 + ht * 16 + (lane & 15)) * 128 + kg * 32);
    v4i lo = src[0], hi = src[1];
    a[ht] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    // accumulator row r of this lane is head ht*16 + 4*kg + r
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[ht * 4 + r] = w[(size_t)t * 64 + ht * 16 + 4 * kg + r];
  }
  if (kHist) hist_zero(hist);

  v8i bcur[4], bnext[4];
  int base = chunk0 + wave * 64;
  if (base < n) load_key_tiles(bcur, k_idx, start, n, base, lane);
  for (int it = 0; it < kFp8Iters; ++it) {
    if (base >= n) break;
    const int nbase = base + kFp8Waves * 64;
    const bool more = (it + 1 < kFp8Iters) && (nbase < n);
    if (more) load_key_tiles(bnext, k_idx, start, n, nbase, lane);

    float part[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      float acc = 0.0f;
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        v4f d = mfma_fp8(a[ht], bcur[kt], (v4f){0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = fmaf(fmaxf(d[r], 0.0f), wv[ht * 4 + r], acc);
      }
      part[kt] = acc;
    }
    // lanes l, l^16, l^32, l^48 hold partial sums of the same 4 keys (one per kt);
    // reduce-scatter so that lane l finishes key base + l.
    const bool b5 = (lane & 32) != 0;
    const bool b4 = (lane & 16) != 0;
    float k0 = b5 ? part[2] : part[0];
    float k1 = b5 ? part[3] : part[1];
    float s0 = b5 ? part[0] : part[2];
    float s1 = b5 ? part[1] : part[3];
    k0 += __shfl_xor(s0, 32, 64);
    k1 += __shfl_xor(s1, 32, 64);
    float keep = b4 ? k1 : k0;
    float send = b4 ? k0 : k1;
    keep += __shfl_xor(send, 16, 64);
    keep += 0.0f;  // -0 -> +0
    const int s = base + lane;
    if (s < n) {
      scores[t * stride + s] = keep;
      if (kHist) atomicAdd(&hist[score_key(keep) >> kHist0Shift], 1u);
    }
    if (more) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) bcur[kt] = bnext[kt];
    }
    base = nbase;
  }
  if (kHist) hist_flush(hist, hist0 + (size_t)t * kHist0Bins);
}

}  // namespace

hipError_t launch_index_f32(const SeqMeta &m, int T, int HI, int DI, const float *q_idx,
                            const float *w, const float *k_idx, float *scores, int64_t stride,
                            uint32_t *hist0, hipStream_t s) {
  if (T == 0 || m.max_kv_len == 0) return hipSuccess;
  dim3 grid((m.max_kv_len + kF32Block - 1) / kF32Block, T);
  hipLaunchKernelGGL(k_index_f32, grid, dim3(kF32Block), 0, s, m, HI, DI, q_idx, w, k_idx,
                     scores, stride, hist0);
  return hipGetLastError();
}

hipError_t launch_index_fp8(const SeqMeta &m, int T, const uint8_t *q_idx, const float *w,
                            const uint8_t *k_idx, float *scores, int64_t stride, uint32_t *hist0,
                            hipStream_t s) {
  if (T == 0 || m.max_kv_len == 0) return hipSuccess;
  dim3 grid((m.max_kv_len + kFp8Chunk - 1) / kFp8Chunk, T);
  if (hist0)
    hipLaunchKernelGGL(k_index_fp8<true>, grid, dim3(256), 0, s, m, q_idx, w, k_idx, scores,
                       stride, hist0);
  else
    hipLaunchKernelGGL(k_index_fp8<false>, grid, dim3(256), 0, s, m, q_idx, w, k_idx, scores,
                       stride, hist0);
  return hipGetLastError();
}

}  // namespace sga
