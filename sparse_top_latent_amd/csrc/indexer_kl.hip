// Indexer KL loss over the sparse top-k selection and its gradients (the
// training side of the indexer, "A.X K2 Technical Report" section 3.4: a KL
// loss aligns the indexer's scores with the attention distribution, computed
// over the sparse selection from the start).
//
// For query t with selected positions S_t (the forward's top-k list) and the
// forward's per-head log-sum-exp lse[t, h]:
//   target_s = sum_h exp(tau q_h . kv_s - lse_h), normalised over S_t
//   I_s      = sum_h w_h ReLU(qI_h . kI_s),  q = softmax over S_t of I
//   loss_t   = sum_s target_s (log target_s - log q_s)
//   g_s      = q_s - target_s                 (the target is a constant)
//   d_w[h]   = sum_s g_s ReLU(z_hs)
//   d_qI[h]  = sum_s g_s w_h [z_hs > 0] kI_s
//   d_kI[s] += sum_h g_s w_h [z_hs > 0] qI_h  (added into the caller's buffer)
//
// Kernels per call:
//   k_kl_mass_mfma  one workgroup per (64 selected rows, query), MI355X shapes:
//                   the head-summed attention mass of each row, logits by bf16
//                   MFMA with the query slice in VGPRs, and (FP8 index
//                   tensors) each row's indexer score;
//   k_kl_rows       one workgroup per (64 rows, query): each row's indexer score
//                   (and, for the other shapes, its attention mass, fp32 dot
//                   products from q in LDS);
//   k_kl_loss       one workgroup per query: the two normalisations, the loss
//                   and g;
//   k_kl_backward   one workgroup per (64 rows, query): z again and the
//                   gradient products (bf16 and fp32 MFMA for 64 x 128 FP8
//                   index tensors), d_kI by fp32 atomics, per-chunk partials
//                   of d_w and d_qI;
//   k_kl_reduce     sums the partials over the chunks (fixed order).
// The softmax, loss and reductions are fp32 on the vector ALUs.

#include "kernels.h"

namespace sga {
namespace {

constexpr int kKlRows = 64;     // selected rows per workgroup
constexpr int kKlThreads = 256; // 4 threads per row

// 8 consecutive values of element type dt starting at element i of p (i a
// multiple of 8); MXFP8 values take the E8M0 scale of their 32-value block.
__device__ __forceinline__ void load8(const void *p, int dt, const uint8_t *scale, int64_t row_elems,
                                      int64_t row, int d, float v[8]) {
  const int64_t i = row * row_elems + d;
  if (dt == SGA_BF16) {
    const uint4 r = *(const uint4 *)((const uint16_t *)p + i);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  } else if (dt == SGA_F32) {
    const float4 a = *(const float4 *)((const float *)p + i), b = *(const float4 *)((const float *)p + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint2 r = *(const uint2 *)((const uint8_t *)p + i);
    const float sc = dt == SGA_MXFP8_E4M3FN ? e8m0_to_f32(scale[row * (row_elems / 32) + d / 32]) : 1.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = e4m3fn_to_f32((r.x >> (8 * k)) & 0xffu) * sc;
      v[4 + k] = e4m3fn_to_f32((r.y >> (8 * k)) & 0xffu) * sc;
    }
  }
}

struct KlArgs {
  SeqMeta meta;
  int T, H, D, HI, DI, k;
  float tau;
  const void *q;
  int q_dtype;
  const void *kv;
  int kv_dtype;
  const uint8_t *kv_scale;
  const void *q_idx;
  const float *w;
  const void *k_idx;
  int idx_dtype;
  const int32_t *topk_idx;
  const float *lse;
  float *loss, *d_w, *d_q_idx, *d_k_idx;
  float *mass, *score, *grad;  // [T, k] each
  float *part_w, *part_q;      // [T, chunks, HI], [T, chunks, HI, DI]
  int chunks;
};

// cache row of selected slot r of query t (-1: none)
__device__ __forceinline__ int64_t sel_row(const KlArgs &a, int t, int r, int n, int64_t start) {
  const int32_t pos = a.topk_idx[(size_t)t * a.k + r];
  return (pos >= 0 && pos < n) ? kv_row(a.meta, a.meta.q_seq[t], start, pos) : -1;
}

constexpr int kKlBatch = 4;
constexpr int kGzLd = 65;  // LDS row stride of the backward's g-weighted masks (odd: no bank conflicts)

// LDS row stride (in dwords) of a table read by four threads of different
// rows at once (the 4 head groups of k_kl_rows): congruent to 4 mod 64, so
// that their 16-byte reads fall on four different groups of banks
__host__ __device__ __forceinline__ int kl_ld(int dwords) { return dwords + (68 - dwords % 64) % 64; }  // 8-value chunks of a latent row requested together by k_kl_rows

// dot[i] += q[h] . v over 8 values at d, for the heads h = hg + 4 i of this thread
__device__ __forceinline__ void head_dots(const unsigned char *qs, bool qbf, int H, int D, int hg, int d,
                                          const float v[8], float dot[16]) {
  const int ld = kl_ld(qbf ? D / 2 : D) * (qbf ? 2 : 1);  // row stride in elements
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int h = hg + 4 * i;
    if (h < H) {
      float qv[8];
      if (qbf) {
        const uint4 r = *(const uint4 *)((const uint16_t *)qs + h * ld + d);
        const uint32_t wd[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qv[2 * e] = __uint_as_float(wd[e] << 16);
          qv[2 * e + 1] = __uint_as_float(wd[e] & 0xffff0000u);
        }
      } else {
        const float4 x = *(const float4 *)((const float *)qs + h * ld + d);
        const float4 y = *(const float4 *)((const float *)qs + h * ld + d + 4);
        qv[0] = x.x; qv[1] = x.y; qv[2] = x.z; qv[3] = x.w;
        qv[4] = y.x; qv[5] = y.y; qv[6] = y.z; qv[7] = y.w;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) dot[i] = fmaf(qv[e], v[e], dot[i]);
    }
  }
}

template <bool kMass>
__global__ __launch_bounds__(kKlThreads) void k_kl_rows(KlArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const bool qbf = a.q_dtype == SGA_BF16;
  const int qild = kl_ld(a.DI);                                    // padded rows (see kl_ld)
  const int qld = kl_ld(qbf ? a.D / 2 : a.D) * (qbf ? 2 : 1);
  float *qi = (float *)smem;                          // [HI, qild] index query, fp32
  float *wsh = qi + a.HI * qild;                      // [HI]
  unsigned char *qs = (unsigned char *)(wsh + 64);   // [H, qld] query as stored (bf16 or fp32)
  const int t = blockIdx.y, r0 = blockIdx.x * kKlRows;
  const int tid = threadIdx.x, j = tid >> 2, hg = tid & 3;
  int64_t start;
  const int n = query_candidates(a.meta, t, &start);
  for (int i = tid; i < a.HI * a.DI; i += kKlThreads)
    qi[(i / a.DI) * qild + i % a.DI] =
        a.idx_dtype == SGA_F32 ? ((const float *)a.q_idx)[(size_t)t * a.HI * a.DI + i]
                               : e4m3fn_to_f32(((const uint8_t *)a.q_idx)[(size_t)t * a.HI * a.DI + i]);
  for (int i = tid; i < a.HI; i += kKlThreads) wsh[i] = a.w[(size_t)t * a.HI + i];
  for (int i = tid; kMass && i < a.H * a.D; i += kKlThreads) {
    const int o = (i / a.D) * qld + i % a.D;
    if (qbf)
      ((uint16_t *)qs)[o] = ((const uint16_t *)a.q)[(size_t)t * a.H * a.D + i];
    else
      ((float *)qs)[o] = ((const float *)a.q)[(size_t)t * a.H * a.D + i];
  }
  __syncthreads();
  const int r = r0 + j;
  const int64_t row = r < a.k ? sel_row(a, t, r, n, start) : -1;
  // attention mass: heads hg, hg + 4, ... of row j
  float dot[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) dot[i] = 0.0f;
  // bf16 and MXFP8 rows are requested kKlBatch chunks of 8 values at a time
  // before any arithmetic on them: one memory latency per batch instead of
  // one per chunk
  const bool staged = a.kv_dtype == SGA_BF16 || a.kv_dtype == SGA_MXFP8_E4M3FN;
  if (kMass && row >= 0 && staged) {
    for (int base = 0; base < a.D; base += 8 * kKlBatch) {
      uint4 st[kKlBatch];
#pragma unroll
      for (int c = 0; c < kKlBatch; ++c) {
        const int d = base + c * 8;
        if (d < a.D) {
          if (a.kv_dtype == SGA_BF16) {
            st[c] = *(const uint4 *)((const uint16_t *)a.kv + row * a.D + d);
          } else {
            const uint2 r = *(const uint2 *)((const uint8_t *)a.kv + row * a.D + d);
            st[c] = make_uint4(r.x, r.y, a.kv_scale[row * (a.D / 32) + d / 32], 0u);
          }
        }
      }
#pragma unroll
      for (int c = 0; c < kKlBatch; ++c) {
        const int d = base + c * 8;
        if (d < a.D) {
          float v[8];
          if (a.kv_dtype == SGA_BF16) {
            const uint32_t wd[4] = {st[c].x, st[c].y, st[c].z, st[c].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[2 * e] = __uint_as_float(wd[e] << 16);
              v[2 * e + 1] = __uint_as_float(wd[e] & 0xffff0000u);
            }
          } else {
            const float sc = e8m0_to_f32(st[c].z);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[e] = e4m3fn_to_f32((st[c].x >> (8 * e)) & 0xffu) * sc;
              v[4 + e] = e4m3fn_to_f32((st[c].y >> (8 * e)) & 0xffu) * sc;
            }
          }
          head_dots(qs, qbf, a.H, a.D, hg, d, v, dot);
        }
      }
    }
  } else if (kMass && row >= 0) {
    for (int d = 0; d < a.D; d += 8) {
      float v[8];
      load8(a.kv, a.kv_dtype, a.kv_scale, a.D, row, d, v);
      head_dots(qs, qbf, a.H, a.D, hg, d, v, dot);
    }
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int h = hg + 4 * i;
    if (h < a.H && row >= 0) m += __expf(a.tau * dot[i] - a.lse[(size_t)t * a.H + h]);
  }
  // indexer score: index heads hg, hg + 4, ...
  float z[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  if (row >= 0) {
    // the key row is requested 4 chunks of 8 values at a time
    for (int base = 0; base < a.DI; base += 32) {
      float kv8[4][8];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (base + c * 8 < a.DI) load8(a.k_idx, a.idx_dtype, nullptr, a.DI, row, base + c * 8, kv8[c]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (base + c * 8 < a.DI) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int h = hg + 4 * i;
            if (h < a.HI) {
              const float *qh = qi + h * qild + base + c * 8;
#pragma unroll
              for (int e = 0; e < 8; ++e) z[i] = fmaf(qh[e], kv8[c][e], z[i]);
            }
          }
        }
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int h = hg + 4 * i;
    if (h < a.HI) s = fmaf(fmaxf(z[i], 0.0f), wsh[h], s);
  }
  // sum over the 4 threads of the row (consecutive lanes)
  m += __shfl_xor(m, 1);
  m += __shfl_xor(m, 2);
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  if (hg == 0 && r < a.k) {
    if (kMass) a.mass[(size_t)t * a.k + r] = row >= 0 ? m : 0.0f;
    a.score[(size_t)t * a.k + r] = row >= 0 ? s : -INFINITY;
  }
}

// Attention mass of 64 selected rows with bf16 MFMA (64 heads, bf16 q, bf16
// or MXFP8 rows, Dc + Dr = 32 kKlKsteps): wave w takes heads 16 w .. 16 w + 15
// and all 64 rows, S^T = rows . q^T per 16-row tile (16x16x32 bf16 MFMA; the
// query slice stays in VGPRs as the B operand; MXFP8 rows are expanded
// exactly to bf16 on the way in).
constexpr int kKlKsteps = 18;

// 8 E4M3FN bytes -> 8 bf16 (exact), as a 16-byte MFMA operand
__device__ __forceinline__ v4i fp8x8_to_bf16(uint2 w8) {
  return (v4i){(int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w8.x, 1.0f, false)),
               (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w8.x, 1.0f, true)),
               (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w8.y, 1.0f, false)),
               (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w8.y, 1.0f, true))};
}

// With kScores (64 FP8 index heads x 128 dims) the same workgroup also
// computes each row's indexer score: z = kI . qI^T per 16-row tile by bf16
// MFMA (E4M3FN values are exact in bf16, so z is the fp32 sum of exact
// products), then sum_h w_h ReLU(z) over the wave's 16 heads and the 4 waves.
template <bool kScores>
__global__ __launch_bounds__(kKlThreads) void k_kl_mass_mfma(KlArgs a) {
  __shared__ float part[kKlThreads / 64][kKlRows];
  __shared__ float spart[kKlThreads / 64][kKlRows];
  __shared__ int64_t rows[kKlRows];
  const int t = blockIdx.y, r0 = blockIdx.x * kKlRows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
  int64_t start;
  const int n = query_candidates(a.meta, t, &start);
  if (tid < kKlRows) {
    const int r = r0 + tid;
    rows[tid] = r < a.k ? sel_row(a, t, r, n, start) : -1;
  }
  const int head = wave * 16 + c16;
  const uint16_t *qh = (const uint16_t *)a.q + ((size_t)t * 64 + head) * a.D;
  v4i qreg[kKlKsteps];
#pragma unroll
  for (int ks = 0; ks < kKlKsteps; ++ks) qreg[ks] = *(const v4i *)(qh + ks * 32 + 8 * g);
  const float lse_h = a.lse[(size_t)t * 64 + head];
  const bool mx = a.kv_dtype == SGA_MXFP8_E4M3FN;
  // index query of index head `head` (B operand) and its weight
  v4i qireg[4];
  float w_h = 0.0f;
  if (kScores) {
    const uint8_t *qih = (const uint8_t *)a.q_idx + ((size_t)t * 64 + head) * 128;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qireg[ks] = fp8x8_to_bf16(*(const uint2 *)(qih + ks * 32 + 8 * g));
    w_h = a.w[(size_t)t * 64 + head];
  }
  __syncthreads();
  for (int rt = 0; rt < kKlRows / 16; ++rt) {
    const int64_t row = rows[rt * 16 + c16];
    v4i av[kKlKsteps];
#pragma unroll
    for (int ks = 0; ks < kKlKsteps; ++ks) {
      const int d = ks * 32 + 8 * g;
      if (row < 0) {
        av[ks] = (v4i){0, 0, 0, 0};
      } else if (!mx) {
        av[ks] = *(const v4i *)((const uint16_t *)a.kv + row * a.D + d);
      } else {
        const uint2 w8 = *(const uint2 *)((const uint8_t *)a.kv + row * a.D + d);
        const float sc = e8m0_to_f32(a.kv_scale[row * (a.D / 32) + ks]);
        av[ks] = (v4i){(int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w8.x, sc, false)),
                       (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w8.x, sc, true)),
                       (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w8.y, sc, false)),
                       (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w8.y, sc, true))};
      }
    }
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kKlKsteps; ++ks)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av[ks]), __builtin_bit_cast(v8bf, qreg[ks]),
                                                     acc, 0, 0, 0);
    v4f zc = {0.f, 0.f, 0.f, 0.f};
    if (kScores) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const v4i kb = row < 0 ? (v4i){0, 0, 0, 0}
                               : fp8x8_to_bf16(*(const uint2 *)((const uint8_t *)a.k_idx + row * 128 + ks * 32 + 8 * g));
        zc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, kb), __builtin_bit_cast(v8bf, qireg[ks]),
                                                    zc, 0, 0, 0);
      }
    }
    // acc[i]: logit of row rt*16 + 4 g + i for this lane's head; zc[i]: its z
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = rt * 16 + 4 * g + i;
      float e = rows[j] >= 0 ? __expf(a.tau * acc[i] - lse_h) : 0.0f;
      e += __shfl_xor(e, 1);
      e += __shfl_xor(e, 2);
      e += __shfl_xor(e, 4);
      e += __shfl_xor(e, 8);
      if (c16 == 0) part[wave][j] = e;
      if (kScores) {
        float sc = fmaxf(zc[i], 0.0f) * w_h;
        sc += __shfl_xor(sc, 1);
        sc += __shfl_xor(sc, 2);
        sc += __shfl_xor(sc, 4);
        sc += __shfl_xor(sc, 8);
        if (c16 == 0) spart[wave][j] = sc;
      }
    }
  }
  __syncthreads();
  if (tid < kKlRows && r0 + tid < a.k) {
    float m = 0.0f;
#pragma unroll
    for (int w = 0; w < kKlThreads / 64; ++w) m += part[w][tid];
    a.mass[(size_t)t * a.k + r0 + tid] = rows[tid] >= 0 ? m : 0.0f;
    if (kScores) {
      float sc = 0.0f;
#pragma unroll
      for (int w = 0; w < kKlThreads / 64; ++w) sc += spart[w][tid];
      a.score[(size_t)t * a.k + r0 + tid] = rows[tid] >= 0 ? sc + 0.0f : -INFINITY;
    }
  }
}

__device__ __forceinline__ float block_sum(float v, float *red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = 0.0f;
  for (int i = 0; i < kKlThreads / 64; ++i) s += red[i];
  return s;
}

__device__ __forceinline__ float block_max(float v, float *red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = -INFINITY;
  for (int i = 0; i < kKlThreads / 64; ++i) s = fmaxf(s, red[i]);
  return s;
}

__global__ __launch_bounds__(kKlThreads) void k_kl_loss(KlArgs a) {
  __shared__ float red[kKlThreads / 64];
  const int t = blockIdx.x;
  const float *sc = a.score + (size_t)t * a.k, *ms = a.mass + (size_t)t * a.k;
  float mx = -INFINITY, tot = 0.0f;
  for (int r = threadIdx.x; r < a.k; r += kKlThreads) {
    mx = fmaxf(mx, sc[r]);
    tot += ms[r];
  }
  mx = block_max(mx, red);
  tot = block_sum(tot, red);
  float z = 0.0f;
  if (mx > -INFINITY)
    for (int r = threadIdx.x; r < a.k; r += kKlThreads) z += __expf(sc[r] - mx);
  z = block_sum(z, red);
  const float lz = mx + __logf(z);
  float loss = 0.0f;
  for (int r = threadIdx.x; r < a.k; r += kKlThreads) {
    float g = 0.0f;
    if (sc[r] > -INFINITY) {
      const float logq = sc[r] - lz;
      const float tg = tot > 0.0f ? ms[r] / tot : 0.0f;
      if (tg > 0.0f) loss += tg * (__logf(tg) - logq);
      g = __expf(logq) - tg;
    }
    a.grad[(size_t)t * a.k + r] = g;
  }
  loss = block_sum(loss, red);
  if (threadIdx.x == 0) a.loss[t] = mx > -INFINITY ? loss : 0.0f;
}

// kMfmaZ (64 FP8 index heads x 128 dims): z by bf16 MFMA as in
// k_kl_mass_mfma, wave w taking index heads 16 w .. 16 w + 15
template <bool kMfmaZ>
__global__ __launch_bounds__(kKlThreads) void k_kl_backward(KlArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // rows of qi and kr are padded by four words: 16-byte aligned, and the z
  // loop's lanes (16 rows x 4 heads per wave, same d) hit distinct banks
  const int ld = a.DI + 4;
  float *qi = (float *)smem;                 // [HI, DI + 1]
  float *wsh = qi + a.HI * ld;               // [64]
  float *kr = wsh + 64;                      // [kKlRows, DI + 1] selected index keys
  float *gz = kr + kKlRows * ld;             // [kKlRows, kGzLd]: g w [z > 0]
  float *rz = gz + kKlRows * kGzLd;          // [kKlRows, kGzLd]: g ReLU(z)
  __shared__ float gr[kKlRows];
  __shared__ int64_t rows[kKlRows];
  const int t = blockIdx.y, r0 = blockIdx.x * kKlRows;
  const int tid = threadIdx.x;
  int64_t start;
  const int n = query_candidates(a.meta, t, &start);
  for (int i = tid; i < a.HI * a.DI; i += kKlThreads)
    qi[(i / a.DI) * ld + i % a.DI] =
        a.idx_dtype == SGA_F32 ? ((const float *)a.q_idx)[(size_t)t * a.HI * a.DI + i]
                               : e4m3fn_to_f32(((const uint8_t *)a.q_idx)[(size_t)t * a.HI * a.DI + i]);
  for (int i = tid; i < a.HI; i += kKlThreads) wsh[i] = a.w[(size_t)t * a.HI + i];
  if (tid < kKlRows) {
    const int r = r0 + tid;
    const int64_t row = r < a.k ? sel_row(a, t, r, n, start) : -1;
    rows[tid] = row;
    gr[tid] = row >= 0 ? a.grad[(size_t)t * a.k + r] : 0.0f;
  }
  __syncthreads();
  for (int i = tid; i < kKlRows * (a.DI / 8); i += kKlThreads) {
    const int j = i / (a.DI / 8), d = (i % (a.DI / 8)) * 8;
    float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (rows[j] >= 0) load8(a.k_idx, a.idx_dtype, nullptr, a.DI, rows[j], d, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) kr[j * ld + d + e] = v[e];
  }
  __syncthreads();
  if (kMfmaZ) {
    const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
    const int h = wave * 16 + c16;
    const uint8_t *qih = (const uint8_t *)a.q_idx + ((size_t)t * 64 + h) * 128;
    v4i qireg[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qireg[ks] = fp8x8_to_bf16(*(const uint2 *)(qih + ks * 32 + 8 * g));
#pragma unroll
    for (int rt = 0; rt < kKlRows / 16; ++rt) {
      const int64_t row = rows[rt * 16 + c16];
      v4f zc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const v4i kb = row < 0 ? (v4i){0, 0, 0, 0}
                               : fp8x8_to_bf16(*(const uint2 *)((const uint8_t *)a.k_idx + row * 128 + ks * 32 + 8 * g));
        zc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, kb), __builtin_bit_cast(v8bf, qireg[ks]),
                                                    zc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = rt * 16 + 4 * g + i;
        gz[j * kGzLd + h] = zc[i] > 0.0f ? gr[j] * wsh[h] : 0.0f;
        rz[j * kGzLd + h] = gr[j] * fmaxf(zc[i], 0.0f);
      }
    }
  } else {
    // z of (row j, index head h) for 4 threads per row
    const int j = tid >> 2, hg = tid & 3;
    for (int h = hg; h < a.HI; h += 4) {
      float z = 0.0f;
      for (int d = 0; d < a.DI; d += 4) {
        const float4 x = *(const float4 *)(qi + h * ld + d), y = *(const float4 *)(kr + j * ld + d);
        z = fmaf(x.x, y.x, fmaf(x.y, y.y, fmaf(x.z, y.z, fmaf(x.w, y.w, z))));
      }
      gz[j * kGzLd + h] = z > 0.0f ? gr[j] * wsh[h] : 0.0f;
      rz[j * kGzLd + h] = gr[j] * fmaxf(z, 0.0f);
    }
  }
  __syncthreads();
  const size_t chunk = (size_t)t * a.chunks + blockIdx.x;
  for (int h = tid; h < a.HI; h += kKlThreads) {
    float s = 0.0f;
    for (int j = 0; j < kKlRows; ++j) s += rz[j * kGzLd + h];
    a.part_w[chunk * a.HI + h] = s;
  }
  if (kMfmaZ) {
    // 64 x 128 shapes: both gradient products by fp32 MFMA 16x16x4 (fp32
    // operands, as g is too small for bf16 at this precision). Wave w takes
    // index-head tile w of d_qI = gz^T kr and row tile w of d_kI = gz qi,
    // each over the 8 tiles of 16 d.
    const int lane = tid & 63, wave = tid >> 6, g4 = lane >> 4, c16 = lane & 15;
    v4f accq[8], acck[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) accq[dt] = acck[dt] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int ks = 0; ks < 16; ++ks) {
      const int kk = ks * 4 + g4;  // row (d_qI) or index head (d_kI) of this lane's k
      const float aq = gz[kk * kGzLd + wave * 16 + c16];          // A[i = head][k = row]
      const float ak = gz[(wave * 16 + c16) * kGzLd + kk];        // A[i = row][k = head]
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        accq[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(aq, kr[kk * ld + dt * 16 + c16], accq[dt], 0, 0, 0);
        acck[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(ak, qi[kk * ld + dt * 16 + c16], acck[dt], 0, 0, 0);
      }
    }
    // C[i = 4 g4 + r][j = c16] of each tile
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * g4 + r, d = dt * 16 + c16;
        a.part_q[chunk * 64 * 128 + (size_t)(wave * 16 + i) * 128 + d] = accq[dt][r];
        const int j = wave * 16 + i;
        if (rows[j] >= 0 && gr[j] != 0.0f) atomicAdd(a.d_k_idx + rows[j] * 128 + d, acck[dt][r]);
      }
    return;
  }
  // four consecutive outputs per thread (16-byte LDS reads)
  for (int i = 4 * tid; i < a.HI * a.DI; i += 4 * kKlThreads) {
    const int h = i / a.DI, d = i % a.DI;
    float4 s = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < kKlRows; ++j) {
      const float gv = gz[j * kGzLd + h];
      const float4 x = *(const float4 *)(kr + j * ld + d);
      s.x = fmaf(gv, x.x, s.x); s.y = fmaf(gv, x.y, s.y); s.z = fmaf(gv, x.z, s.z); s.w = fmaf(gv, x.w, s.w);
    }
    *(float4 *)(a.part_q + chunk * a.HI * a.DI + i) = s;
  }
  for (int i = 4 * tid; i < kKlRows * a.DI; i += 4 * kKlThreads) {
    const int j = i / a.DI, d = i % a.DI;
    if (rows[j] < 0 || gr[j] == 0.0f) continue;
    float4 s = {0.f, 0.f, 0.f, 0.f};
    for (int h = 0; h < a.HI; ++h) {
      const float gv = gz[j * kGzLd + h];
      const float4 x = *(const float4 *)(qi + h * ld + d);
      s.x = fmaf(gv, x.x, s.x); s.y = fmaf(gv, x.y, s.y); s.z = fmaf(gv, x.z, s.z); s.w = fmaf(gv, x.w, s.w);
    }
    float *dk = a.d_k_idx + rows[j] * a.DI + d;
    atomicAdd(dk, s.x);
    atomicAdd(dk + 1, s.y);
    atomicAdd(dk + 2, s.z);
    atomicAdd(dk + 3, s.w);
  }
}

__global__ __launch_bounds__(kKlThreads) void k_kl_reduce(KlArgs a) {
  const int t = blockIdx.y;
  const int i = blockIdx.x * kKlThreads + threadIdx.x;  // over HI * DI + HI outputs
  const int nq = a.HI * a.DI;
  if (i >= nq + a.HI) return;
  float s = 0.0f;
  if (i < nq) {
    for (int c = 0; c < a.chunks; ++c) s += a.part_q[((size_t)t * a.chunks + c) * nq + i];
    a.d_q_idx[(size_t)t * nq + i] = s;
  } else {
    const int h = i - nq;
    for (int c = 0; c < a.chunks; ++c) s += a.part_w[((size_t)t * a.chunks + c) * a.HI + h];
    a.d_w[(size_t)t * a.HI + h] = s;
  }
}

}  // namespace

size_t indexer_kl_ws_bytes(int T, int k, int HI, int DI) {
  const size_t chunks = (k + kKlRows - 1) / kKlRows;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return 3 * al((size_t)T * k * 4) + al((size_t)T * chunks * HI * 4) + al((size_t)T * chunks * HI * DI * 4);
}

size_t indexer_kl_smem(int H, int D, int HI, int DI, int q_dtype) {
  const size_t rows = ((size_t)HI * kl_ld(DI) + 64) * 4 + (size_t)H * kl_ld(q_dtype == SGA_BF16 ? D / 2 : D) * 4;
  const size_t back = ((size_t)HI * (DI + 4) + 64 + (size_t)kKlRows * (DI + 4) + 2 * kKlRows * kGzLd) * 4;
  return rows > back ? rows : back;
}

hipError_t launch_indexer_kl(const SeqMeta &m, int T, int H, int D, int HI, int DI, int k, float tau,
                             const void *q, int q_dtype, const void *kv, int kv_dtype,
                             const uint8_t *kv_scale, const void *q_idx, const float *w,
                             const void *k_idx, int idx_dtype, const int32_t *topk_idx,
                             const float *lse, float *loss, float *d_w, float *d_q_idx, float *d_k_idx,
                             void *ws, hipStream_t s) {
  if (T == 0) return hipSuccess;
  KlArgs a;
  a.meta = m;
  a.T = T; a.H = H; a.D = D; a.HI = HI; a.DI = DI; a.k = k; a.tau = tau;
  a.q = q; a.q_dtype = q_dtype; a.kv = kv; a.kv_dtype = kv_dtype; a.kv_scale = kv_scale;
  a.q_idx = q_idx; a.w = w; a.k_idx = k_idx; a.idx_dtype = idx_dtype;
  a.topk_idx = topk_idx; a.lse = lse;
  a.loss = loss; a.d_w = d_w; a.d_q_idx = d_q_idx; a.d_k_idx = d_k_idx;
  a.chunks = (k + kKlRows - 1) / kKlRows;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char *c = (char *)ws;
  a.mass = (float *)c; c += al((size_t)T * k * 4);
  a.score = (float *)c; c += al((size_t)T * k * 4);
  a.grad = (float *)c; c += al((size_t)T * k * 4);
  a.part_w = (float *)c; c += al((size_t)T * a.chunks * HI * 4);
  a.part_q = (float *)c;
  size_t smem = indexer_kl_smem(H, D, HI, DI, q_dtype);
  // the MI355X shapes take the attention mass from the MFMA kernel
  const bool mfma = H == 64 && q_dtype == SGA_BF16 && D == 32 * kKlKsteps &&
                    (kv_dtype == SGA_BF16 || kv_dtype == SGA_MXFP8_E4M3FN);
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void *)k_kl_rows<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    (void)hipFuncSetAttribute((const void *)k_kl_rows<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    (void)hipFuncSetAttribute((const void *)k_kl_backward<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    (void)hipFuncSetAttribute((const void *)k_kl_backward<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    (void)hipGetLastError();
    attr = true;
  }
  const dim3 grid(a.chunks, T);
  if (mfma && HI == 64 && DI == 128 && idx_dtype == SGA_FP8_E4M3FN) {
    hipLaunchKernelGGL(k_kl_mass_mfma<true>, grid, dim3(kKlThreads), 0, s, a);
  } else if (mfma) {
    hipLaunchKernelGGL(k_kl_mass_mfma<false>, grid, dim3(kKlThreads), 0, s, a);
    hipLaunchKernelGGL(k_kl_rows<false>, grid, dim3(kKlThreads), ((size_t)HI * kl_ld(DI) + 64) * 4, s, a);
  } else {
    hipLaunchKernelGGL(k_kl_rows<true>, grid, dim3(kKlThreads), smem, s, a);
  }
  hipLaunchKernelGGL(k_kl_loss, dim3(T), dim3(kKlThreads), 0, s, a);
  if (HI == 64 && DI == 128 && idx_dtype == SGA_FP8_E4M3FN)
    hipLaunchKernelGGL(k_kl_backward<true>, grid, dim3(kKlThreads), smem, s, a);
  else
    hipLaunchKernelGGL(k_kl_backward<false>, grid, dim3(kKlThreads), smem, s, a);
  hipLaunchKernelGGL(k_kl_reduce, dim3((HI * DI + HI + kKlThreads - 1) / kKlThreads, T), dim3(kKlThreads), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace sga
