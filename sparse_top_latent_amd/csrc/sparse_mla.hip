// Sparse MLA over the selected latent rows, followed by the sigmoid output gate.
//
// Source: "A.X-K2: a sparse-attention upgrade that costs nothing, trained
// natively in FP8", section "Sparse Gated Attention" (MLA runs exactly over the
// selected set KV[I_topk]; a learned head-specific gate is applied to the
// attention output before Wo); "SK Telecom Opens A.X K2: 688B Parameters and
// One Telling Benchmark", block-diagram caption (sigmoid output gate); "A.X K2
// Technical Report", section 2 (MLA backbone with a head-specific output gate).
//
// Absorbed MLA: all heads share one cached row [c_s | kR_s] per position, so a
// gathered row serves every head. For query t and head h:
//   logit_s = tau * q[t,h,:] . row_s ;  p = softmax over the selected rows ;
//   o = sum_s p_s c_s ;  y = sigmoid(g[t,h,:]) * o.
//
// Kernels:
//  * k_mla_f32: generic fp32 path, one workgroup per (query, head).
//  * k_mla_split (MI355X path, H = 64, Dc = 512, Dr = 64): the selected rows of
//    a query are cut into splits of 128; one workgroup per (split, query)
//    gathers 32-row tiles into LDS (bf16, or MXFP8 expanded exactly to bf16),
//    and each of its 4 waves owns 16 heads:
//      S^T = rows . Q^T  with bf16 16x16x32 MFMA (the query slice stays in VGPRs),
//      online softmax per head in fp32 (exp2 domain),
//      O^T += V^T . P^T  with bf16 MFMA; P^T comes straight from the S^T
//      accumulator layout, V^T is read column-wise from the LDS tile.
//    It writes an fp32 partial (max, sum, O) per (query, split, head).
//  * k_mla_combine: merges the splits of each (query, head) with the usual
//    log-sum-exp rescaling and applies the gate in the epilogue.

#include "kernels.h"

namespace sga {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// --------------------------------------------------------------------------
// block reductions
// --------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}
template <bool kMax>
__device__ __forceinline__ float block_reduce(float v, float *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = kMax ? wave_max(v) : wave_sum(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nw; ++i) r = kMax ? fmaxf(r, red[i]) : r + red[i];
  __syncthreads();
  return r;
}

// --------------------------------------------------------------------------
// generic fp32 path
// --------------------------------------------------------------------------
constexpr int kF32Block = 256;
constexpr int kF32MaxD = 1024;
constexpr int kF32MaxK = 4096;

__global__ __launch_bounds__(kF32Block) void k_mla_f32(MlaArgs a) {
  __shared__ float qs[kF32MaxD];
  __shared__ float pr[kF32MaxK];
  __shared__ int64_t rows[kF32MaxK];
  __shared__ float red[kF32Block / 64];
  const int h = blockIdx.x, t = blockIdx.y;
  const int D = a.Dc + a.Dr;
  int64_t start;
  const int L = seq_len_clipped(a.meta, a.meta.q_seq[t], &start);
  const float *q = (const float *)a.q + ((size_t)t * a.H + h) * D;
  const float *kv = (const float *)a.kv;
  for (int i = threadIdx.x; i < D; i += kF32Block) qs[i] = q[i];
  __syncthreads();
  float mx = -INFINITY;
  for (int r = threadIdx.x; r < a.k; r += kF32Block) {
    int32_t pos = a.topk_idx[(size_t)t * a.k + r];
    bool ok = pos >= 0 && pos < L;
    int64_t row = ok ? start + pos : -1;
    float lg = -INFINITY;
    if (ok) {
      const float *kr = kv + row * D;
      float acc = 0.0f;
      for (int d = 0; d < D; ++d) acc = fmaf(qs[d], kr[d], acc);
      lg = a.tau * acc;
    }
    rows[r] = row;
    pr[r] = lg;
    mx = fmaxf(mx, lg);
  }
  mx = block_reduce<true>(mx, red);
  float sum = 0.0f;
  for (int r = threadIdx.x; r < a.k; r += kF32Block) {
    float p = rows[r] >= 0 ? __expf(pr[r] - mx) : 0.0f;
    pr[r] = p;
    sum += p;
  }
  sum = block_reduce<false>(sum, red);  // includes a barrier: pr[] is complete
  const bool empty = !(mx > -INFINITY);
  const float inv = empty ? 0.0f : 1.0f / sum;
  for (int c = threadIdx.x; c < a.Dc; c += kF32Block) {
    float acc = 0.0f;
    for (int r = 0; r < a.k; ++r) {
      int64_t row = rows[r];
      if (row >= 0) acc = fmaf(pr[r], kv[row * D + c], acc);
    }
    float o = acc * inv;
    size_t oi = ((size_t)t * a.H + h) * a.Dc + c;
    if (a.gate) o *= sigmoidf_exact_ends(load_as_f32(a.gate, a.gate_dtype, oi));
    store_from_f32(a.out, a.out_dtype, oi, o);
  }
  if (a.lse && threadIdx.x == 0) a.lse[(size_t)t * a.H + h] = empty ? -INFINITY : mx + __logf(sum);
}

// --------------------------------------------------------------------------
// MI355X path
// --------------------------------------------------------------------------
constexpr int kH = 64, kDc = 512, kD = 576;  // d_rope = 64
constexpr int kTile = 32;                 // rows per LDS tile
constexpr int kLdsStride = kD + 8;        // bf16 elements per LDS row (pad 16 B)
constexpr int kKsteps = kD / 32;          // 18 MFMA k-steps for q . row
constexpr int kCt = kDc / 16;             // 32 channel tiles of the value

__device__ __forceinline__ v4f mfma_bf16(const v8bf &a, const v8bf &b, const v4f &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8bf as_v8bf(const v4i &x) { return __builtin_bit_cast(v8bf, x); }

template <bool kMx>
__device__ __forceinline__ void gather_tile(uint16_t *tile, const int64_t *rows, int r0, int nrows,
                                            const void *kv, const uint8_t *kv_scale) {
  if (!kMx) {
    // 32 rows x 72 chunks of 16 bytes
    const uint8_t *base = (const uint8_t *)kv;
#pragma unroll
    for (int j = 0; j < (kTile * 72) / 256; ++j) {
      int c = threadIdx.x + 256 * j;
      int r = c / 72, col = c - r * 72;
      int ri = r0 + r;
      int64_t g = ri < nrows ? rows[ri] : -1;
      v4i v = {0, 0, 0, 0};
      if (g >= 0) v = __builtin_nontemporal_load((const v4i *)(base + g * (kD * 2) + col * 16));
      *(v4i *)(tile + r * kLdsStride + col * 8) = v;
    }
  } else {
    // 32 rows x 36 chunks of 16 E4M3FN values; chunk col lies in scale block col/2
    const uint8_t *base = (const uint8_t *)kv;
    for (int c = threadIdx.x; c < kTile * 36; c += 256) {
      int r = c / 36, col = c - r * 36;
      int ri = r0 + r;
      int64_t g = ri < nrows ? rows[ri] : -1;
      v4i out0 = {0, 0, 0, 0}, out1 = {0, 0, 0, 0};
      if (g >= 0) {
        v4i v = __builtin_nontemporal_load((const v4i *)(base + g * kD + col * 16));
        float sc = e8m0_to_f32(kv_scale[g * (kD / 32) + (col >> 1)]);
        uint32_t w[4] = {(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            uint32_t b0 = (w[i] >> (16 * hh)) & 0xFFu;
            uint32_t b1 = (w[i] >> (16 * hh + 8)) & 0xFFu;
            uint32_t lo = f32_to_bf16_bits(e4m3fn_to_f32(b0) * sc);
            uint32_t hi = f32_to_bf16_bits(e4m3fn_to_f32(b1) * sc);
            o[i * 2 + hh] = lo | (hi << 16);
          }
        }
        out0 = (v4i){(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
        out1 = (v4i){(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
      }
      v4i *dst = (v4i *)(tile + r * kLdsStride + col * 16);
      dst[0] = out0;
      dst[1] = out1;
    }
  }
}

template <bool kMx>
__global__ __launch_bounds__(256) void k_mla_split(MlaArgs a, float *__restrict__ opart,
                                                   float2 *__restrict__ ml) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTile * kLdsStride];
  __shared__ int64_t rows[kMlaRowsPerSplit];
  const int split = blockIdx.x, t = blockIdx.y, S = gridDim.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  int64_t start;
  const int L = seq_len_clipped(a.meta, a.meta.q_seq[t], &start);
  const int r0 = split * kMlaRowsPerSplit;
  const int nrows = min(kMlaRowsPerSplit, a.k - r0);
  for (int r = threadIdx.x; r < kMlaRowsPerSplit; r += 256) {
    int32_t pos = r < nrows ? a.topk_idx[(size_t)t * a.k + r0 + r] : -1;
    rows[r] = (pos >= 0 && pos < L) ? start + pos : -1;
  }
  // query slice of this wave's head (B operand of S^T = rows . Q^T)
  const int head = wave * 16 + c16;
  const uint8_t *qh = (const uint8_t *)a.q + ((size_t)t * kH + head) * kD * 2;
  v8bf qreg[kKsteps];
#pragma unroll
  for (int ks = 0; ks < kKsteps; ++ks) qreg[ks] = as_v8bf(*(const v4i *)(qh + (ks * 32 + 8 * g) * 2));

  v4f acc[kCt];
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) acc[ct] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  const float scale2 = a.tau * kLog2e;  // logits kept in the exp2 domain

  const int ntiles = (nrows + kTile - 1) / kTile;
  for (int tt = 0; tt < ntiles; ++tt) {
    __syncthreads();
    gather_tile<kMx>(tile, rows, tt * kTile, nrows, a.kv, a.kv_scale);
    __syncthreads();
    // S^T[row][head] for the two 16-row halves of the tile
    v4f s[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      v4f sacc = {0.f, 0.f, 0.f, 0.f};
      const uint16_t *rp = tile + (rt * 16 + c16) * kLdsStride + 8 * g;
#pragma unroll
      for (int ks = 0; ks < kKsteps; ++ks) sacc = mfma_bf16(as_v8bf(*(const v4i *)(rp + ks * 32)), qreg[ks], sacc);
      s[rt] = sacc;
    }
    float lg[8];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int ri = tt * kTile + (j >> 2) * 16 + 4 * g + (j & 3);
      bool ok = ri < nrows && rows[ri] >= 0;
      lg[j] = ok ? s[j >> 2][j & 3] * scale2 : -INFINITY;
      mt = fmaxf(mt, lg[j]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    if (!(m_new > -INFINITY)) continue;  // nothing valid yet for this head
    const float alpha = exp2f(m_run - m_new);
    float p[8], ps = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = exp2f(lg[j] - m_new);
      ps += p[j];
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    v8bf pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) pb[j] = (__bf16)p[j];
    // V^T operand: rows {4g..4g+3, 16+4g..16+4g+3}, channel ct*16 + c16
    const uint16_t *vp = tile + c16;
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) {
      v8bf va;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        int r = (j < 4) ? 4 * g + j : 16 + 4 * g + (j - 4);
        va[j] = __builtin_bit_cast(__bf16, vp[r * kLdsStride + ct * 16]);
      }
      acc[ct] = mfma_bf16(va, pb, acc[ct] * alpha);
    }
  }
  // partial O^T: lane holds channels ct*16 + 4g + i of head `head`
  const size_t pbase = (((size_t)t * S + split) * kH + head) * kDc;
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) *(v4f *)(opart + pbase + ct * 16 + 4 * g) = acc[ct];
  if (g == 0) ml[((size_t)t * S + split) * kH + head] = make_float2(m_run, l_run);
}

__global__ __launch_bounds__(128) void k_mla_combine(MlaArgs a, const float *__restrict__ opart,
                                                     const float2 *__restrict__ ml, int S) {
  const int h = blockIdx.x, t = blockIdx.y;
  const int c = threadIdx.x * 4;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[((size_t)t * S + s) * kH + h].x);
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (M > -INFINITY) {
    float wsum = 0.0f;
    for (int s = 0; s < S; ++s) {
      float2 v = ml[((size_t)t * S + s) * kH + h];
      float wgt = v.x > -INFINITY ? exp2f(v.x - M) : 0.0f;
      if (wgt == 0.0f) continue;
      wsum += wgt * v.y;
      v4f x = *(const v4f *)(opart + (((size_t)t * S + s) * kH + h) * kDc + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = fmaf(wgt, x[i], o[i]);
    }
    const float inv = 1.0f / wsum;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] *= inv;
    lse = M / kLog2e + __logf(wsum);
  }
  const size_t oi = ((size_t)t * kH + h) * kDc + c;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float y = o[i];
    if (a.gate) y *= sigmoidf_exact_ends(load_as_f32(a.gate, a.gate_dtype, oi + i));
    store_from_f32(a.out, a.out_dtype, oi + i, y);
  }
  if (a.lse && threadIdx.x == 0) a.lse[(size_t)t * kH + h] = lse;
}

}  // namespace

hipError_t launch_mla_f32(const MlaArgs &a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_mla_f32, dim3(a.H, a.T), dim3(kF32Block), 0, s, a);
  return hipGetLastError();
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int mla_splits(int k) { return (k + kMlaRowsPerSplit - 1) / kMlaRowsPerSplit; }

size_t mla_split_ws_bytes(int T, int k) {
  size_t S = (size_t)mla_splits(k);
  return align256((size_t)T * S * kH * kDc * 4) + align256((size_t)T * S * kH * sizeof(float2));
}

hipError_t launch_mla_split(const MlaArgs &a, void *ws, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int S = mla_splits(a.k);
  float *opart = (float *)ws;
  float2 *ml = (float2 *)((char *)ws + align256((size_t)a.T * S * kH * kDc * 4));
  if (a.kv_dtype == SGA_MXFP8_E4M3FN)
    hipLaunchKernelGGL(k_mla_split<true>, dim3(S, a.T), dim3(256), 0, s, a, opart, ml);
  else
    hipLaunchKernelGGL(k_mla_split<false>, dim3(S, a.T), dim3(256), 0, s, a, opart, ml);
  return hipGetLastError();
}

hipError_t launch_mla_combine(const MlaArgs &a, const void *ws, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int S = mla_splits(a.k);
  const float *opart = (const float *)ws;
  const float2 *ml = (const float2 *)((const char *)ws + align256((size_t)a.T * S * kH * kDc * 4));
  hipLaunchKernelGGL(k_mla_combine, dim3(kH, a.T), dim3(128), 0, s, a, opart, ml, S);
  return hipGetLastError();
}

}  // namespace sga
