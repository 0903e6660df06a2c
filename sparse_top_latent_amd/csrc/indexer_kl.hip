// Indexer KL loss restricted to the sparse selection, and its gradients (the
// training side of the indexer, "A.X K2 Technical Report" section 3.4: a KL
// loss pulls the indexer's ranking toward the attention weights, computed
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
//   k_kl_mass_lds   one workgroup per (64 selected rows, query), MI355X shapes
//   k_kl_mass_mx    with bf16 rows (_lds) or MXFP8 rows (_mx): the
//                   head-summed attention mass of each row, logits by bf16
//                   MFMA with the query slice in VGPRs (rows read from one
//                   LDS copy of the workgroup's 64 rows), and (FP8 index
//                   tensors) each row's indexer score and the workgroup's
//                   partials of the query's softmax normalisers;
//   k_kl_rows       one workgroup per (64 rows, query): each row's indexer score
//                   (and, for the other shapes, its attention mass, fp32 dot
//                   products from q in LDS);
//   k_kl_grad       one workgroup per (64 rows, query), 64 FP8 index heads x
//                   128 dims: the query's normalisers (from the mass
//                   workgroups' partials where the MFMA mass kernels ran) and
//                   loss, g, z again
//                   (bf16 MFMA) and both gradient products (bf16 MFMA on an
//                   exact three-part bf16 split of g w [z > 0]), d_kI added
//                   by fp32 atomics (plain stores for queries that own their
//                   rows), per-chunk partials of d_w and d_qI;
//   k_kl_loss,      the other shapes: one workgroup per query for the two
//   k_kl_backward   normalisations, the loss and g, then one per (64 rows,
//                   query) for z and the gradient products on the vector ALUs;
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
  float4 *part_n;              // [T, chunks]: a mass workgroup's (max score, sum exp(score - max), sum mass); or null
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
// or MXFP8 rows, Dc + Dr = 32 kKlKsteps): the workgroup's rows are copied once
// into LDS; wave w takes heads 16 w .. 16 w + 15 and all 64 rows, S^T = rows .
// q^T per 16-row tile (16x16x32 bf16 MFMA; the query slice stays in VGPRs as
// the B operand; MXFP8 rows are expanded exactly to bf16 as they are read).
//
// With kScores (64 FP8 index heads x 128 dims) the same workgroup also
// computes each row's indexer score: wave w takes rows 16 w .. 16 w + 15,
// z = kI . qI^T against the 4 tiles of 16 index heads by bf16 MFMA (E4M3FN
// values are exact in bf16, so z is the fp32 sum of exact products), then
// sum_h w_h ReLU(z) over the 64 heads.
constexpr int kKlKsteps = 18;

// 8 E4M3FN bytes -> 8 bf16 (exact), as a 16-byte MFMA operand
__device__ __forceinline__ v4i fp8x8_to_bf16(uint2 w8) {
  return (v4i){(int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w8.x, 1.0f, false)),
               (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w8.x, 1.0f, true)),
               (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w8.y, 1.0f, false)),
               (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w8.y, 1.0f, true))};
}

static_assert(kKlRows == 64, "the mass epilogue takes one row per lane of wave 0");
// Called by wave 0 (threads 0..63, one per row of the workgroup) with row
// tid's mass m and indexer score sc: stores both, and with scores the
// workgroup's partials of the query's normalisers, (max score, sum of exp(score
// - max), sum of mass) over its rows, which k_kl_grad combines.
template <bool kScores>
__device__ __forceinline__ void mass_epilogue(const KlArgs &a, int t, int r0, int tid, bool selected, float m, float sc) {
  const bool live = r0 + tid < a.k;
  const float mv = live && selected ? m : 0.0f;
  const float sv = live && selected ? sc + 0.0f : -INFINITY;
  if (live) {
    a.mass[(size_t)t * a.k + r0 + tid] = mv;
    if (kScores) a.score[(size_t)t * a.k + r0 + tid] = sv;
  }
  if (kScores && a.part_n) {
    float mx = sv;
    for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float se = sv > -INFINITY ? __expf(sv - mx) : 0.0f, sm = mv;
    for (int o = 1; o < 64; o <<= 1) {
      se += __shfl_xor(se, o);
      sm += __shfl_xor(sm, o);
    }
    if (tid == 0) a.part_n[(size_t)t * a.chunks + blockIdx.x] = make_float4(mx, se, sm, 0.0f);
  }
}

// bf16 latent rows: the workgroup's 64 rows are copied once into LDS
// (LDS-DMA) and every wave reads its MFMA operands from there, instead of
// each of the 4 waves loading every row from memory. Row r's 16-byte chunk c
// sits at chunk slot
// r * 72 + (c ^ kl_row_swz(r)): a row is 288 dwords, so every row starts on
// the same bank of a 128-byte bank window, and a 16-byte operand read of 16
// rows (one chunk each) is served 8 lanes at a time; r & 7 gives those 8
// rows 8 different chunk positions (by gfx950's bank-conflict counter, as
// for the MLA tiles).
constexpr int kKlRowChunks = 72;                         // 16-byte chunks per 576-wide bf16 row
constexpr size_t kKlLdsRows = (size_t)kKlRows * kKlRowChunks * 16;  // 73,728 B
__device__ __forceinline__ int kl_row_swz(int r) { return r & 7; }
__device__ __forceinline__ int kl_swz(int r, int c) { return r * kKlRowChunks + (c ^ kl_row_swz(r)); }

template <bool kScores>
__global__ __launch_bounds__(kKlThreads) void k_kl_mass_lds(KlArgs a) {
  constexpr int kRt = kKlRows / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char tile[];  // [64 rows][72 chunks]
  __shared__ float part[kKlThreads / 64][kKlRows];
  __shared__ float spart[kKlRows];
  __shared__ int64_t rows[kKlRows];
  typedef __attribute__((address_space(3))) void lds_void_t;
  const int t = blockIdx.y, r0 = blockIdx.x * kKlRows;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int head = wave * 16 + c16;
  // the selected positions and the sequence first, then the query-side
  // operands, which do not depend on the selection: their loads are in
  // flight while the cache rows are worked out and copied
  const int32_t pos = (tid < kKlRows && r0 + tid < a.k) ? a.topk_idx[(size_t)t * a.k + r0 + tid] : -1;
  int64_t start;
  const int n = query_candidates(a.meta, t, &start);
  const uint16_t *qh = (const uint16_t *)a.q + ((size_t)t * 64 + head) * a.D;
  v4i qreg[kKlKsteps];
#pragma unroll
  for (int ks = 0; ks < kKlKsteps; ++ks) qreg[ks] = *(const v4i *)(qh + ks * 32 + 8 * g);
  const float lse_h = a.lse[(size_t)t * 64 + head];
  // index scores: wave w takes rows 16 w .. 16 w + 15 against all 64 index
  // heads (B operands of the 4 head tiles), so each index key is loaded once
  v4i qireg[kScores ? 4 : 1][4];
  float w_hb[kScores ? 4 : 1];
  if (kScores) {
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const uint8_t *qih = (const uint8_t *)a.q_idx + ((size_t)t * 64 + hb * 16 + c16) * 128;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qireg[hb][ks] = fp8x8_to_bf16(*(const uint2 *)(qih + ks * 32 + 8 * g));
      w_hb[hb] = a.w[(size_t)t * 64 + hb * 16 + c16];
    }
  }
  if (tid < kKlRows) rows[tid] = (pos >= 0 && pos < n) ? kv_row(a.meta, a.meta.q_seq[t], start, pos) : -1;
  lds_barrier();  // rows[] ready; the query loads stay in flight
  // the copies: chunk slot c = u * 256 + tid holds row c / 72, chunk
  // (c % 72) ^ swizzle; unselected rows copy any 16 readable bytes (their
  // logits are never used)
#pragma unroll
  for (int u = 0; u < kKlRows * kKlRowChunks / 256; ++u) {
    const int c = u * 256 + tid;
    const int r = c / kKlRowChunks;
    const int col = (c - r * kKlRowChunks) ^ kl_row_swz(r);
    const int64_t row = rows[r];
    const void *src = row >= 0 ? (const void *)((const uint16_t *)a.kv + row * a.D + col * 8)
                               : (const void *)(a.q);  // any readable 16 bytes; masked below
    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)(tile + (u * 256 + wave * 64) * 16), 16, 0, 0);
  }
  // the index key of the lane's own row, requested together with the row
  // copies (unselected rows load nothing and give zeros)
  const int64_t krow = rows[wave * 16 + c16];
  uint2 kraw[4];
  if (kScores) {
    const uint8_t *kr = (const uint8_t *)a.k_idx + krow * 128 + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kraw[ks] = krow >= 0 ? *(const uint2 *)(kr + ks * 32) : make_uint2(0u, 0u);
  }
  __syncthreads();  // every copy has landed (the barrier waits for this wave's loads first)
  // the four 16-row tiles as four independent accumulation chains, k-step
  // by k-step (one chain per tile in turn left each MFMA waiting on the one
  // before it)
  v4f accs[kRt];
#pragma unroll
  for (int rt = 0; rt < kRt; ++rt) accs[rt] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < kKlKsteps; ++ks)
#pragma unroll
    for (int rt = 0; rt < kRt; ++rt) {
      const v4i av = *(const v4i *)(tile + kl_swz(rt * 16 + c16, 4 * ks + g) * 16);
      accs[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av),
                                                         __builtin_bit_cast(v8bf, qreg[ks]), accs[rt], 0, 0, 0);
    }
  v4f zcs[4];
  if (kScores) {
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) zcs[hb] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const v4i kb = krow < 0 ? (v4i){0, 0, 0, 0} : fp8x8_to_bf16(kraw[ks]);
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        zcs[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, kb),
                                                          __builtin_bit_cast(v8bf, qireg[hb][ks]), zcs[hb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int rt = 0; rt < kRt; ++rt) {
    const v4f acc = accs[rt];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = rt * 16 + 4 * g + i;
      float e = rows[j] >= 0 ? __expf(a.tau * acc[i] - lse_h) : 0.0f;
      e += __shfl_xor(e, 1);
      e += __shfl_xor(e, 2);
      e += __shfl_xor(e, 4);
      e += __shfl_xor(e, 8);
      if (c16 == 0) part[wave][j] = e;
    }
  }
  if (kScores) {
    // zcs[hb][i]: z of row 16 wave + 4 g + i for index head 16 hb + c16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float sc = 0.0f;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) sc = fmaf(fmaxf(zcs[hb][i], 0.0f), w_hb[hb], sc);
      sc += __shfl_xor(sc, 1);
      sc += __shfl_xor(sc, 2);
      sc += __shfl_xor(sc, 4);
      sc += __shfl_xor(sc, 8);
      if (c16 == 0) spart[wave * 16 + 4 * g + i] = sc;
    }
  }
  __syncthreads();
  if (tid < kKlRows) {  // wave 0
    float m = 0.0f;
#pragma unroll
    for (int w = 0; w < kKlThreads / 64; ++w) m += part[w][tid];
    mass_epilogue<kScores>(a, t, r0, tid, rows[tid] >= 0, m, kScores ? spart[tid] : 0.0f);
  }
}

// MXFP8 rows: the workgroup's 64 raw rows (576 E4M3FN bytes
// each, 36 chunks of 16 bytes) are copied once into LDS by LDS-DMA and their
// E8M0 scales staged beside them; every wave expands its operands from there
// (8 bytes and one scale per lane and k-step). Row r's chunk c sits at slot
// r * 36 + (c ^ ((r >> 1) & 3)): a row is 576 bytes, so a 128-byte bank
// window sees only two row phases; the XOR (which keeps c within its group of
// four, 36 being a multiple of 4) gives 8 neighbouring rows 8 different 16-byte
// positions.
constexpr int kKlMxChunks = 36;                                    // 16-byte chunks per 576-byte row
constexpr size_t kKlLdsMx = (size_t)kKlRows * kKlMxChunks * 16;    // 36,864 B
__device__ __forceinline__ int kl_mx_slot(int r, int c) { return r * kKlMxChunks + (c ^ ((r >> 1) & 3)); }

template <bool kScores>
__global__ __launch_bounds__(kKlThreads) void k_kl_mass_mx(KlArgs a) {
  constexpr int kRt = kKlRows / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char tile[];  // [64 rows][36 chunks]
  __shared__ float part[kKlThreads / 64][kKlRows];
  __shared__ float spart[kKlRows];
  __shared__ int64_t rows[kKlRows];
  __shared__ uint8_t scl[kKlRows * kKlKsteps];  // E8M0 scale of (row, k-step)
  typedef __attribute__((address_space(3))) void lds_void_t;
  const int t = blockIdx.y, r0 = blockIdx.x * kKlRows;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int head = wave * 16 + c16;
  // the selected positions and the sequence first, then the query-side
  // operands, which do not depend on the selection
  const int32_t pos = (tid < kKlRows && r0 + tid < a.k) ? a.topk_idx[(size_t)t * a.k + r0 + tid] : -1;
  int64_t start;
  const int n = query_candidates(a.meta, t, &start);
  const uint16_t *qh = (const uint16_t *)a.q + ((size_t)t * 64 + head) * a.D;
  v4i qreg[kKlKsteps];
#pragma unroll
  for (int ks = 0; ks < kKlKsteps; ++ks) qreg[ks] = *(const v4i *)(qh + ks * 32 + 8 * g);
  const float lse_h = a.lse[(size_t)t * 64 + head];
  v4i qireg[kScores ? 4 : 1][4];
  float w_hb[kScores ? 4 : 1];
  if (kScores) {
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const uint8_t *qih = (const uint8_t *)a.q_idx + ((size_t)t * 64 + hb * 16 + c16) * 128;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qireg[hb][ks] = fp8x8_to_bf16(*(const uint2 *)(qih + ks * 32 + 8 * g));
      w_hb[hb] = a.w[(size_t)t * 64 + hb * 16 + c16];
    }
  }
  if (tid < kKlRows) rows[tid] = (pos >= 0 && pos < n) ? kv_row(a.meta, a.meta.q_seq[t], start, pos) : -1;
  lds_barrier();  // rows[] ready; the query loads stay in flight
  // the row copies: slot c = u * 256 + tid holds row c / 36, chunk
  // (c % 36) ^ swizzle; unselected rows copy any 16 readable bytes (their
  // logits are never used)
#pragma unroll
  for (int u = 0; u < kKlRows * kKlMxChunks / 256; ++u) {
    const int c = u * 256 + tid;
    const int r = c / kKlMxChunks;
    const int col = (c - r * kKlMxChunks) ^ ((r >> 1) & 3);
    const int64_t row = rows[r];
    const void *src = row >= 0 ? (const void *)((const uint8_t *)a.kv + row * a.D + col * 16) : (const void *)(a.q);
    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)(tile + (u * 256 + wave * 64) * 16), 16, 0, 0);
  }
  // the scales (unselected rows: 2^0)
  uint8_t sv[(kKlRows * kKlKsteps + kKlThreads - 1) / kKlThreads];
#pragma unroll
  for (int u = 0; u < (kKlRows * kKlKsteps + kKlThreads - 1) / kKlThreads; ++u) {
    const int i = u * kKlThreads + tid;
    const int64_t row = i < kKlRows * kKlKsteps ? rows[i / kKlKsteps] : -1;
    sv[u] = row >= 0 ? a.kv_scale[row * kKlKsteps + i % kKlKsteps] : (uint8_t)127;
  }
  // the index key of the lane's own row (unselected rows load nothing)
  const int64_t krow = rows[wave * 16 + c16];
  uint2 kraw[4];
  if (kScores) {
    const uint8_t *kr = (const uint8_t *)a.k_idx + krow * 128 + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kraw[ks] = krow >= 0 ? *(const uint2 *)(kr + ks * 32) : make_uint2(0u, 0u);
  }
#pragma unroll
  for (int u = 0; u < (kKlRows * kKlKsteps + kKlThreads - 1) / kKlThreads; ++u) {
    const int i = u * kKlThreads + tid;
    if (i < kKlRows * kKlKsteps) scl[i] = sv[u];
  }
  __syncthreads();  // every copy has landed and the scales are staged
  v4f accs[kRt];
#pragma unroll
  for (int rt = 0; rt < kRt; ++rt) accs[rt] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < kKlKsteps; ++ks)
#pragma unroll
    for (int rt = 0; rt < kRt; ++rt) {
      const int r = rt * 16 + c16;
      const uint2 w8 = *(const uint2 *)(tile + kl_mx_slot(r, 2 * ks + (g >> 1)) * 16 + (g & 1) * 8);
      const float sc = e8m0_to_f32(scl[r * kKlKsteps + ks]);
      const v4i av = {(int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w8.x, sc, false)),
                      (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w8.x, sc, true)),
                      (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w8.y, sc, false)),
                      (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w8.y, sc, true))};
      accs[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av),
                                                         __builtin_bit_cast(v8bf, qreg[ks]), accs[rt], 0, 0, 0);
    }
#pragma unroll
  for (int rt = 0; rt < kRt; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = rt * 16 + 4 * g + i;
      float e = rows[j] >= 0 ? __expf(a.tau * accs[rt][i] - lse_h) : 0.0f;
      e += __shfl_xor(e, 1);
      e += __shfl_xor(e, 2);
      e += __shfl_xor(e, 4);
      e += __shfl_xor(e, 8);
      if (c16 == 0) part[wave][j] = e;
    }
  }
  if (kScores) {
    v4f zcs[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) zcs[hb] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const v4i kb = krow < 0 ? (v4i){0, 0, 0, 0} : fp8x8_to_bf16(kraw[ks]);
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        zcs[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, kb),
                                                          __builtin_bit_cast(v8bf, qireg[hb][ks]), zcs[hb], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float sc = 0.0f;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) sc = fmaf(fmaxf(zcs[hb][i], 0.0f), w_hb[hb], sc);
      sc += __shfl_xor(sc, 1);
      sc += __shfl_xor(sc, 2);
      sc += __shfl_xor(sc, 4);
      sc += __shfl_xor(sc, 8);
      if (c16 == 0) spart[wave * 16 + 4 * g + i] = sc;
    }
  }
  __syncthreads();
  if (tid < kKlRows) {  // wave 0
    float m = 0.0f;
#pragma unroll
    for (int w = 0; w < kKlThreads / 64; ++w) m += part[w][tid];
    mass_epilogue<kScores>(a, t, r0, tid, rows[tid] >= 0, m, kScores ? spart[tid] : 0.0f);
  }
}

// kLdsOnly: the barriers wait for LDS operations only (lds_barrier), so
// global loads the caller has in flight stay in flight
template <bool kLdsOnly = false>
__device__ __forceinline__ float block_sum(float v, float *red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if (kLdsOnly) lds_barrier(); else __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  if (kLdsOnly) lds_barrier(); else __syncthreads();
  float s = 0.0f;
  for (int i = 0; i < kKlThreads / 64; ++i) s += red[i];
  return s;
}

template <bool kLdsOnly = false>
__device__ __forceinline__ float block_max(float v, float *red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if (kLdsOnly) lds_barrier(); else __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  if (kLdsOnly) lds_barrier(); else __syncthreads();
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

// The backward for the shapes k_kl_grad does not take (fp32 tensors, other
// head counts): z, then both gradient products on the fp32 vector ALUs.
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
  __syncthreads();
  const size_t chunk = (size_t)t * a.chunks + blockIdx.x;
  for (int h = tid; h < a.HI; h += kKlThreads) {
    float s = 0.0f;
    for (int j = 0; j < kKlRows; ++j) s += rz[j * kGzLd + h];
    a.part_w[chunk * a.HI + h] = s;
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

// ---------------------------------------------------------------------------
// k_kl_grad: the loss and the whole backward of one (64 selected rows, query)
// workgroup for 64 FP8 index heads x 128 dims, in one kernel.
//
// Every workgroup of a query first reduces the query's scores and masses
// (2 x k floats, held in L2 after the mass kernel) to the two normalisers:
// log Z of the score softmax and the total mass; the first workgroup also
// adds up the loss. Each thread then has g for its own rows.
//
// The gradient products are bf16 MFMA 16x16x32 with an exact three-way split
// of the fp32 factor G[j,h] = g_j w_h [z_jh > 0] = G1 + G2 + G3 (each part the
// bf16 rounding of what the previous parts leave; the three carry 24
// significant bits, fp32's precision), while the other operand, the E4M3FN
// index keys or query, is exact in bf16. Every product is then exact and the
// MFMA accumulates in fp32, as an fp32 product would:
//   d_qI[h,d] = sum_j G[j,h] kI[j,d]   (A = G^T [h][j], B = kI^T [d][j])
//   d_kI[j,d] = sum_h G[j,h] qI[h,d]   (A = G   [j][h], B = qI^T [d][h])
// The two products run one after the other through the same two LDS arrays
// (the operand of each lane is 8 consecutive k values: one 16-byte read).
// ---------------------------------------------------------------------------
constexpr int kGradLd = 72;  // bf16 row stride of the operand arrays (36 dwords: 16 rows' 16-byte reads hit distinct banks)
constexpr int kGradMaxPer = 16;  // scores per thread for k <= 4096

__device__ __forceinline__ uint16_t bf16_bits_rn(float x) {
  // round to nearest even (the parts are finite; NaN never reaches here)
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// x = p[0] + p[1] + p[2] + (a remainder below 2^-24 |x|), each part a bf16
__device__ __forceinline__ void split3_bf16(float x, uint16_t (&p)[3]) {
  p[0] = bf16_bits_rn(x);
  const float r1 = x - bf16_bits_to_f32(p[0]);
  p[1] = bf16_bits_rn(r1);
  const float r2 = r1 - bf16_bits_to_f32(p[1]);
  p[2] = bf16_bits_rn(r2);
}

// kPartN: the normalisers come from the mass kernel's per-workgroup partials
// (a.part_n), and only the first workgroup of a query, which writes its loss,
// loads every score and mass; otherwise every workgroup reduces them all.
// kMinWg: workgroups per CU the registers must allow (3 for grids of more
// than two workgroups per CU: 168 VGPRs instead of 184, one spilled; 1 keeps
// every register for grids the CUs hold at once).
template <bool kPartN, int kMinWg>
__global__ __launch_bounds__(kKlThreads, kMinWg) void k_kl_grad(KlArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t opA[3][64 * kGradLd];  // G^T, then G (three parts)
  __shared__ __attribute__((aligned(16))) uint16_t opB[128 * kGradLd];    // kI^T, then qI^T
  __shared__ float red[kKlThreads / 64];
  __shared__ float rzw[kKlThreads / 64][64];  // d_w partials of the 4 waves
  __shared__ float gsh[kKlRows];
  __shared__ int64_t rows[kKlRows];
  __shared__ int s_shared_rows;
  const int t = blockIdx.y, r0 = blockIdx.x * kKlRows;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // May another query add into the cache rows this query selects? Not when
  // the caches are contiguous, no other query names this query's sequence,
  // and no other sequence's rows overlap its rows: then this query's
  // additions into d_k_idx need no atomics (its positions are distinct, so
  // each (row, d) is this workgroup's alone). Decided from the query and
  // sequence tables (up to 1,024 entries each; past that, and for paged
  // caches, whose pages sequences may share, the atomics stay). Every
  // workgroup of the query reaches the same decision.
  bool shared_rows = a.meta.page_shift != 0 || a.T > 1024 || a.meta.num_seqs > 1024;
  if (!shared_rows) {
    const int sb = a.meta.q_seq[t];
    int64_t s0;
    const int64_t l0 = seq_len_clipped(a.meta, sb, &s0);
    for (int u = tid; u < a.T; u += kKlThreads)
      if (u != t && a.meta.q_seq[u] == sb) shared_rows = true;
    for (int u = tid; u < a.meta.num_seqs; u += kKlThreads) {
      if (u == sb) continue;
      int64_t s1;
      const int64_t l1 = seq_len_clipped(a.meta, u, &s1);
      if (l0 > 0 && l1 > 0 && s1 < s0 + l0 && s0 < s1 + l1) shared_rows = true;
    }
  }
  if (tid == 0) s_shared_rows = 0;
  // everything that depends on nothing else is requested first: the index
  // query of all 64 heads (bf16 B operands of the 4 head tiles, exact) and
  // their weights, the query's scores and masses, and the selected positions
  v4i qireg[4][4];
  float w_hb[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const uint8_t *qih = (const uint8_t *)a.q_idx + ((size_t)t * 64 + hb * 16 + c16) * 128;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qireg[hb][ks] = fp8x8_to_bf16(*(const uint2 *)(qih + ks * 32 + 8 * g));
    w_hb[hb] = a.w[(size_t)t * 64 + hb * 16 + c16];
  }
  const float *sc = a.score + (size_t)t * a.k, *ms = a.mass + (size_t)t * a.k;
  const bool all_rows = !kPartN || blockIdx.x == 0;  // uniform over the workgroup
  float scv[kGradMaxPer], msv[kGradMaxPer];
#pragma unroll
  for (int i = 0; i < kGradMaxPer; ++i) {
    const int r = tid + i * kKlThreads;
    scv[i] = all_rows && r < a.k ? sc[r] : -INFINITY;
    msv[i] = all_rows && r < a.k ? ms[r] : 0.0f;
  }
  // kPartN: the chunks' partials (one per lane; a.chunks <= 64 here) and the
  // score and mass of row r0 + tid
  float4 pn = make_float4(-INFINITY, 0.0f, 0.0f, 0.0f);
  float own_s = -INFINITY, own_m = 0.0f;
  if (kPartN) {
    if (lane < a.chunks) pn = a.part_n[(size_t)t * a.chunks + lane];
    if (tid < kKlRows && r0 + tid < a.k) {
      own_s = sc[r0 + tid];
      own_m = ms[r0 + tid];
    }
  }
  int64_t start;
  const int n = query_candidates(a.meta, t, &start);
  if (tid < kKlRows) {
    const int r = r0 + tid;
    rows[tid] = r < a.k ? sel_row(a, t, r, n, start) : -1;
  }
  lds_barrier();  // rows[] ready (and s_shared_rows cleared); the loads above stay in flight
  if (shared_rows) s_shared_rows = 1;  // read after later barriers
  // the index key of the lane's z row (wave w takes rows 16 w .. 16 w + 15);
  // it stays in flight through the normalisers below (whose barriers wait
  // for LDS operations only)
  const int64_t krow = rows[wave * 16 + c16];  // -1: not selected (loads nothing)
  uint2 kraw[4];
  {
    const uint8_t *kr = (const uint8_t *)a.k_idx + krow * 128 + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kraw[ks] = krow >= 0 ? *(const uint2 *)(kr + ks * 32) : make_uint2(0u, 0u);
  }

  // the query's normalisers (as k_kl_loss computes them): with kPartN every
  // wave combines the chunks' partials itself (butterfly sums, so every lane
  // of every wave holds the same values), otherwise a block reduction
  float mx = -INFINITY, tot = 0.0f, zs = 0.0f;
  if (kPartN) {
    mx = pn.x;
    for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    zs = pn.x > -INFINITY ? pn.y * __expf(pn.x - mx) : 0.0f;
    tot = pn.z;
    for (int o = 1; o < 64; o <<= 1) {
      zs += __shfl_xor(zs, o);
      tot += __shfl_xor(tot, o);
    }
  } else {
#pragma unroll
    for (int i = 0; i < kGradMaxPer; ++i) {
      mx = fmaxf(mx, scv[i]);
      tot += msv[i];
    }
    mx = block_max<true>(mx, red);
    tot = block_sum<true>(tot, red);
    if (mx > -INFINITY)
#pragma unroll
      for (int i = 0; i < kGradMaxPer; ++i)
        if (tid + i * kKlThreads < a.k) zs += __expf(scv[i] - mx);
    zs = block_sum<true>(zs, red);
  }
  const float lz = mx + __logf(zs);
  if (blockIdx.x == 0) {  // uniform over the workgroup
    float loss = 0.0f;
#pragma unroll
    for (int i = 0; i < kGradMaxPer; ++i) {
      if (tid + i * kKlThreads < a.k && scv[i] > -INFINITY) {
        const float tg = tot > 0.0f ? msv[i] / tot : 0.0f;
        if (tg > 0.0f) loss += tg * (__logf(tg) - (scv[i] - lz));
      }
    }
    loss = block_sum<true>(loss, red);
    if (tid == 0) a.loss[t] = mx > -INFINITY ? loss : 0.0f;
  }
  // g of the workgroup's rows: row j's score and mass sit in thread
  // (r0 + j) % 256, entry (r0 + j) / 256 (kPartN: in thread j)
  if (kPartN) {
    if (tid < kKlRows)
      gsh[tid] = (r0 + tid < a.k && rows[tid] >= 0 && own_s > -INFINITY)
                     ? __expf(own_s - lz) - (tot > 0.0f ? own_m / tot : 0.0f)
                     : 0.0f;
  } else {
    const int owner = r0 % kKlThreads;  // r0 is a multiple of 64: rows j < 64 stay within one entry
    const int i0 = r0 / kKlThreads;
    if (tid >= owner && tid < owner + kKlRows) {
      const int j = tid - owner;
      float gv = 0.0f;
#pragma unroll
      for (int i = 0; i < kGradMaxPer; ++i)
        if (i == i0 && r0 + j < a.k && rows[j] >= 0 && scv[i] > -INFINITY)
          gv = __expf(scv[i] - lz) - (tot > 0.0f ? msv[i] / tot : 0.0f);
      gsh[j] = gv;
    }
  }
  lds_barrier();  // gsh[] ready

  // z = kI . qI^T of the wave's 16 rows against the 4 head tiles; the wave
  // also stores its rows' keys transposed (kI^T [d][j]) for d_qI
  v4f zc[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) zc[hb] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const v4i kb = krow < 0 ? (v4i){0, 0, 0, 0} : fp8x8_to_bf16(kraw[ks]);
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
      zc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, kb),
                                                       __builtin_bit_cast(v8bf, qireg[hb][ks]), zc[hb], 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      opB[(ks * 32 + 8 * g + e) * kGradLd + wave * 16 + c16] = (uint16_t)((uint32_t)kb[e >> 1] >> (16 * (e & 1)));
  }
  // G for rows 16 wave + 4 g + i and head 16 hb + c16, its parts into G^T
  // [h][j] (four consecutive j per 8-byte store), and d_w's partial sums
  float gval[4][4];
  float gj[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) gj[i] = gsh[wave * 16 + 4 * g + i];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    uint16_t pp[4][3];
    float rzs = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gval[hb][i] = zc[hb][i] > 0.0f ? gj[i] * w_hb[hb] : 0.0f;
      rzs += gj[i] * fmaxf(zc[hb][i], 0.0f);
      split3_bf16(gval[hb][i], pp[i]);
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const uint2 v = make_uint2((uint32_t)pp[0][p] | ((uint32_t)pp[1][p] << 16),
                                 (uint32_t)pp[2][p] | ((uint32_t)pp[3][p] << 16));
      *(uint2 *)&opA[p][(hb * 16 + c16) * kGradLd + wave * 16 + 4 * g] = v;
    }
    rzs += __shfl_xor(rzs, 16);
    rzs += __shfl_xor(rzs, 32);
    if (g == 0) rzw[wave][hb * 16 + c16] = rzs;
  }
  const size_t chunk = (size_t)t * a.chunks + blockIdx.x;
  __syncthreads();  // G^T, kI^T and the d_w partials complete
  if (tid < 64) a.part_w[chunk * 64 + tid] = (rzw[0][tid] + rzw[1][tid]) + (rzw[2][tid] + rzw[3][tid]);

  // d_qI: wave w takes heads 16 w .. 16 w + 15, all 128 d
  {
    const int head = wave * 16 + c16;
    v4f acc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v4i av[3];
#pragma unroll
      for (int p = 0; p < 3; ++p) av[p] = *(const v4i *)&opA[p][head * kGradLd + ks * 32 + 8 * g];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const v4i bv = *(const v4i *)&opB[(dt * 16 + c16) * kGradLd + ks * 32 + 8 * g];
#pragma unroll
        for (int p = 0; p < 3; ++p)
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av[p]),
                                                            __builtin_bit_cast(v8bf, bv), acc[dt], 0, 0, 0);
      }
    }
    // C[i = head 16 w + 4 g + r][j = d]
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        a.part_q[chunk * 64 * 128 + (size_t)(wave * 16 + 4 * g + r) * 128 + dt * 16 + c16] = acc[dt][r];
  }
  __syncthreads();  // every wave is done with G^T and kI^T

  // G [j][h] parts and qI^T [d][h] for d_kI (wave w stores head tile w of qI^T)
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t pp[3];
      split3_bf16(gval[hb][i], pp);
      const int j = wave * 16 + 4 * g + i;
#pragma unroll
      for (int p = 0; p < 3; ++p) opA[p][j * kGradLd + hb * 16 + c16] = pp[p];
    }
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
    if (hb == wave)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          opB[(ks * 32 + 8 * g + e) * kGradLd + hb * 16 + c16] =
              (uint16_t)((uint32_t)qireg[hb][ks][e >> 1] >> (16 * (e & 1)));
  __syncthreads();

  // d_kI: wave w takes rows 16 w .. 16 w + 15, all 128 d; added into the
  // caller's buffer
  {
    v4f acc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v4i av[3];
#pragma unroll
      for (int p = 0; p < 3; ++p) av[p] = *(const v4i *)&opA[p][(wave * 16 + c16) * kGradLd + ks * 32 + 8 * g];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const v4i bv = *(const v4i *)&opB[(dt * 16 + c16) * kGradLd + ks * 32 + 8 * g];
#pragma unroll
        for (int p = 0; p < 3; ++p)
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av[p]),
                                                            __builtin_bit_cast(v8bf, bv), acc[dt], 0, 0, 0);
      }
    }
    const bool atomic = s_shared_rows != 0;  // uniform over the workgroup
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = wave * 16 + 4 * g + r;
      const int64_t row = rows[j];
      if (row >= 0 && gsh[j] != 0.0f) {
        float *dk = a.d_k_idx + row * 128 + c16;
        if (atomic) {
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) atomicAdd(dk + dt * 16, acc[dt][r]);
        } else {
          float old[8];
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) old[dt] = dk[dt * 16];
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) dk[dt * 16] = old[dt] + acc[dt][r];
        }
      }
    }
  }
}

// d_q_idx and d_w: the partials summed over the chunks in a fixed order. A
// workgroup takes 64 float4 outputs of d_q_idx; its four thread groups each
// add a quarter of the chunks (eight loads in flight per thread), and the
// four sums are added in group order. The first workgroup of a query also
// sums d_w.
constexpr int kRedOut = 64;
constexpr int kRedGroups = kKlThreads / kRedOut;

__global__ __launch_bounds__(kKlThreads) void k_kl_reduce(KlArgs a) {
  __shared__ float4 part[kRedGroups][kRedOut];
  const int t = blockIdx.y, tid = threadIdx.x;
  const int nq4 = a.HI * a.DI / 4;  // HI * DI is a multiple of 8
  const int oo = tid % kRedOut, grp = tid / kRedOut;
  const int o = blockIdx.x * kRedOut + oo;
  const int per = (a.chunks + kRedGroups - 1) / kRedGroups;
  const int c0 = min(a.chunks, grp * per), c1 = min(a.chunks, c0 + per);
  float4 s = {0.f, 0.f, 0.f, 0.f};
  if (o < nq4) {
    const float4 *src = (const float4 *)a.part_q + (size_t)t * a.chunks * nq4 + o;
    int c = c0;
    for (; c + 8 <= c1; c += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = src[(size_t)(c + u) * nq4];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
      }
    }
    for (; c < c1; ++c) {
      const float4 v = src[(size_t)c * nq4];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
  }
  part[grp][oo] = s;
  __syncthreads();
  if (grp == 0 && o < nq4) {
#pragma unroll
    for (int q = 1; q < kRedGroups; ++q) {
      const float4 v = part[q][oo];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    ((float4 *)a.d_q_idx)[(size_t)t * nq4 + o] = s;
  }
  if (blockIdx.x == 0 && tid < a.HI) {
    const float *src = a.part_w + (size_t)t * a.chunks * a.HI + tid;
    float w = 0.0f;
    int c = 0;
    for (; c + 8 <= a.chunks; c += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = src[(size_t)(c + u) * a.HI];
#pragma unroll
      for (int u = 0; u < 8; ++u) w += v[u];
    }
    for (; c < a.chunks; ++c) w += src[(size_t)c * a.HI];
    a.d_w[(size_t)t * a.HI + tid] = w;
  }
}

}  // namespace

size_t indexer_kl_ws_bytes(int T, int k, int HI, int DI) {
  const size_t chunks = (k + kKlRows - 1) / kKlRows;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return 3 * al((size_t)T * k * 4) + al((size_t)T * chunks * HI * 4) + al((size_t)T * chunks * HI * DI * 4) +
         al((size_t)T * chunks * 16);
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
  a.part_q = (float *)c; c += al((size_t)T * a.chunks * HI * DI * 4);
  a.part_n = nullptr;
  size_t smem = indexer_kl_smem(H, D, HI, DI, q_dtype);
  // the MI355X shapes take the attention mass from the MFMA kernel
  const bool mfma = H == 64 && q_dtype == SGA_BF16 && D == 32 * kKlKsteps &&
                    (kv_dtype == SGA_BF16 || kv_dtype == SGA_MXFP8_E4M3FN);
  // one-time set-up (a function-local static is initialised exactly once,
  // also when several host threads arrive together)
  static const bool attr = [] {
    (void)hipFuncSetAttribute((const void *)k_kl_rows<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    (void)hipFuncSetAttribute((const void *)k_kl_rows<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    (void)hipFuncSetAttribute((const void *)k_kl_backward, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    (void)hipFuncSetAttribute((const void *)k_kl_mass_lds<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kKlLdsRows);
    (void)hipFuncSetAttribute((const void *)k_kl_mass_lds<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kKlLdsRows);
    (void)hipGetLastError();
    return true;
  }();
  (void)attr;
  const dim3 grid(a.chunks, T);
  const bool lds_rows = kv_dtype == SGA_BF16;  // bf16 rows are staged in LDS once per workgroup
  if (mfma && HI == 64 && DI == 128 && idx_dtype == SGA_FP8_E4M3FN) {
    a.part_n = (float4 *)c;  // the mass kernel's normaliser partials
    if (lds_rows)
      hipLaunchKernelGGL(k_kl_mass_lds<true>, grid, dim3(kKlThreads), kKlLdsRows, s, a);
    else
      hipLaunchKernelGGL(k_kl_mass_mx<true>, grid, dim3(kKlThreads), kKlLdsMx, s, a);
  } else if (mfma) {
    if (lds_rows)
      hipLaunchKernelGGL(k_kl_mass_lds<false>, grid, dim3(kKlThreads), kKlLdsRows, s, a);
    else
      hipLaunchKernelGGL(k_kl_mass_mx<false>, grid, dim3(kKlThreads), kKlLdsMx, s, a);
    hipLaunchKernelGGL(k_kl_rows<false>, grid, dim3(kKlThreads), ((size_t)HI * kl_ld(DI) + 64) * 4, s, a);
  } else {
    hipLaunchKernelGGL(k_kl_rows<true>, grid, dim3(kKlThreads), smem, s, a);
  }
  if (HI == 64 && DI == 128 && idx_dtype == SGA_FP8_E4M3FN && k <= kGradMaxPer * kKlThreads) {
    const bool many = (size_t)a.chunks * T > 2 * (size_t)device_cu_count();
    if (a.part_n && a.chunks <= 64) {
      if (many)
        hipLaunchKernelGGL((k_kl_grad<true, 3>), grid, dim3(kKlThreads), 0, s, a);
      else
        hipLaunchKernelGGL((k_kl_grad<true, 1>), grid, dim3(kKlThreads), 0, s, a);
    } else {
      if (many)
        hipLaunchKernelGGL((k_kl_grad<false, 3>), grid, dim3(kKlThreads), 0, s, a);
      else
        hipLaunchKernelGGL((k_kl_grad<false, 1>), grid, dim3(kKlThreads), 0, s, a);
    }
  } else {
    hipLaunchKernelGGL(k_kl_loss, dim3(T), dim3(kKlThreads), 0, s, a);
    hipLaunchKernelGGL(k_kl_backward, grid, dim3(kKlThreads), smem, s, a);
  }
  hipLaunchKernelGGL(k_kl_reduce, dim3((HI * DI / 4 + kRedOut - 1) / kRedOut, T), dim3(kKlThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace sga
