// Cache append: new tokens' latent rows and index keys written into caller-
// chosen cache rows in the caches' storage formats (MXFP8 / bf16 / fp32 rows,
// FP8 E4M3FN / fp32 index keys).
//
// MXFP8 follows the OCP microscaling definition that the A.X K2 Technical
// Report's FP8 section trains with (E4M3 elements, one E8M0 scale per 32
// consecutive values): the block scale is 2^(floor(log2 max|v|) - 8), 8 being
// the exponent of E4M3's largest value 448, clamped to 2^-127 .. 2^127;
// elements are v / scale rounded to nearest even and saturated at 448; a
// block holding an inf or a NaN stores scale 0xFF and 0x7F elements.
//
// Work unit: one lane converts 8 consecutive values of one row (16 B of bf16
// or 32 B of fp32 in, 8 B of FP8 / 16 B of bf16 / 32 B of fp32 out), so a
// wave moves 512 consecutive values and every access is a full-width vector
// access. The four lanes of one 32-value block (a DPP quad) exchange their
// maxima with two quad permutes. Latent-row units come first in the grid,
// index-key units after them; an MXFP8 row is a multiple of 32 values, so a
// quad never straddles the two parts or two rows.

#include "kernels.h"

namespace sga {
namespace {

constexpr int kAppendBlock = 256;

struct F8 {
  float v[8];
};

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// the new rows are read once: non-temporal loads keep them out of the way
template <int kSrc>
__device__ __forceinline__ void load8(const void *base, int64_t elem, F8 &x, uint4 &raw) {
  if (kSrc == SGA_BF16) {
    const v4u r = __builtin_nontemporal_load((const v4u *)((const uint16_t *)base + elem));
    raw = make_uint4(r.x, r.y, r.z, r.w);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x.v[2 * k] = __uint_as_float(w[k] << 16);
      x.v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  } else {
    const v4f *p = (const v4f *)((const float *)base + elem);
    const v4f a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
    x.v[0] = a.x; x.v[1] = a.y; x.v[2] = a.z; x.v[3] = a.w;
    x.v[4] = b.x; x.v[5] = b.y; x.v[6] = b.z; x.v[7] = b.w;
  }
}

__device__ __forceinline__ void store_f32(void *base, int64_t elem, const F8 &x) {
  float4 *p = (float4 *)((float *)base + elem);
  p[0] = make_float4(x.v[0], x.v[1], x.v[2], x.v[3]);
  p[1] = make_float4(x.v[4], x.v[5], x.v[6], x.v[7]);
}

// fp32 -> bf16 bits, to nearest even; NaN -> the quiet NaN of its sign
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int kSrc>
__device__ __forceinline__ void store_bf16(void *base, int64_t elem, const F8 &x, const uint4 &raw) {
  uint4 o;
  if (kSrc == SGA_BF16) {
    o = raw;  // already bf16: a copy
  } else {
    o.x = bf16_rne(x.v[0]) | (bf16_rne(x.v[1]) << 16);
    o.y = bf16_rne(x.v[2]) | (bf16_rne(x.v[3]) << 16);
    o.z = bf16_rne(x.v[4]) | (bf16_rne(x.v[5]) << 16);
    o.w = bf16_rne(x.v[6]) | (bf16_rne(x.v[7]) << 16);
  }
  *(uint4 *)((uint16_t *)base + elem) = o;
}

// 8 values in E4M3 units -> 8 E4M3FN bytes. The hardware conversion rounds
// to nearest even; magnitudes past 448 are clamped first (E4M3FN has no
// infinity). With kNan, a NaN is written as 0x7F or 0xFF by its sign,
// whatever the conversion makes of it; without, the values are finite.
template <bool kNan>
__device__ __forceinline__ uint2 to_e4m3fn(const F8 &y) {
  float c[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    c[e] = kNan ? (fabsf(y.v[e]) > 448.0f ? copysignf(448.0f, y.v[e]) : y.v[e])
                : __builtin_amdgcn_fmed3f(y.v[e], -448.0f, 448.0f);
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], w1, true);
  uint32_t w[2] = {(uint32_t)w0, (uint32_t)w1};
  if (kNan) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (y.v[e] != y.v[e]) {
        const uint32_t code = (__float_as_uint(y.v[e]) >> 31) ? 0xffu : 0x7fu;
        const int sh = 8 * (e & 3);
        w[e >> 2] = (w[e >> 2] & ~(0xffu << sh)) | (code << sh);
      }
    }
  }
  return make_uint2(w[0], w[1]);
}

// Largest |value| bit pattern of the lane's 8 values, as an unsigned integer:
// for non-negative floats the integer order is the numeric order, and any inf
// or NaN compares above every finite value.
__device__ __forceinline__ uint32_t abs_bits_max(const F8 &x) {
  uint32_t m = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = max(m, __float_as_uint(x.v[e]) & 0x7fffffffu);
  return m;
}

// max over the DPP quad (4 consecutive lanes) holding one 32-value block
__device__ __forceinline__ uint32_t quad_max(uint32_t m) {
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xb1, 0xf, 0xf, false));  // quad_perm 1,0,3,2
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4e, 0xf, 0xf, false));  // quad_perm 2,3,0,1
  return m;
}

struct AppendArgs {
  const void *kv_new;     // [N, D]
  const void *kidx_new;   // [N, DI]
  const int64_t *slots;   // [N]
  void *kv;               // [rows, D]
  uint8_t *kv_scale;      // [rows, D / 32] (MXFP8)
  void *k_idx;            // [rows, DI]
  int64_t rows;
  uint32_t kv_units;      // N * D / 8
  uint32_t total_units;   // kv_units + N * DI / 8
  uint32_t row_units;     // D / 8
  uint32_t key_units;     // DI / 8
};

// One unit: 8 consecutive values of one token's latent row or index key.
struct Unit {
  F8 x;
  uint4 raw;
  int64_t slot;
  uint32_t tok, j;
  bool kv;
};

template <int kSrc>
__device__ __forceinline__ void unit_load(const AppendArgs &a, uint32_t u, Unit &w) {
  w.kv = u < a.kv_units;
  const uint32_t v = w.kv ? u : u - a.kv_units;
  const uint32_t per = w.kv ? a.row_units : a.key_units;
  w.tok = v / per;
  w.j = v - w.tok * per;
  const void *src = w.kv ? a.kv_new : a.kidx_new;
  // tok < N keeps the source load inside the new rows whatever the slot
  load8<kSrc>(src, (int64_t)w.tok * per * 8 + w.j * 8, w.x, w.raw);
  w.slot = a.slots[w.tok];
}

template <int kSrc, int kKv, int kIdx>
__device__ __forceinline__ void unit_store(const AppendArgs &a, const Unit &w) {
  // a dropped token drops its whole row, so the quad of an MXFP8 block stays together
  if (w.slot < 0 || w.slot >= a.rows) return;
  if (w.kv) {
    const int64_t dst = w.slot * a.row_units * 8 + w.j * 8;
    if (kKv == SGA_F32) {
      store_f32(a.kv, dst, w.x);
    } else if (kKv == SGA_BF16) {
      store_bf16<kSrc>(a.kv, dst, w.x, w.raw);
    } else {
      const uint32_t ef = quad_max(abs_bits_max(w.x)) >> 23;  // biased exponent of the block max
      uint2 codes;
      uint32_t sbyte;
      if (ef == 255u) {  // inf or NaN in the block
        sbyte = 0xffu;
        codes = make_uint2(0x7f7f7f7fu, 0x7f7f7f7fu);
      } else {
        // E8M0 byte = max(floor(log2 max) - 8, -127) + 127; a zero or
        // subnormal maximum (ef = 0) lands on the smallest scale
        sbyte = ef > 8u ? ef - 8u : 0u;
        const float inv = __uint_as_float((254u - sbyte) << 23);  // 2^-(sbyte - 127), exact
        F8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) y.v[e] = w.x.v[e] * inv;
        codes = to_e4m3fn<false>(y);
      }
      *(uint2 *)((uint8_t *)a.kv + dst) = codes;
      if ((w.j & 3u) == 0u) a.kv_scale[w.slot * (int64_t)(a.row_units / 4) + w.j / 4] = (uint8_t)sbyte;
    }
  } else {
    const int64_t dst = w.slot * a.key_units * 8 + w.j * 8;
    if (kIdx == SGA_F32)
      store_f32(a.k_idx, dst, w.x);
    else
      *(uint2 *)((uint8_t *)a.k_idx + dst) = to_e4m3fn<true>(w.x);
  }
}

// Each thread takes kAppendUnits units, kAppendBlock apart, and issues all of
// their loads before converting any: more bytes in flight per wave.
constexpr int kAppendUnits = 2;

template <int kSrc, int kKv, int kIdx>
__global__ __launch_bounds__(kAppendBlock) void k_cache_append(AppendArgs a) {
  const uint32_t base = blockIdx.x * (kAppendBlock * kAppendUnits) + threadIdx.x;
  Unit w[kAppendUnits];
#pragma unroll
  for (int r = 0; r < kAppendUnits; ++r) {
    const uint32_t u = base + r * kAppendBlock;
    if (u < a.total_units) unit_load<kSrc>(a, u, w[r]);
  }
#pragma unroll
  for (int r = 0; r < kAppendUnits; ++r) {
    const uint32_t u = base + r * kAppendBlock;
    if (u < a.total_units) unit_store<kSrc, kKv, kIdx>(a, w[r]);
  }
}

template <int kSrc, int kKv, int kIdx>
hipError_t launch3(const AppendArgs &a, hipStream_t s) {
  const uint32_t per_block = kAppendBlock * kAppendUnits;
  const uint32_t blocks = (a.total_units + per_block - 1) / per_block;
  hipLaunchKernelGGL((k_cache_append<kSrc, kKv, kIdx>), dim3(blocks), dim3(kAppendBlock), 0, s, a);
  return hipGetLastError();
}

template <int kSrc, int kKv>
hipError_t launch2(const AppendArgs &a, int idx_dtype, hipStream_t s) {
  return idx_dtype == SGA_F32 ? launch3<kSrc, kKv, SGA_F32>(a, s)
                              : launch3<kSrc, kKv, SGA_FP8_E4M3FN>(a, s);
}

template <int kSrc>
hipError_t launch1(const AppendArgs &a, int kv_dtype, int idx_dtype, hipStream_t s) {
  switch (kv_dtype) {
    case SGA_F32: return launch2<kSrc, SGA_F32>(a, idx_dtype, s);
    case SGA_BF16: return launch2<kSrc, SGA_BF16>(a, idx_dtype, s);
    default: return launch2<kSrc, SGA_MXFP8_E4M3FN>(a, idx_dtype, s);
  }
}

}  // namespace

hipError_t launch_cache_append(int64_t N, int D, int DI, int src_dtype, const void *kv_new,
                               const void *kidx_new, const int64_t *slots, int64_t rows,
                               int kv_dtype, void *kv, uint8_t *kv_scale, int idx_dtype,
                               void *k_idx, hipStream_t s) {
  AppendArgs a;
  a.kv_new = kv_new;
  a.kidx_new = kidx_new;
  a.slots = slots;
  a.kv = kv;
  a.kv_scale = kv_scale;
  a.k_idx = k_idx;
  a.rows = rows;
  a.row_units = (uint32_t)(D / 8);
  a.key_units = (uint32_t)(DI / 8);
  a.kv_units = kv_new ? (uint32_t)(N * (D / 8)) : 0u;
  a.total_units = a.kv_units + (kidx_new ? (uint32_t)(N * (DI / 8)) : 0u);
  if (a.total_units == 0) return hipSuccess;
  if (a.row_units == 0) a.row_units = 1;  // unused when kv_units is 0
  if (a.key_units == 0) a.key_units = 1;
  return src_dtype == SGA_F32 ? launch1<SGA_F32>(a, kv_dtype, idx_dtype, s)
                              : launch1<SGA_BF16>(a, kv_dtype, idx_dtype, s);
}

}  // namespace sga
