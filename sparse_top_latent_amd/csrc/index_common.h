// Device helpers shared by the FP8 indexer kernels (decode and prefill):
// the LDS key-tile layout, the FP8 MFMA, the weighted-ReLU epilogue and the
// cross-lane score reduction. See index_scores.hip for the arithmetic.
#pragma once

#include "common.h"
#include "kernels.h"

namespace sga {
namespace {

constexpr int kIdxTileKeys = 64;  // keys per LDS tile
constexpr int kIdxTileBytes = kIdxTileKeys * 128;

// Query rows are grouped in runs of kPfGroup for the prefill kernel.
constexpr int kPfGroup = 8;


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

// Piece swizzle of key row r in LDS: the 16-byte piece q of the row is
// stored at piece q ^ key_swz(r). A ds_read_b128 of the B operand reads 16
// consecutive rows with one piece each. The counters of gfx950
// (SQ_LDS_BANK_CONFLICT) fit a read served 8 lanes at a time over 128 bytes
// of banks: a 128-byte row starts on the same bank as every other row, so
// the 8 rows of each 8-lane group need 8 distinct piece positions, which any
// bijection of r & 7 gives. With (r >> 1) & 7 (distinct only over 16-lane
// groups against 256 bytes of banks) half of the LDS-active cycles of the
// prefill indexer were bank conflicts; with this swizzle there are none
// (the kernel time did not change: the pass is bound by its MFMA work).
__device__ __forceinline__ int key_swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

// B operand of key tile kt (keys 16 kt .. 16 kt + 15 of a 64-key LDS tile):
// key 16 kt + c16, bytes [32 kg, 32 kg + 32) of its 128-byte row.
__device__ __forceinline__ v8i load_key_operand(const unsigned char *tb, int kt, int kg, int c16) {
  const int r = kt * 16 + c16;
  const unsigned char *row = tb + r * 128;
  const v4i lo = *(const v4i *)(row + (((2 * kg) ^ key_swz(r)) << 4));
  const v4i hi = *(const v4i *)(row + (((2 * kg + 1) ^ key_swz(r)) << 4));
  return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// Weighted-ReLU head sums of kQ queries over one 64-key tile: part[j][kt]
// (lane l) is the sum, over the 16 heads this lane's accumulator rows cover,
// of w[h] * max(0, qI[h] . k) for query j and key 16 kt + l % 16.
//
// On gfx950 the epilogue (a max and an FMA per accumulator element) costs
// about as many cycles as the MFMA itself and overlaps with MFMA work only in
// part (counters: a VALU issue in about half of the MFMA-busy cycles), so it
// is kept as short as it can be; each sum is split over two accumulators so
// that consecutive FMAs do not wait on each other. The B operand is read
// per 16-key tile, which also bounds how many MFMA results are live at once.
// load_b(kt) returns the B operand of key tile kt.
template <int kQ, class LoadB>
__device__ __forceinline__ void score_tiles(const v8i (&a)[kQ][4], LoadB load_b,
                                            const float (&wv)[kQ][16], float (&part)[kQ][4]) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const v8i b = load_b(kt);
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

}  // namespace
}  // namespace sga
