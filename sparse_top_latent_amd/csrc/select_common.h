// Device helpers of the radix top-k select.
#pragma once

#include "kernels.h"

namespace sga {

// Finds the bin b holding the `want`-th largest element of a histogram: the
// count of elements in bins above b (returned in *above) is < want and adding
// bin b reaches want. Each of blockDim threads owns NB/blockDim consecutive
// bins; the exclusive scan in thread order is then a suffix scan over bins.
// Returns -1 when the histogram holds fewer than `want` elements.
template <int NB>
__device__ __forceinline__ int find_threshold_bin(const uint32_t *hist, uint32_t want,
                                                  uint32_t *above, uint32_t *scratch,
                                                  int *res) {
  const int per = NB / (int)blockDim.x;
  const int tid = threadIdx.x;
  const int hi_bin = NB - 1 - tid * per;
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) local += hist[hi_bin - i];
  uint32_t total;
  uint32_t excl = block_exclusive_scan(local, scratch, &total);
  if (tid == 0) {
    res[0] = -1;
    res[1] = 0;
  }
  __syncthreads();
  if (excl < want && excl + local >= want) {
    uint32_t acc = excl;
    for (int i = 0; i < per; ++i) {
      uint32_t c = hist[hi_bin - i];
      if (acc + c >= want) {
        res[0] = hi_bin - i;
        res[1] = (int)acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
  int b = res[0];
  *above = (uint32_t)res[1];
  __syncthreads();
  return b;
}

// Level-0 threshold of query t from its completed histogram (written by an
// earlier kernel); stored to w.thr[t] as (b0, count above b0). Needs
// blockDim.x == 256: every thread loads its 16 consecutive bins with four
// 16-byte loads and keeps them in registers.
__device__ __forceinline__ void publish_threshold0(const TopkWs &w, int t, int k,
                                                   uint32_t *scratch, int *res) {
  constexpr int kPer = kHist0Bins / 256;
  const int tid = threadIdx.x;
  const int lo_bin = kHist0Bins - (tid + 1) * kPer;  // thread owns [lo_bin, lo_bin + 16)
  const uint4 *g = (const uint4 *)(w.hist0 + (size_t)t * kHist0Bins + lo_bin);
  uint32_t h[kPer];
#pragma unroll
  for (int q = 0; q < kPer / 4; ++q) {
    const uint4 v = g[q];
    h[4 * q] = v.x;
    h[4 * q + 1] = v.y;
    h[4 * q + 2] = v.z;
    h[4 * q + 3] = v.w;
  }
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) local += h[i];
  uint32_t total;
  const uint32_t excl = block_exclusive_scan(local, scratch, &total);  // counts above my bins
  const uint32_t want = (uint32_t)k;
  if (excl < want && excl + local >= want) {
    uint32_t acc = excl;
#pragma unroll
    for (int i = kPer - 1; i >= 0; --i) {  // highest bin first
      if (acc + h[i] >= want) {
        w.thr[t] = make_uint2((uint32_t)(lo_bin + i), acc);
        break;
      }
      acc += h[i];
    }
  }
  (void)res;
}

}  // namespace sga
