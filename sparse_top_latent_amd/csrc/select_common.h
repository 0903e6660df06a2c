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

// Writes the nonzero bins of a 4096-bin LDS level-0 histogram as the list of
// slot `slot` of query t: the entry count, then entries (bin << 20 | count)
// in descending bin order. Needs blockDim.x == 256 (each thread scans 16
// consecutive bins) and a completed histogram (the caller synchronises).
// kPacked: two 16-bit bins per LDS word. A slot never holds more entries than
// the positions it covers, which bounds them by w.slot_words - 4.
template <bool kPacked>
__device__ __forceinline__ void write_hist0_list(const uint32_t *hist, const TopkWs &w, int t,
                                                 int slot, uint32_t *scratch) {
  const int tid = threadIdx.x;
  uint32_t c[16];
  if (kPacked) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t v = hist[tid * 8 + q];
      c[2 * q] = v & 0xFFFFu;
      c[2 * q + 1] = v >> 16;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = hist[tid * 16 + i];
  }
  uint32_t nz = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) nz += c[i] != 0u;
  uint32_t total;
  uint32_t asc = block_exclusive_scan(nz, scratch, &total);  // ascending rank of my first entry
  uint32_t *list = w.lists + (size_t)t * w.list_q_stride + (size_t)slot * w.slot_words;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (c[i]) list[1 + (total - 1 - asc++)] = ((uint32_t)(tid * 16 + i) << 20) | c[i];
  if (tid == 0) list[0] = total;
}

// Level-0 histogram of query t from the lists of its slots, added into a
// zeroed LDS histogram by kBlock threads; returns the threshold bin b0 (the
// bin holding the k-th largest key) and the count above it in *above.
// One 64-byte load per slot brings its count and its 15 highest bins. The
// result is exact once b0 is at or above the lowest bin read from every
// truncated list (all bins at or above it were then counted in full), which
// holds unless the k-th key lies deep in a slot's range; otherwise the rest
// of the truncated lists is read and b0 is found again.
template <int kBlock>
__device__ __forceinline__ int merge_lists_threshold(const TopkWs &ws, int t, int n, int k,
                                                     uint32_t *hist, int *floor_max,
                                                     uint32_t *scratch, int *res,
                                                     uint32_t *above) {
  const int tid = threadIdx.x;
  const int nslots = (n + ws.slot_keys - 1) / ws.slot_keys;  // slots that wrote a list
  const uint32_t *base = ws.lists + (size_t)t * ws.list_q_stride;
  if (tid == 0) *floor_max = -1;
  __syncthreads();
  int floor = -1;
  for (int sl = tid; sl < nslots; sl += kBlock) {
    const uint4 *p = (const uint4 *)(base + (size_t)sl * ws.slot_words);
    const uint4 q0 = p[0], q1 = p[1], q2 = p[2], q3 = p[3];
    const uint32_t wd[16] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w,
                             q2.x, q2.y, q2.z, q2.w, q3.x, q3.y, q3.z, q3.w};
    const uint32_t cnt = wd[0];
#pragma unroll
    for (int i = 1; i < 16; ++i)
      if ((uint32_t)i <= cnt) atomicAdd(&hist[wd[i] >> 20], wd[i] & 0xFFFFFu);
    if (cnt > 15u) floor = max(floor, (int)(wd[15] >> 20));
  }
  if (floor >= 0) atomicMax(floor_max, floor);
  __syncthreads();
  int b0 = find_threshold_bin<kHist0Bins>(hist, (uint32_t)k, above, scratch, res);
  if (b0 < *floor_max) {  // uniform: the head of some list was not enough
    for (int sl = tid; sl < nslots; sl += kBlock) {
      const uint32_t *l = base + (size_t)sl * ws.slot_words;
      const uint32_t cnt = l[0];
      for (uint32_t i = 16; i <= cnt; ++i) atomicAdd(&hist[l[i] >> 20], l[i] & 0xFFFFFu);
    }
    __syncthreads();
    b0 = find_threshold_bin<kHist0Bins>(hist, (uint32_t)k, above, scratch, res);
  }
  return b0;
}

}  // namespace sga
