// Device helpers of the radix top-k select.
#pragma once

#include "kernels.h"

namespace sga {

// Finds the bin b holding the `want`-th largest element of an NB-bin LDS
// histogram: the count of elements in bins above b (returned in *above) is
// < want and adding bin b reaches want. Each of the kBlock threads reads
// NB / kBlock consecutive bins into registers; an exclusive scan in thread
// order is then a suffix scan over bins, and the thread whose range reaches
// `want` searches its own registers. Returns -1 when the histogram holds fewer
// than `want` elements. `scratch` needs kBlock / 64 words, `res` two ints.
template <int NB, int kBlock>
__device__ __forceinline__ int find_threshold_bin(const uint32_t *hist, uint32_t want,
                                                  uint32_t *above, uint32_t *scratch,
                                                  int *res) {
  constexpr int kPer = NB / kBlock;
  static_assert(kPer * kBlock == NB && (kPer % 4 == 0 || kPer < 4), "bins per thread");
  const int tid = threadIdx.x;
  const int lo_bin = NB - kPer * (tid + 1);  // this thread owns bins lo_bin .. lo_bin + kPer - 1
  uint32_t c[kPer];
  if constexpr (kPer % 4 == 0) {
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      const uint4 x = *(const uint4 *)(hist + lo_bin + 4 * q);
      c[4 * q] = x.x;
      c[4 * q + 1] = x.y;
      c[4 * q + 2] = x.z;
      c[4 * q + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPer; ++i) c[i] = hist[lo_bin + i];
  }
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) local += c[i];
  uint32_t total;
  const uint32_t excl = block_exclusive_scan(local, scratch, &total);
  if (excl < want && excl + local >= want) {
    // highest bin first
    uint32_t acc = excl;
    int bin = -1;
    uint32_t at = 0;
#pragma unroll
    for (int i = kPer - 1; i >= 0; --i) {
      if (bin < 0 && acc + c[i] >= want) {
        bin = lo_bin + i;
        at = acc;
      }
      acc += c[i];
    }
    res[0] = bin;
    res[1] = (int)at;
  }
  __syncthreads();
  if (total < want) {
    *above = total;
    return -1;
  }
  *above = (uint32_t)res[1];
  return res[0];
}

// The same search done by one full wave, with no barrier: lane l sums the
// NB / 64 bins below the top NB - (NB / 64) l; a wave prefix sum finds the
// lane whose range reaches `want`, and the lanes then take that range one bin
// each, highest first, to find the bin. Returns the same result for every lane.
template <int NB>
__device__ __forceinline__ int wave_find_threshold_bin(const uint32_t *hist, uint32_t want,
                                                       uint32_t *above) {
  constexpr int kPer = NB / 64;
  static_assert(kPer % 4 == 0 && kPer <= 64, "bins per lane");
  const int lane = threadIdx.x & 63;
  const int lo = NB - kPer * (lane + 1);
  uint32_t local = 0;
#pragma unroll
  for (int q = 0; q < kPer / 4; ++q) {
    const uint4 x = *(const uint4 *)(hist + lo + 4 * q);
    local += x.x + x.y + x.z + x.w;
  }
  const uint32_t inc = wave_inclusive_scan(local);
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
  if (total < want) {
    *above = total;
    return -1;
  }
  const uint32_t excl = inc - local;
  const int L = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)__ballot(excl < want && inc >= want)) - 1);
  const uint32_t ex_l = (uint32_t)__builtin_amdgcn_readlane((int)excl, L);
  const int top = NB - 1 - kPer * L;  // highest bin of lane L's range
  const uint32_t c = lane < kPer ? hist[top - lane] : 0u;
  const uint32_t s = wave_inclusive_scan(c);
  const int J = __builtin_amdgcn_readfirstlane(
      __ffsll((unsigned long long)__ballot(lane < kPer && ex_l + s >= want)) - 1);
  *above = ex_l + (uint32_t)__builtin_amdgcn_readlane((int)(s - c), J);
  return top - J;
}

// Level-0 threshold search of one wave over list heads held in registers:
// lane l < nl holds a head e[0..15] (entry count, then up to 15 entries
// bin << 20 | count in descending bin order). Same result as adding the heads
// into a 4096-bin histogram and calling wave_find_threshold_bin, in two
// passes over 64 bins each: first the 64 buckets of 64 bins (bin >> 6), then
// the 64 bins of the bucket that holds the `want`-th element. `h` is 128
// words of LDS used by this wave alone (its LDS operations take effect in
// order). Returns the same result for every lane.
__device__ __forceinline__ int wave_heads_threshold_bin(uint32_t *h, const uint32_t (&e)[16], int nl,
                                                        uint32_t want, uint32_t *above) {
  const int lane = threadIdx.x & 63;
  h[lane] = 0u;
  h[64 + lane] = 0u;
  if (lane < nl) {
#pragma unroll
    for (int i = 1; i < 16; ++i)
      if ((uint32_t)i <= e[0]) atomicAdd(&h[e[i] >> 26], e[i] & 0xFFFFFu);
  }
  // lane l takes bucket 63 - l: an inclusive scan over lanes is a suffix
  // scan over buckets
  const uint32_t cc = h[63 - lane];
  const uint32_t inc = wave_inclusive_scan(cc);
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
  if (total < want) {
    *above = total;
    return -1;
  }
  const int L = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)__ballot(inc >= want)) - 1);
  const uint32_t above_c = (uint32_t)__builtin_amdgcn_readlane((int)(inc - cc), L);
  const uint32_t bucket = 63u - (uint32_t)L;
  if (lane < nl) {
#pragma unroll
    for (int i = 1; i < 16; ++i)
      if ((uint32_t)i <= e[0] && (e[i] >> 26) == bucket) atomicAdd(&h[64 + ((e[i] >> 20) & 63u)], e[i] & 0xFFFFFu);
  }
  const uint32_t fc = h[64 + 63 - lane];
  const uint32_t finc = above_c + wave_inclusive_scan(fc);
  const int J = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)__ballot(finc >= want)) - 1);
  *above = (uint32_t)__builtin_amdgcn_readlane((int)(finc - fc), J);
  return (int)(bucket << 6) + 63 - J;
}

// Writes the nonzero bins of a 4096-bin LDS level-0 histogram as the list of
// slot `slot` of query t: the entry count, then entries (bin << 20 | count)
// in descending bin order. kBlock threads (blockDim.x) scan 4096 / kBlock
// consecutive bins each; the histogram must be complete (the caller
// synchronises). kPacked: two 16-bit bins per LDS word. A slot never holds
// more entries than the positions it covers, which bounds them by
// w.slot_words - 4.
template <bool kPacked, int kBlock>
__device__ __forceinline__ void write_hist0_list(const uint32_t *hist, const TopkWs &w, int t,
                                                 int slot, uint32_t *scratch) {
  constexpr int kPer = kHist0Bins / kBlock;
  static_assert(kPer * kBlock == kHist0Bins && kPer % 2 == 0, "bins per thread");
  const int tid = threadIdx.x;
  uint32_t c[kPer];
  if (kPacked) {
#pragma unroll
    for (int q = 0; q < kPer / 2; ++q) {
      const uint32_t v = hist[tid * (kPer / 2) + q];
      c[2 * q] = v & 0xFFFFu;
      c[2 * q + 1] = v >> 16;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPer; ++i) c[i] = hist[tid * kPer + i];
  }
  uint32_t nz = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) nz += c[i] != 0u;
  uint32_t total;
  uint32_t asc = block_exclusive_scan(nz, scratch, &total);  // ascending rank of my first entry
  uint32_t *list = w.lists + (size_t)t * w.list_q_stride + (size_t)slot * w.slot_words;
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (c[i]) list[1 + (total - 1 - asc++)] = ((uint32_t)(tid * kPer + i) << 20) | c[i];
  if (tid == 0) list[0] = total;
}

}  // namespace sga
