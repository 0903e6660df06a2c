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
// into a 4096-bin histogram and calling wave_find_threshold_bin: the bin b
// such that the heads hold fewer than `want` keys above b and at least `want`
// at or above it (*above: the keys above b), or -1 with *above the heads'
// total when they hold fewer than `want`. The count of keys at or above a bin
// never increases with the bin, so a binary search over the range of bins the
// heads hold finds b; each probe is a per-lane sum over its entries and one
// wave sum, all in registers (no LDS, so no same-address conflicts, which the
// top bins shared by all slots would cause). Returns the same result for
// every lane.
__device__ __forceinline__ int wave_heads_threshold_bin(const uint32_t (&e)[16], int nl, uint32_t want,
                                                        uint32_t *above) {
  const int lane = threadIdx.x & 63;
  uint32_t bins[15], cnts[15];
  const uint32_t ne = lane < nl ? min(e[0], 15u) : 0u;
#pragma unroll
  for (int i = 0; i < 15; ++i) {
    const bool ok = (uint32_t)i < ne;
    bins[i] = e[i + 1] >> 20;
    cnts[i] = ok ? (e[i + 1] & 0xFFFFFu) : 0u;
  }
  // keys of the heads at or above bin x (the same value in every lane)
  auto count_ge = [&](int x) {
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 15; ++i) c += bins[i] >= (uint32_t)x ? cnts[i] : 0u;
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan(c), 63);
  };
  // the range of bins held: [lo, hi]
  int hi = ne ? (int)bins[0] : -1, lo = ne ? (int)bins[ne - 1] : 4096;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    hi = max(hi, __shfl_xor(hi, d, 64));
    lo = min(lo, __shfl_xor(lo, d, 64));
  }
  const uint32_t total = count_ge(0);
  if (total < want) {
    *above = total;
    return -1;
  }
  // the largest x in [lo, hi] with count_ge(x) >= want (count_ge(lo) = total)
  lo = __builtin_amdgcn_readfirstlane(lo);
  hi = __builtin_amdgcn_readfirstlane(hi);
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (count_ge(mid) >= want) lo = mid; else hi = mid - 1;
  }
  *above = count_ge(lo + 1);
  return lo;
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

// Candidates of the top-k finish (below) for a workgroup of kBlock threads:
// round r holds candidates [r * kRound, r * kRound + kRound) of the query,
// thread tid the kPer consecutive ones from r * kRound + kPer tid. Reads past
// the end are clamped into the array and not used.
template <int kBlock>
struct FinishInput {
  static constexpr int kPer = 4096 / kBlock;  // candidates per thread and round
  static constexpr int kRound = kBlock * kPer;
  static_assert(kPer % 2 == 0, "candidate pairs");
  uint2 c[kPer];  // round 0, kept in registers
  uint4 th;       // the query's totals from k_topk_select
};

template <int kBlock>
__device__ __forceinline__ void finish_load_round(const TopkWs &ws, int t, int r,
                                                  uint2 (&pr)[FinishInput<kBlock>::kPer]) {
  constexpr int kPer = FinishInput<kBlock>::kPer;
  const uint2 *cand = ws.entries + (size_t)t * ws.nchunk * kTopkChunk;
  const uint32_t cap = (uint32_t)ws.nchunk * kTopkChunk;
  const uint32_t f0 = (uint32_t)r * FinishInput<kBlock>::kRound + threadIdx.x * kPer;
#pragma unroll
  for (int i = 0; i < kPer; i += 2) {
    const uint32_t f = min(f0 + i, cap - 2);
    const uint4 x = *(const uint4 *)(cand + f);
    pr[i] = make_uint2(x.x, x.y);
    pr[i + 1] = make_uint2(x.z, x.w);
  }
}

// Requests the finish's first round of candidates and the query's totals. It
// depends on nothing else, so a caller can issue it first and overlap its
// latency with other lookups (the data is only used for queries with n_t > k).
template <int kBlock>
__device__ __forceinline__ void finish_request(const TopkWs &ws, int t, FinishInput<kBlock> &in) {
  finish_load_round<kBlock>(ws, t, 0, in.c);
  in.th = ws.thr[t];
}

// The last step of the top-k select for query t, done by one workgroup of
// kBlock threads: from the candidates k_topk_select wrote (position order) and
// its totals (b0, keys above bin b0, candidates), the level-1 and level-2
// histograms give the exact k-th key K* and the number of ties at K* to take;
// then, round by round in position order, one packed scan gives every
// selected candidate its output index. `out(o, pos)` is called once for each
// o in [0, k) (in no particular order across threads). `in` comes from
// finish_request. LDS: `hist` holds 2 * 1024 words, `scratch` kBlock / 64,
// `res` 2. Every thread of the workgroup must call it (it has barriers, which
// wait for LDS operations only, so loads the caller has in flight stay in
// flight). Only for queries with n_t > k.
template <int kBlock, class Out>
__device__ __forceinline__ void finish_query(int k, const TopkWs &ws, int t, FinishInput<kBlock> &in,
                                             uint32_t *hist, uint32_t *scratch, int *res, Out out) {
  constexpr int kPer = FinishInput<kBlock>::kPer;
  constexpr int kRound = FinishInput<kBlock>::kRound;
  const int tid = threadIdx.x;
  const uint32_t cap = (uint32_t)ws.nchunk * kTopkChunk;
  auto load_round = [&](int r, uint2 (&pr)[kPer]) { finish_load_round<kBlock>(ws, t, r, pr); };
  uint2 (&p0r)[kPer] = in.c;
  const uint4 th = in.th;
  const uint32_t ub0 = th.x, above0 = th.y;
  const uint32_t total = min(th.z, cap);
  for (int i = tid; i < 2 * kHist12Bins; i += kBlock) hist[i] = 0u;
  lds_barrier();
  const int rounds = (int)((total + kRound - 1) / kRound);
  auto valid = [&](int r, int i) { return (uint32_t)r * kRound + tid * kPer + i < total; };
  uint32_t *hist1 = hist, *hist2 = hist + kHist12Bins;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // Keep the candidates in the registers they were loaded into: without this
  // the compiler may load them again for each pass.
  auto pin = [&](uint2 (&pr)[kPer]) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) asm volatile("" : "+v"(pr[i].x), "+v"(pr[i].y));
  };
  // threshold bin of a level histogram, found by wave 0 and shared
  auto find_bin = [&](const uint32_t *h, uint32_t want, uint32_t *above) {
    if (wave == 0) {
      uint32_t a;
      const int b = wave_find_threshold_bin<kHist12Bins>(h, want, &a);
      if (lane == 0) {
        res[0] = b;
        res[1] = (int)a;
      }
    }
    lds_barrier();
    *above = (uint32_t)res[1];
    return res[0];
  };
  pin(p0r);
  // level 1: key bits 19..10 of the keys in bin b0
  auto level1 = [&](int r, const uint2 (&pr)[kPer]) {
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (valid(r, i) && (pr[i].y >> kHist0Shift) == ub0) atomicAdd(&hist1[(pr[i].y >> 10) & 1023u], 1u);
  };
  level1(0, p0r);
  for (int r = 1; r < rounds; ++r) {
    uint2 pr[kPer];
    load_round(r, pr);
    pin(pr);
    level1(r, pr);
  }
  lds_barrier();
  uint32_t want = (uint32_t)k - above0;
  uint32_t above1;
  const int b1 = find_bin(hist1, want, &above1);
  want -= above1;
  const uint32_t prefix22 = (ub0 << 10) | (uint32_t)b1;  // key bits 31..10 of K*
  // level 2: the last 10 bits among the keys that share the top 22 bits
  auto level2 = [&](int r, const uint2 (&pr)[kPer]) {
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (valid(r, i) && (pr[i].y >> 10) == prefix22) atomicAdd(&hist2[pr[i].y & 1023u], 1u);
  };
  level2(0, p0r);
  for (int r = 1; r < rounds; ++r) {
    uint2 pr[kPer];
    load_round(r, pr);
    pin(pr);
    level2(r, pr);
  }
  lds_barrier();
  uint32_t above2;
  const int b2 = find_bin(hist2, want, &above2);
  want -= above2;
  const uint32_t kstar = (prefix22 << 10) | (uint32_t)b2;  // the exact k-th largest key
  const uint32_t take = want;                                 // ties at kstar to keep

  // ordered emission, round by round: one scan gives, per thread, the keys
  // above K* and the ties at K* in front of its run (16 bits each: a round
  // holds at most 4096 candidates)
  uint32_t gt_run = 0, tie_run = 0;
  auto emit = [&](int r, const uint2 (&pr)[kPer]) {
    uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const bool ok = valid(r, i);
      n_gt += ok && pr[i].y > kstar;
      n_eq += ok && pr[i].y == kstar;
    }
    uint32_t tot;
    const uint32_t pre = block_exclusive_scan<true>((n_eq << 16) | n_gt, scratch, &tot);
    uint32_t tr = tie_run + (pre >> 16);                      // ties in front of this run
    uint32_t o2 = gt_run + (pre & 0xFFFFu) + min(tr, take);   // outputs in front of it
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (!valid(r, i)) continue;
      bool sel = pr[i].y > kstar;
      if (pr[i].y == kstar) {
        sel = tr < take;
        ++tr;
      }
      if (sel) {
        if (o2 < (uint32_t)k) out(o2, (int32_t)pr[i].x);
        ++o2;
      }
    }
    gt_run += tot & 0xFFFFu;
    tie_run += tot >> 16;
  };
  emit(0, p0r);
  for (int r = 1; r < rounds; ++r) {
    uint2 pr[kPer];
    load_round(r, pr);
    pin(pr);
    emit(r, pr);
  }
}

}  // namespace sga
