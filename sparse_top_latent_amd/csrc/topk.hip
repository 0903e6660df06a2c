// Per-query top-k select: the k positions of largest score, ties to the lowest
// position, returned in ascending position order (-1 padding when n_t < k).
//
// Source: "A.X-K2: a sparse-attention upgrade that costs nothing, trained
// natively in FP8", section "Sparse Gated Attention" (2,048 single positions
// survive per query, chosen one by one rather than in blocks); "A.X K2
// Technical Report", section 3.4 (the indexer's selection size).
//
// Exact radix select on the order-preserving 32-bit key of each fp32 score,
// most significant digit first (12 + 10 + 10 bits):
//  1. level-0 histogram of key bits 31..20, as one list of nonzero bins per
//     producer workgroup ("slot", written by the indexer in the fused layer,
//     or by k_topk_hist0): no global atomics and nothing cleared beforehand.
//     The producer also records the query's candidate count n_t.
//  2. k_topk_select, one workgroup per (slot, query):
//     a. merges the heads of the query's lists into the level-0 histogram and
//        finds the threshold bin b0 (the bin holding the k-th largest key);
//        every workgroup of a query reaches the same result;
//     b. the same heads give each slot's number of keys with digit >= b0, so
//        the workgroup knows where its candidates go in position order: it
//        writes its (position, key) pairs with digit >= b0 straight to their
//        final place in the query's candidate array.
//  3. k_topk_finish, one workgroup per query, holds the candidates (at most a
//     few thousand for k = 2048) in registers: the level-1 histogram (key bits
//     19..10) of bin b0 and then the level-2 histogram of the pairs sharing the
//     top 22 bits of the threshold give the exact k-th key K* and how many ties
//     at K* to take; an ordered pass emits key > K* plus the first `take` ties,
//     which are the lowest positions because the candidates are in position
//     order.
// No atomics decide the output, so it is deterministic.

#include "kernels.h"
#include "select_common.h"

namespace sga {

namespace {

constexpr int kSelBlock = 256;
constexpr int kSelWaves = kSelBlock / 64;
constexpr int kSelPer = 4096 / kSelBlock;          // consecutive scores per thread and batch
constexpr int kSelBatch = kSelBlock * kSelPer;     // 4096 positions
constexpr int kFinBlock = 1024;                    // threads of the finishing workgroup

__global__ __launch_bounds__(256) void k_topk_hist0(SeqMeta m, const float *__restrict__ scores,
                                                    int64_t stride, TopkWs ws) {
  __shared__ uint32_t hist[kHist0Bins];
  __shared__ uint32_t scratch[256 / 64];
  const int t = blockIdx.y;
  int64_t start;
  const int n = query_candidates(m, t, &start);
  if (blockIdx.x == 0 && threadIdx.x == 0) ws.ncand[t] = make_int2(n, (int32_t)start);
  const int c0 = blockIdx.x * kTopkChunk;
  if (c0 >= n) return;
  // all of this thread's scores are requested before the histogram is
  // cleared (clamped into the row; positions past n are not counted), so the
  // loads overlap each other and the clearing instead of waiting one by one
  constexpr int kPer = kTopkChunk / 256;
  const float *row = scores + t * stride;
  float v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) v[j] = row[min(c0 + j * 256 + (int)threadIdx.x, n - 1)];
  for (int i = threadIdx.x; i < kHist0Bins; i += 256) hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (c0 + j * 256 + (int)threadIdx.x < n) atomicAdd(&hist[score_key(v[j]) >> kHist0Shift], 1u);
  __syncthreads();
  write_hist0_list<false, 256>(hist, ws, t, blockIdx.x, scratch);
}

// kSelPer consecutive scores from position p on; positions at or past the end
// of the row read its last element (their values are never used).
template <bool kVec>
__device__ __forceinline__ void load_scores(const float *row, int64_t stride, int64_t p, float (&v)[kSelPer]) {
  if (kVec) {
    // stride % 4 == 0 and p % 4 == 0: a float4 either lies inside the row or
    // starts at or past its end
#pragma unroll
    for (int q = 0; q < kSelPer / 4; ++q) {
      const int64_t a = p + 4 * q;
      const float4 x = *(const float4 *)(row + (a < stride - 4 ? a : stride - 4));
      v[4 * q] = x.x;
      v[4 * q + 1] = x.y;
      v[4 * q + 2] = x.z;
      v[4 * q + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) v[j] = row[p + j < stride ? p + j : stride - 1];
  }
}

// Sum of the counts of the list entries with bin >= b0 among the first `cnt`
// entries of a list (entries in descending bin order).
__device__ __forceinline__ uint32_t head_count_ge(const uint32_t (&wd)[16], uint32_t b0) {
  const uint32_t cnt = wd[0];
  uint32_t c = 0;
#pragma unroll
  for (int i = 1; i < 16; ++i)
    if ((uint32_t)i <= cnt && (wd[i] >> 20) >= b0) c += wd[i] & 0xFFFFFu;
  return c;
}

__device__ __forceinline__ uint32_t list_count_ge(const uint32_t *l, uint32_t b0) {
  const uint32_t cnt = l[0];
  uint32_t c = 0;
  for (uint32_t i = 1; i <= cnt; ++i) {
    const uint32_t e = l[i];
    if ((e >> 20) < b0) break;
    c += e & 0xFFFFFu;
  }
  return c;
}

template <bool kVec>
__global__ __launch_bounds__(kSelBlock) void k_topk_select(SeqMeta m, int k,
                                                           const float *__restrict__ scores,
                                                           int64_t stride, TopkWs ws,
                                                           int32_t *__restrict__ topk_idx) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[kHist0Bins];  // level 0; levels 1 and 2 in the last workgroup
  __shared__ uint32_t scratch[kSelWaves];
  __shared__ int res[2];
  __shared__ int floor_max;
  __shared__ uint32_t s_base;
  __shared__ uint32_t s_misc[2];
  const int tid = threadIdx.x;
  const int t = blockIdx.y, slot = blockIdx.x;
  const int skeys = ws.slot_keys;
  const int max_slots = gridDim.x;
  const float *row = scores + (int64_t)t * stride;
  const uint32_t *lbase = ws.lists + (size_t)t * ws.list_q_stride;
  const int64_t c0 = (int64_t)slot * skeys;
  if (m.max_kv_len <= k) {
    // every query keeps all its candidates (no lists were needed)
    int64_t start;
    const int n = query_candidates(m, t, &start);
    if (slot == 0)
      for (int i = tid; i < k; i += kSelBlock) topk_idx[(size_t)t * k + i] = i < n ? i : -1;
    return;
  }

  // Requested first, before anything waits on the sequence lookup: the head
  // (count and 15 highest bins) of list `tid` and this thread's first scores.
  // Only threads below the slot count read a head (the others' values are
  // never used; they would re-read the last list, 64 bytes a thread).
  uint4 h0 = make_uint4(0u, 0u, 0u, 0u), h1 = h0, h2 = h0, h3 = h0;
  if (tid < max_slots) {
    const uint4 *hp = (const uint4 *)(lbase + (size_t)tid * ws.slot_words);
    h0 = hp[0];
    h1 = hp[1];
    h2 = hp[2];
    h3 = hp[3];
  }
  float v[kSelPer];
  load_scores<kVec>(row, stride, c0 + tid * kSelPer, v);

  const int n = ws.ncand[t].x;
  if (n <= k) {
    // every candidate is kept: positions 0..n-1, then -1 (no candidates for
    // k_topk_finish)
    if (slot == 0) {
      for (int i = tid; i < k; i += kSelBlock) topk_idx[(size_t)t * k + i] = i < n ? i : -1;
      if (tid == 0) ws.thr[t] = make_uint4(0u, 0u, 0u, 0u);
    }
    return;
  }
  if (c0 >= n) return;
  const int nslots = (n + skeys - 1) / skeys;  // lists written for this query

  const uint32_t wd[16] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w,
                           h2.x, h2.y, h2.z, h2.w, h3.x, h3.y, h3.z, h3.w};
  uint32_t ub0, above0, total;  // threshold bin, keys above it, candidates of the query

  // ---- a./b. (at most 64 slots) one wave merges the heads, finds b0 and the
  // start of this slot's candidates, without a barrier in between
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  bool done = false;
  if (nslots <= 64) {
    if (wave == 0) {
      uint32_t ab;
      const int b = wave_heads_threshold_bin(wd, nslots, (uint32_t)k, &ab);
      // the heads are exact down to the lowest bin read from every cut list
      const bool cut = __ballot(lane < nslots && wd[0] > 15u && (int)(wd[15] >> 20) > b) != 0;
      const uint32_t cnt = lane < nslots ? head_count_ge(wd, (uint32_t)b) : 0u;
      const uint32_t inc = wave_inclusive_scan(cnt);
      // (lane reads with every lane active: inside the lane-0 branch below the
      // other lanes' values would not be computed)
      const uint32_t all = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
      const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)(inc - cnt), slot);
      if (lane == 0) {
        res[0] = cut ? 0 : 1;
        res[1] = b;
        s_misc[0] = ab;
        s_misc[1] = all;
        s_base = base;
      }
    }
    __syncthreads();
    done = res[0] != 0;
    ub0 = (uint32_t)res[1];
    above0 = s_misc[0];
    total = s_misc[1];
  }
  if (!done) {
    // ---- a. level-0 threshold from the list heads
    __syncthreads();  // the wave path's LDS results have been read
    for (int i = tid; i < kHist0Bins; i += kSelBlock) hist[i] = 0u;
    if (tid == 0) floor_max = -1;
    __syncthreads();
    int floor = -1;
    auto add_head = [&](const uint32_t (&e)[16]) {
      const uint32_t cnt = e[0];
#pragma unroll
      for (int i = 1; i < 16; ++i)
        if ((uint32_t)i <= cnt) atomicAdd(&hist[e[i] >> 20], e[i] & 0xFFFFFu);
      if (cnt > 15u) floor = max(floor, (int)(e[15] >> 20));
    };
    if (tid < nslots) add_head(wd);
    for (int sl = tid + kSelBlock; sl < nslots; sl += kSelBlock) {
      const uint4 *p = (const uint4 *)(lbase + (size_t)sl * ws.slot_words);
      const uint4 a0 = p[0], a1 = p[1], a2 = p[2], a3 = p[3];
      const uint32_t e[16] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w,
                              a2.x, a2.y, a2.z, a2.w, a3.x, a3.y, a3.z, a3.w};
      add_head(e);
    }
    if (floor >= 0) atomicMax(&floor_max, floor);
    __syncthreads();
    int b0 = find_threshold_bin<kHist0Bins, kSelBlock>(hist, (uint32_t)k, &above0, scratch, res);
    // The heads are exact down to the lowest bin read from every cut list; if
    // b0 lies below that, add the rest of the lists and search again (uniform).
    const bool full = b0 < floor_max;
    if (full) {
      for (int sl = tid; sl < nslots; sl += kSelBlock) {
        const uint32_t *l = lbase + (size_t)sl * ws.slot_words;
        const uint32_t cnt = l[0];
        for (uint32_t i = 16; i <= cnt; ++i) atomicAdd(&hist[l[i] >> 20], l[i] & 0xFFFFFu);
      }
      __syncthreads();
      b0 = find_threshold_bin<kHist0Bins, kSelBlock>(hist, (uint32_t)k, &above0, scratch, res);
    }
    ub0 = (uint32_t)b0;

    // ---- b. where this slot's candidates start: the candidates of all earlier
    // slots. Thread tid sums the slots [tid * per, (tid + 1) * per).
    const int per = (nslots + kSelBlock - 1) / kSelBlock;
    const int s_lo = min(nslots, tid * per), s_hi = min(nslots, s_lo + per);
    uint32_t mine = 0, upto = 0;  // candidates of my slots, and of my slots before `slot`
    if (per == 1 && !full) {
      if (tid < nslots) mine = head_count_ge(wd, ub0);
    } else {
      for (int sl = s_lo; sl < s_hi; ++sl) {
        if (sl == slot) upto = mine;
        mine += list_count_ge(lbase + (size_t)sl * ws.slot_words, ub0);
      }
    }
    const uint32_t before = block_exclusive_scan(mine, scratch, &total);
    if (slot >= s_lo && slot < s_hi) s_base = before + upto;
    __syncthreads();
  }
  if (slot == 0 && tid == 0) ws.thr[t] = make_uint4(ub0, above0, total, 0u);

  // ---- write this slot's candidates (position order) at their final place
  uint2 *cand = ws.entries + (size_t)t * ws.nchunk * kTopkChunk;
  const uint32_t cap = (uint32_t)ws.nchunk * kTopkChunk;  // >= max_kv_len >= n >= total
  const int64_t send = min((int64_t)n, c0 + skeys);
  uint32_t o = s_base;
  for (int64_t b = c0; b < send; b += kSelBatch) {
    if (b != c0) load_scores<kVec>(row, stride, b + tid * kSelPer, v);
    const int64_t p0 = b + tid * kSelPer;
    uint32_t keys[kSelPer];
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) {
      keys[j] = score_key(v[j]);
      cnt += (p0 + j < send && (keys[j] >> kHist0Shift) >= ub0) ? 1u : 0u;
    }
    uint32_t btot;
    uint32_t q = o + block_exclusive_scan(cnt, scratch, &btot);
#pragma unroll
    for (int j = 0; j < kSelPer; ++j)
      if (p0 + j < send && (keys[j] >> kHist0Shift) >= ub0) {
        if (q < cap) cand[q] = make_uint2((uint32_t)(p0 + j), keys[j]);
        ++q;
      }
    o += btot;
  }
}

// One workgroup per query: the exact threshold among the candidates written
// by k_topk_select and the ordered output.
__global__ __launch_bounds__(kFinBlock) void k_topk_finish(int k, TopkWs ws, int32_t *__restrict__ topk_idx) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[2 * kHist12Bins];  // levels 1 and 2
  __shared__ uint32_t scratch[kFinBlock / 64];
  __shared__ int res[2];
  const int t = blockIdx.x;
  int32_t *out = topk_idx + (size_t)t * k;
  FinishInput<kFinBlock> in;
  finish_request(ws, t, in);
  finish_query<kFinBlock>(k, ws, t, in, hist, scratch, res, [&](uint32_t o, int32_t pos) { out[o] = pos; });
}

}  // namespace

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// list geometry: at most ceil(n / 256) + 1 slots per query (the smallest
// producer slot covers 256 positions); a slot of K positions takes
// 4 + min(K, 4096) words, so a query needs at most
// max_kv_len + 8192 + 4 * slots words (one partly used slot of at most 8192
// positions beyond max_kv_len)
static size_t list_slots(int max_kv_len) { return ((size_t)max_kv_len + 255) / 256 + 1; }
static size_t list_q_stride(int max_kv_len) {
  return (((size_t)max_kv_len + 8192 + 4 * list_slots(max_kv_len)) + 3) / 4 * 4;
}

size_t topk_ws_bytes(int T, int max_kv_len) {
  size_t nch = ((size_t)max_kv_len + kTopkChunk - 1) / kTopkChunk;
  return align256((size_t)T * list_q_stride(max_kv_len) * 4) + align256((size_t)T * sizeof(uint4)) +
         align256((size_t)T * sizeof(int2)) + align256((size_t)T * nch * kTopkChunk * sizeof(uint2));
}

TopkWs topk_ws_carve(void *ws, int T, int max_kv_len) {
  TopkWs w{};
  w.nchunk = (int32_t)(((size_t)max_kv_len + kTopkChunk - 1) / kTopkChunk);
  w.list_q_stride = (int32_t)list_q_stride(max_kv_len);
  char *p = (char *)ws;
  w.lists = (uint32_t *)p;
  p += align256((size_t)T * w.list_q_stride * 4);
  w.thr = (uint4 *)p;
  p += align256((size_t)T * sizeof(uint4));
  w.ncand = (int2 *)p;
  p += align256((size_t)T * sizeof(int2));
  w.entries = (uint2 *)p;
  return w;
}

hipError_t launch_topk_hist0(const SeqMeta &m, int T, const float *scores, int64_t stride,
                             TopkWs *w, hipStream_t s) {
  w->slot_keys = kTopkChunk;
  w->slot_words = 4 + (kTopkChunk < kHist0Bins ? kTopkChunk : kHist0Bins);
  if (T == 0 || m.max_kv_len == 0) return hipSuccess;
  dim3 grid((m.max_kv_len + kTopkChunk - 1) / kTopkChunk, T);
  hipLaunchKernelGGL(k_topk_hist0, grid, dim3(256), 0, s, m, scores, stride, *w);
  return hipGetLastError();
}

hipError_t launch_topk_select(const SeqMeta &m, int T, int k, const float *scores, int64_t stride,
                              const TopkWs &w, int32_t *topk_idx, hipStream_t s, bool finish) {
  if (T == 0) return hipSuccess;
  int slots = 1;
  if (m.max_kv_len > k) {
    if (w.slot_keys <= 0 || (m.max_kv_len + w.slot_keys - 1) / w.slot_keys > kTopkMaxSlots)
      return hipErrorInvalidValue;  // level-0 lists missing or with too many slots
    slots = (m.max_kv_len + w.slot_keys - 1) / w.slot_keys;
  }
  // (with max_kv_len <= k every query takes the n <= k path before touching
  // the lists or the scores)
  dim3 grid(slots, T);
  const bool vec = stride >= 4 && (stride % 4 == 0) && (((uintptr_t)scores & 15) == 0) && (w.slot_keys % 4 == 0);
  if (vec)
    hipLaunchKernelGGL(k_topk_select<true>, grid, dim3(kSelBlock), 0, s, m, k, scores, stride, w, topk_idx);
  else
    hipLaunchKernelGGL(k_topk_select<false>, grid, dim3(kSelBlock), 0, s, m, k, scores, stride, w, topk_idx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || m.max_kv_len <= k || !finish) return e;
  hipLaunchKernelGGL(k_topk_finish, dim3(T), dim3(kFinBlock), 0, s, k, w, topk_idx);
  return hipGetLastError();
}

}  // namespace sga
