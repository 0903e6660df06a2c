// Per-query top-k select: the k positions of largest score, ties to the lowest
// position, returned in ascending position order (-1 padding when n_t < k).
//
// Source: "A.X-K2: a sparse-attention upgrade that costs nothing, trained
// natively in FP8", section "Sparse Gated Attention" (keep the top 2,048 tokens
// per query, at individual-token granularity rather than in blocks); "A.X K2
// Technical Report", section 3.4 (the indexer selects the top 2,048 tokens).
//
// Exact radix select on the order-preserving 32-bit key of each fp32 score,
// most significant digit first (12 + 10 + 10 bits):
//  1. level-0 histogram of key bits 31..20, as one list of nonzero bins per
//     producer workgroup (written by the indexer in the fused layer, or by
//     k_topk_hist0): no global atomics and nothing to clear beforehand;
//  2. k_topk_scan, one workgroup per 4096 positions: merges the query's lists
//     into the level-0 histogram (every workgroup of a query reaches the same
//     result; the first publishes it), finds the threshold bin b0 (the bin
//     holding the k-th largest key) and compacts, in position order, the
//     (position, key) pairs of its chunk whose digit is >= b0 (everything
//     above b0 is certainly selected; bin b0 holds the threshold);
//  3. k_topk_final, one workgroup per query: stages all pairs in LDS while
//     building the level-1 histogram (key bits 19..10) of bin b0, then the
//     level-2 histogram of the pairs sharing the top 22 bits of the threshold,
//     giving the exact k-th key K* and how many ties at K* to take; an ordered
//     pass then emits key > K* plus the first `take` ties, which are the
//     lowest positions because chunks and their pairs are visited in
//     position order.
// No atomics decide the output, so it is deterministic.

#include "kernels.h"
#include "select_common.h"

namespace sga {

namespace {

constexpr int kScanBlock = 256;
constexpr int kPerThread = kTopkChunk / kScanBlock;  // 16 consecutive scores per thread
constexpr int kFinalBlock = 512;
constexpr int kFinalCap = 12288;                     // pairs staged in LDS (96 KiB)
constexpr int kMaxChunks = 1024;                     // max_kv_len <= 4M

__global__ __launch_bounds__(256) void k_topk_hist0(SeqMeta m, const float *__restrict__ scores,
                                                    int64_t stride, TopkWs ws) {
  __shared__ uint32_t hist[kHist0Bins];
  __shared__ uint32_t scratch[256 / 64 + 1];
  const int t = blockIdx.y;
  int64_t start;
  const int n = query_candidates(m, t, &start);
  const int c0 = blockIdx.x * kTopkChunk;
  if (c0 >= n) return;
  for (int i = threadIdx.x; i < kHist0Bins; i += 256) hist[i] = 0u;
  __syncthreads();
  const float *row = scores + t * stride;
  for (int j = 0; j < kPerThread; ++j) {
    int s = c0 + j * 256 + threadIdx.x;
    if (s < n) atomicAdd(&hist[score_key(row[s]) >> kHist0Shift], 1u);
  }
  __syncthreads();
  write_hist0_list<false>(hist, ws, t, blockIdx.x, scratch);
}

template <bool kVec>
__global__ __launch_bounds__(kScanBlock) void k_topk_scan(SeqMeta m, int k,
                                                          const float *__restrict__ scores,
                                                          int64_t stride, TopkWs ws,
                                                          int32_t *__restrict__ topk_idx) {
  __shared__ uint32_t hist[kHist0Bins];
  __shared__ uint32_t scratch[kScanBlock / 64 + 1];
  __shared__ int res[2];
  __shared__ int floor_max;
  const int t = blockIdx.y;
  int64_t start;
  const int n = query_candidates(m, t, &start);
  if (n <= k) {
    // every candidate is kept: positions 0..n-1, then -1
    if (blockIdx.x == 0)
      for (int i = threadIdx.x; i < k; i += kScanBlock)
        topk_idx[(size_t)t * k + i] = i < n ? i : -1;
    return;
  }
  const int c0 = blockIdx.x * kTopkChunk;
  if (c0 >= n) return;
  // this thread's 16 consecutive scores, requested before the threshold search
  const float *row = scores + t * stride;
  const int p0 = c0 + threadIdx.x * kPerThread;
  float v[kPerThread];
  if (kVec && p0 + kPerThread <= n) {
#pragma unroll
    for (int q = 0; q < kPerThread / 4; ++q) {
      const float4 x = *(const float4 *)(row + p0 + 4 * q);
      v[4 * q] = x.x;
      v[4 * q + 1] = x.y;
      v[4 * q + 2] = x.z;
      v[4 * q + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) v[j] = p0 + j < n ? row[p0 + j] : 0.0f;
  }
  // level-0 threshold of the query from its lists (every workgroup of the
  // query derives the same b0; the first one publishes it for k_topk_final)
  for (int i = threadIdx.x; i < kHist0Bins; i += kScanBlock) hist[i] = 0u;
  uint32_t above0;
  const int b0 = merge_lists_threshold<kScanBlock>(ws, t, n, k, hist, &floor_max, scratch, res, &above0);
  if (blockIdx.x == 0 && threadIdx.x == 0) ws.thr[t] = make_uint2((uint32_t)b0, above0);

  uint32_t keys[kPerThread];
  uint32_t cnt = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const uint32_t key = score_key(v[j]);
    keys[j] = key;
    cnt += (p0 + j < n && (int)(key >> kHist0Shift) >= b0) ? 1u : 0u;
  }
  uint32_t total;
  uint32_t off = block_exclusive_scan(cnt, scratch, &total);  // includes barriers
  uint2 *dst = ws.entries + ((size_t)t * ws.nchunk + blockIdx.x) * kTopkChunk;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    if (p0 + j < n && (int)(keys[j] >> kHist0Shift) >= b0)
      dst[off++] = make_uint2((uint32_t)(p0 + j), keys[j]);
  }
  if (threadIdx.x == 0) ws.counts[(size_t)t * ws.nchunk + blockIdx.x] = total;
}

// Chunk holding flat pair index f (offs ascending, offs[0] = 0, offs[nch] = total > f).
__device__ __forceinline__ int chunk_of(const uint32_t *offs, int nch, uint32_t f) {
  int lo = 0, hi = nch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offs[mid] <= f) lo = mid; else hi = mid - 1;
  }
  return lo;
}

constexpr int kBatch = 8;    // independent loads in flight per thread
__global__ __launch_bounds__(kFinalBlock) void k_topk_final(SeqMeta m, int k, TopkWs ws,
                                                            int32_t *__restrict__ topk_idx) {
  extern __shared__ uint2 pairs[];  // kFinalCap entries
  __shared__ uint32_t hist[kHist12Bins];
  __shared__ uint32_t offs[kMaxChunks + 1];
  __shared__ uint32_t scratch[kFinalBlock / 64 + 1];
  __shared__ int res[2];
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  int64_t start;
  const int n = query_candidates(m, t, &start);
  if (n <= k) return;
  const int nch = (n + kTopkChunk - 1) / kTopkChunk;
  const uint32_t *cnts = ws.counts + (size_t)t * ws.nchunk;
  // chunk counts (<= 2 per thread) and the level-0 result
  const uint32_t c_a = 2 * tid < nch ? cnts[2 * tid] : 0u;
  const uint32_t c_b = 2 * tid + 1 < nch ? cnts[2 * tid + 1] : 0u;
  for (int i = tid; i < kHist12Bins; i += kFinalBlock) hist[i] = 0u;
  const uint2 thr = ws.thr[t];
  const uint32_t b0 = thr.x;
  uint32_t want = (uint32_t)k - thr.y;
  __syncthreads();
  uint32_t total;
  const uint32_t ex = block_exclusive_scan(c_a + c_b, scratch, &total);
  if (2 * tid < nch) offs[2 * tid] = ex;
  if (2 * tid + 1 < nch) offs[2 * tid + 1] = ex + c_a;
  if (tid == 0) offs[nch] = total;
  __syncthreads();

  // stage the pairs in position order (a group of threads per chunk, no
  // search) and build the level-1 histogram (key bits 19..10) of bin b0
  const uint2 *src = ws.entries + (size_t)t * ws.nchunk * kTopkChunk;
  const bool staged = total <= (uint32_t)kFinalCap;
  int gsz = kFinalBlock;
  while (gsz > 1 && gsz > kFinalBlock / nch) gsz >>= 1;  // threads per chunk (power of 2)
  if (gsz * nch > kFinalBlock) gsz = 1;
  const int groups = kFinalBlock / gsz;
  const int gid = tid / gsz, gl = tid % gsz;
  for (int c0 = 0; c0 < nch; c0 += groups) {
    const int c = c0 + gid;
    if (c < nch) {
      const uint32_t cnt = offs[c + 1] - offs[c];
      const uint2 *cs = src + (size_t)c * kTopkChunk;
      for (uint32_t i0 = gl; i0 < cnt; i0 += gsz * kBatch) {
        uint2 v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const uint32_t i = i0 + u * gsz;
          if (i < cnt) v[u] = cs[i];
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const uint32_t i = i0 + u * gsz;
          if (i < cnt) {
            if (staged) pairs[offs[c] + i] = v[u];
            if ((v[u].y >> kHist0Shift) == b0) atomicAdd(&hist[(v[u].y >> 10) & 1023u], 1u);
          }
        }
      }
    }
  }
  __syncthreads();
  uint32_t above1;
  const int b1 = find_threshold_bin<kHist12Bins>(hist, want, &above1, scratch, res);
  want -= above1;
  const uint32_t prefix22 = (b0 << 10) | (uint32_t)b1;  // key bits 31..10 of K*
  auto pair_at = [&](uint32_t f) -> uint2 {
    if (staged) return pairs[f];
    const int c = chunk_of(offs, nch, f);
    return src[(size_t)c * kTopkChunk + (f - offs[c])];
  };
  // level 2: the last 10 bits among the pairs that share the top 22 bits
  for (int i = tid; i < kHist12Bins; i += kFinalBlock) hist[i] = 0u;
  __syncthreads();
  for (uint32_t f = tid; f < total; f += kFinalBlock) {
    const uint32_t key = pair_at(f).y;
    if ((key >> 10) == prefix22) atomicAdd(&hist[key & 1023u], 1u);
  }
  __syncthreads();
  uint32_t above2;
  const int b2 = find_threshold_bin<kHist12Bins>(hist, want, &above2, scratch, res);
  want -= above2;
  const uint32_t kstar = (prefix22 << 10) | (uint32_t)b2;  // the exact k-th largest key
  const uint32_t take = want;                                 // ties at kstar to keep

  // ordered emission: each thread owns a contiguous run of pairs
  const uint32_t seg = (total + kFinalBlock - 1) / kFinalBlock;
  const uint32_t s0 = min(total, tid * seg), s1 = min(total, s0 + seg);
  uint32_t n_gt = 0, n_eq = 0;
  for (uint32_t f = s0; f < s1; ++f) {
    const uint32_t key = pair_at(f).y;
    n_gt += key > kstar;
    n_eq += key == kstar;
  }
  uint32_t tmp;
  const uint32_t tie_base = block_exclusive_scan(n_eq, scratch, &tmp);
  const uint32_t ties_here = tie_base >= take ? 0u : min(n_eq, take - tie_base);
  const uint32_t out_base = block_exclusive_scan(n_gt + ties_here, scratch, &tmp);
  uint32_t o = out_base, tr = tie_base;
  for (uint32_t f = s0; f < s1; ++f) {
    const uint2 pk = pair_at(f);
    bool sel = pk.y > kstar;
    if (pk.y == kstar) {
      sel = tr < take;
      ++tr;
    }
    if (sel) {
      if (o < (uint32_t)k) topk_idx[(size_t)t * k + o] = (int32_t)pk.x;
      ++o;
    }
  }
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
  return align256((size_t)T * list_q_stride(max_kv_len) * 4) + align256((size_t)T * sizeof(uint2)) +
         align256((size_t)T * nch * 4) + align256((size_t)T * nch * kTopkChunk * sizeof(uint2));
}

TopkWs topk_ws_carve(void *ws, int T, int max_kv_len) {
  TopkWs w{};
  w.nchunk = (int32_t)(((size_t)max_kv_len + kTopkChunk - 1) / kTopkChunk);
  w.list_q_stride = (int32_t)list_q_stride(max_kv_len);
  char *p = (char *)ws;
  w.lists = (uint32_t *)p;
  p += align256((size_t)T * w.list_q_stride * 4);
  w.thr = (uint2 *)p;
  p += align256((size_t)T * sizeof(uint2));
  w.counts = (uint32_t *)p;
  p += align256((size_t)T * w.nchunk * 4);
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

hipError_t launch_topk_scan(const SeqMeta &m, int T, int k, const float *scores, int64_t stride,
                            const TopkWs &w, int32_t *topk_idx, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (m.max_kv_len > k && (w.slot_keys <= 0 || (m.max_kv_len + w.slot_keys - 1) / w.slot_keys > kTopkMaxSlots))
    return hipErrorInvalidValue;  // level-0 lists missing or with too many slots
  int nch = m.max_kv_len > 0 ? (m.max_kv_len + kTopkChunk - 1) / kTopkChunk : 1;
  dim3 grid(nch, T);
  const bool vec = (stride % 4 == 0) && (((uintptr_t)scores & 15) == 0);
  if (vec)
    hipLaunchKernelGGL(k_topk_scan<true>, grid, dim3(kScanBlock), 0, s, m, k, scores, stride, w,
                       topk_idx);
  else
    hipLaunchKernelGGL(k_topk_scan<false>, grid, dim3(kScanBlock), 0, s, m, k, scores, stride, w,
                       topk_idx);
  return hipGetLastError();
}

hipError_t launch_topk_final(const SeqMeta &m, int T, int k, const TopkWs &w, int32_t *topk_idx,
                             hipStream_t s) {
  if (T == 0 || m.max_kv_len <= k) return hipSuccess;
  const size_t dyn = (size_t)kFinalCap * sizeof(uint2);
  static bool attr_set = false;
  if (!attr_set) {
    // allow more than the default dynamic LDS; a refusal surfaces at launch
    (void)hipFuncSetAttribute((const void *)k_topk_final,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    (void)hipGetLastError();
    attr_set = true;
  }
  hipLaunchKernelGGL(k_topk_final, dim3(T), dim3(kFinalBlock), dyn, s, m, k, w, topk_idx);
  return hipGetLastError();
}

}  // namespace sga
