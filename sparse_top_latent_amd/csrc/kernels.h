// Host-side launchers of the SGA kernels (one translation unit per kernel family).
#pragma once

#include <atomic>

#include "common.h"

namespace sga {

// Compute units of the current device, looked up once per device (safe to
// call from several host threads: a race only repeats the lookup).
inline int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) {
    (void)hipGetLastError();
    c = 256;
  }
  cache[dev].store(c, std::memory_order_relaxed);
  return c;
}

// --- indexer score pass ----------------------------------------------------
// scores[t * stride + s] for s < n_t.
struct TopkWs;
// With `sel` set, the indexer also writes the level-0 histogram lists of the
// top-k select (and records their slot geometry in *sel).
hipError_t launch_index_f32(const SeqMeta &m, int T, int k, int HI, int DI, const float *q_idx,
                            const float *w, const float *k_idx, float *scores, int64_t stride,
                            TopkWs *sel, hipStream_t s);
hipError_t launch_index_fp8(const SeqMeta &m, int T, int k, const uint8_t *q_idx, const float *w,
                            const uint8_t *k_idx, float *scores, int64_t stride, TopkWs *sel,
                            hipStream_t s);
// Query-tiled FP8 scores for the query-row groups whose rows all name one
// sequence (other groups are left untouched); used by launch_index_fp8.
hipError_t launch_index_fp8_prefill(const SeqMeta &m, int T, const uint8_t *q_idx, const float *w,
                                    const uint8_t *k_idx, float *scores, int64_t stride,
                                    hipStream_t s);

// Streaming-read reference (the index kernel's LDS-DMA copy pattern without
// the scoring) over bytes / 8192 whole tiles of src; one word per workgroup
// (at most kStreamReadBlocksPerCu per CU) goes to sink.
constexpr int kStreamReadBlocksPerCu = 2;
hipError_t launch_stream_read(const uint8_t *src, int64_t bytes, uint32_t *sink, hipStream_t s);

// --- top-k select -----------------------------------------------------------
// The level-0 histogram of a query (4096 bins of the top 12 key bits) arrives
// as lists, one per producer workgroup ("slot") covering slot_keys positions.
// Slot `slot` of query t starts at word t * list_q_stride + slot * slot_words
// of `lists` (16-byte aligned): its entry count, then the entries
// (bin << 20 | count) in descending bin order. No global atomics build them
// and nothing is cleared beforehand. A producer also records, from its
// workgroup 0 of query t, n_t and the cache row of position 0 of the query's
// sequence in ncand[t] (the row is 0 in the paged layout; rows fit 32 bits).
constexpr int kTopkMaxSlots = 4096;  // level-0 list slots one query may use
struct TopkWs {
  uint32_t *lists;        // [T, list_q_stride]
  int32_t list_q_stride;  // words reserved per query
  int32_t slot_keys;      // positions one slot covers (set by the producer's launcher)
  int32_t slot_words;     // words per slot: 4 + at most 4096 entries (set by the producer's launcher)
  uint4 *thr;             // [T] (b0, keys above bin b0, candidates, 0)
  int2 *ncand;            // [T] (candidate count n_t, row of position 0)
  uint2 *entries;         // [T, nchunk * kTopkChunk] candidates (position, key)
  int32_t nchunk;         // ceil(max_kv_len / kTopkChunk)
};
size_t topk_ws_bytes(int T, int max_kv_len);
TopkWs topk_ws_carve(void *ws, int T, int max_kv_len);
hipError_t launch_topk_hist0(const SeqMeta &m, int T, const float *scores, int64_t stride,
                             TopkWs *w, hipStream_t s);
// Select (one workgroup per (slot, query)) and finish (one per query); needs
// the lists and ncand from a producer launched earlier on the same stream.
// With finish false only the select kernel runs; the last step is then left
// to the consumer (the fused MLA split kernel, see MlaArgs::sel).
hipError_t launch_topk_select(const SeqMeta &m, int T, int k, const float *scores, int64_t stride,
                              const TopkWs &w, int32_t *topk_idx, hipStream_t s, bool finish = true);

// --- sparse MLA + gate ---------------------------------------------------------
struct MlaArgs {
  SeqMeta meta;
  int T, H, Dc, Dr, k;
  float tau;
  const void *q;
  int q_dtype;
  const void *kv;
  int kv_dtype;
  const uint8_t *kv_scale;
  const int32_t *topk_idx;
  const void *gate;
  int gate_dtype;
  void *out;
  int out_dtype;
  float *lse;
  // fused top-k finish (split kernel only): with fuse set, the split kernel
  // takes its rows from the select kernel's candidates in `sel` instead of
  // topk_idx, and writes the selected positions to topk_out when it is set
  bool fuse;
  TopkWs sel;
  int32_t *topk_out;
};
// generic fp32 path (one workgroup per (query, head))
hipError_t launch_mla_f32(const MlaArgs &a, hipStream_t s);
// MI355X path: H=64, Dc=512, Dr=64, bf16 or MXFP8 rows
constexpr int kMlaRowsPerSplit = 128;
size_t mla_split_ws_bytes(int T, int k);
// whether the MLA runs as whole queries (no partials, no combine pass)
bool mla_whole_query_path(int T, int kv_dtype, int page_shift);
hipError_t launch_mla_split(const MlaArgs &a, void *ws, hipStream_t s);
// whether the split kernel should do the top-k's last step itself (fuse)
bool mla_fuse_finish(int T, int k);
hipError_t launch_mla_combine(const MlaArgs &a, const void *ws, hipStream_t s);

// --- cache append ---------------------------------------------------------------
// Token i's row kv_new[i] (D values) and key kidx_new[i] (DI values) go to cache
// row slots[i] in kv_dtype / idx_dtype; slots outside [0, rows) are dropped.
// A NULL kv_new or kidx_new skips that part. Needs D and DI multiples of 8
// (D of 32 for MXFP8) and N * (D + DI) / 8 < 2^32.
hipError_t launch_cache_append(int64_t N, int D, int DI, int src_dtype, const void *kv_new,
                               const void *kidx_new, const int64_t *slots, int64_t rows,
                               int kv_dtype, void *kv, uint8_t *kv_scale, int idx_dtype,
                               void *k_idx, hipStream_t s);

// --- indexer KL loss (training side) ------------------------------------------
size_t indexer_kl_ws_bytes(int T, int k, int HI, int DI);
// LDS bytes the KL kernels need (must stay within 160 KiB)
size_t indexer_kl_smem(int H, int D, int HI, int DI, int q_dtype);
hipError_t launch_indexer_kl(const SeqMeta &m, int T, int H, int D, int HI, int DI, int k, float tau,
                             const void *q, int q_dtype, const void *kv, int kv_dtype,
                             const uint8_t *kv_scale, const void *q_idx, const float *w,
                             const void *k_idx, int idx_dtype, const int32_t *topk_idx,
                             const float *lse, float *loss, float *d_w, float *d_q_idx, float *d_k_idx,
                             void *ws, hipStream_t s);

}  // namespace sga
