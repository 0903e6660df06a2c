// Sparse MLA over the selected latent rows, followed by the sigmoid output gate.
//
// Source: "A.X-K2: a sparse-attention upgrade that costs nothing, trained
// natively in FP8", section "Sparse Gated Attention" (attention reads only the
// chosen latent rows; a learned per-head gate multiplies the attention result
// ahead of Wo); "SK Telecom Opens A.X K2: 688B Parameters and One Telling
// Benchmark", block-diagram caption (sigmoid output gate); "A.X K2 Technical
// Report", section 2 (the MLA backbone carries a per-head output gate).
//
// Absorbed MLA: all heads share one cached row [c_s | kR_s] per position, so a
// gathered row serves every head. For query t and head h:
//   logit_s = tau * q[t,h,:] . row_s ;  p = softmax over the selected rows ;
//   o = sum_s p_s c_s ;  y = sigmoid(g[t,h,:]) * o.
//
// Kernels:
//  * k_mla_f32: generic fp32 path, one workgroup per (query, head).
//  * k_mla_split8 (MI355X path, H = 64, Dc = 512, Dr = 64): the selected rows
//    of a query are cut into splits of 128, 256 or 512 (one, two or four
//    rounds of 128); one workgroup per (split, query) gathers 32-row tiles
//    into LDS (bf16, or MXFP8 expanded exactly to bf16). Its 8 waves form two
//    sets of 4 that take alternate tiles and merge at the end. Per wave:
//      S^T = rows . Q^T  with bf16 16x16x32 MFMA (the query slice stays in VGPRs),
//      online softmax per head in fp32 (exp2 domain),
//      O^T += V^T . P^T  with bf16 MFMA; P^T comes straight from the S^T
//      accumulator layout, V^T is read column-wise from the LDS tile.
//    It writes a partial (max, sum in fp32; O in bf16) per (query, split, head).
//  * k_mla_combine: merges the splits of each (query, head) with the usual
//    log-sum-exp rescaling and applies the gate in the epilogue; partials are
//    stored and read in the split kernel's register order (coalesced).

#include "kernels.h"
#include "select_common.h"

namespace sga {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// --------------------------------------------------------------------------
// block reductions
// --------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}
template <bool kMax>
__device__ __forceinline__ float block_reduce(float v, float *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = kMax ? wave_max(v) : wave_sum(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nw; ++i) r = kMax ? fmaxf(r, red[i]) : r + red[i];
  __syncthreads();
  return r;
}

// --------------------------------------------------------------------------
// generic fp32 path
// --------------------------------------------------------------------------
constexpr int kF32Block = 256;
constexpr int kF32MaxD = 1024;
constexpr int kF32MaxK = 4096;

__global__ __launch_bounds__(kF32Block) void k_mla_f32(MlaArgs a) {
  __shared__ float qs[kF32MaxD];
  __shared__ float pr[kF32MaxK];
  __shared__ int64_t rows[kF32MaxK];
  __shared__ float red[kF32Block / 64];
  const int h = blockIdx.x, t = blockIdx.y;
  const int D = a.Dc + a.Dr;
  int64_t start;
  const int L = seq_len_clipped(a.meta, a.meta.q_seq[t], &start);
  const float *q = (const float *)a.q + ((size_t)t * a.H + h) * D;
  const float *kv = (const float *)a.kv;
  for (int i = threadIdx.x; i < D; i += kF32Block) qs[i] = q[i];
  __syncthreads();
  float mx = -INFINITY;
  for (int r = threadIdx.x; r < a.k; r += kF32Block) {
    int32_t pos = a.topk_idx[(size_t)t * a.k + r];
    bool ok = pos >= 0 && pos < L;
    int64_t row = ok ? kv_row(a.meta, a.meta.q_seq[t], start, pos) : -1;
    float lg = -INFINITY;
    if (ok) {
      const float *kr = kv + row * D;
      float acc = 0.0f;
      for (int d = 0; d < D; ++d) acc = fmaf(qs[d], kr[d], acc);
      lg = a.tau * acc;
    }
    rows[r] = row;
    pr[r] = lg;
    mx = fmaxf(mx, lg);
  }
  mx = block_reduce<true>(mx, red);
  float sum = 0.0f;
  for (int r = threadIdx.x; r < a.k; r += kF32Block) {
    float p = rows[r] >= 0 ? __expf(pr[r] - mx) : 0.0f;
    pr[r] = p;
    sum += p;
  }
  sum = block_reduce<false>(sum, red);  // includes a barrier: pr[] is complete
  const bool empty = !(mx > -INFINITY);
  const float inv = empty ? 0.0f : 1.0f / sum;
  for (int c = threadIdx.x; c < a.Dc; c += kF32Block) {
    float acc = 0.0f;
    for (int r = 0; r < a.k; ++r) {
      int64_t row = rows[r];
      if (row >= 0) acc = fmaf(pr[r], kv[row * D + c], acc);
    }
    float o = acc * inv;
    size_t oi = ((size_t)t * a.H + h) * a.Dc + c;
    if (a.gate) o *= sigmoidf_exact_ends(load_as_f32(a.gate, a.gate_dtype, oi));
    store_from_f32(a.out, a.out_dtype, oi, o);
  }
  if (a.lse && threadIdx.x == 0) a.lse[(size_t)t * a.H + h] = empty ? -INFINITY : mx + __logf(sum);
}

// --------------------------------------------------------------------------
// MI355X path
// --------------------------------------------------------------------------
constexpr int kH = 64, kDc = 512, kD = 576;  // d_rope = 64
constexpr int kTile = 32;                     // rows per LDS tile
constexpr int kMaxTiles = kMlaRowsPerSplit / kTile;
constexpr int kMaxRounds = 4;                 // rounds of 128 rows one split kernel workgroup may take
constexpr int kRowChunks = kD * 2 / 16;       // 72 16-byte chunks per bf16 row
constexpr int kTileBytes = kTile * kD * 2;    // 36,864
constexpr int kBfDma = kTile * kRowChunks / 256;  // 9 DMA issues per thread per tile
constexpr int kMxChunks = kTile * kD / 16;    // 1,152 16-byte chunks of E4M3FN values per tile
constexpr int kMxDma = 5;                     // 1,280 slots per tile (the last 128 are padding)
constexpr int kMxRawBytes = kMxDma * 256 * 16;
constexpr int kScales = kD / 32;              // 18 E8M0 scales per row
constexpr int kKsteps = kD / 32;              // 18 MFMA k-steps for q . row
constexpr int kCt = kDc / 16;                 // 32 channel tiles of the value
constexpr float kRescaleSlack = 8.0f;         // log2 headroom before the running max moves

constexpr size_t kBfSmem = (size_t)kMaxTiles * kTileBytes;
// k_mla_split8<MXFP8>: the raw tiles, one expanded bf16 tile per wave set, the scales
constexpr size_t kMx8Smem = (size_t)kMaxTiles * kMxRawBytes + 2 * kTileBytes + kMlaRowsPerSplit * kScales;
static_assert(kMx8Smem + kMaxRounds * kMlaRowsPerSplit * 4 <= 160 * 1024, "LDS of k_mla_split8<MXFP8>");
static_assert(4 * kCt * 64 * 16 + 2 * 4 * 64 * 8 <= kMx8Smem, "the set merge reuses the tile area");

// 16 zero bytes: the DMA source of rows that are not selected
__device__ __attribute__((aligned(16))) uint32_t g_zero16[4];

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ v4f mfma_bf16(const v8bf &a, const v8bf &b, const v4f &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8bf as_v8bf(const v4i &x) { return __builtin_bit_cast(v8bf, x); }

// 16-byte chunk `chunk` of tile row `row` lives at chunk slot
// row*72 + (chunk ^ row_swz(row)): an XOR swizzle inside aligned groups of 8
// chunks that spreads same-column reads of consecutive rows over the LDS
// banks (a row is 288 dwords, so every row starts on the same bank of a
// 128-byte bank window). Chosen by the bank-conflict counter of gfx950
// (SQ_LDS_BANK_CONFLICT) among XOR swizzles of period 16 in the row: with
// row & 7 the whole-query kernel has no conflict cycles and the split
// kernel 91 K per launch (16 x 128K), against 134 M and 615 K with
// (row >> 1) & 7; swizzles that separate rows 4 apart instead (bits 1..0 of
// the row moved up) doubled them. Kernel times did not change with any of
// them (the MLA passes are not bound by LDS bandwidth).
__device__ __forceinline__ int row_swz(int row) { return row & 7; }
__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowChunks + (chunk ^ row_swz(row)); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that waits for this wave's LDS operations but not for its
// outstanding global->LDS DMAs (a __syncthreads() would drain those too).
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void dma16(const void *src, unsigned char *lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void *)lds_wave_base, 16, 0, 0);
}

// --------------------------------------------------------------------------
// Split kernel (bf16 or MXFP8 latent cache), two waves per SIMD.
//
// 8 waves: wave w serves heads 16 (w % 4) .. 16 (w % 4) + 15 for the tiles of
// its set (w / 4): set 0 takes tiles 0 and 2, set 1 tiles 1 and 3, each with
// its own running max, sum and output accumulator. Each set requests both of
// its tiles at once (with all 8 waves issuing, the gather runs near the
// random-row rate of the memory system). At the end the sets swap half of
// their accumulators through LDS and each merges and writes half of the
// partial.
// --------------------------------------------------------------------------
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// One block of four O^T channel tiles: V^T operands through the transposed
// read (ds_read_b64_tr_b16) of rows 4g.. (lo) and 16 rows further (hi). The
// compiler waits for the wave's outstanding LDS-DMA copies before the first
// such read; in practice the rest of the gather lands while the QK^T block in
// front of it runs, so the wait costs little.
template <int kM, int N>
__device__ __forceinline__ void pv_block_b(const unsigned char *tile, const int (&voff)[4], const v8bf &pb,
                                           v4f (&acc)[N]) {
  static_assert(4 * kM + 3 < N, "accumulator block");
  typedef __attribute__((address_space(3))) v4bf lds_v4bf;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v4bf lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf *)(tile + voff[i] + kM * 128));
    const v4bf hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf *)(tile + voff[i] + kM * 128 + 16 * kRowChunks * 16));
    const v8bf va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    acc[4 * kM + i] = mfma_bf16(va, pb, acc[4 * kM + i]);
  }
}

// The same block for a tile whose neighbours in the LDS ring are still being
// copied: the compiler cannot tell the transposed read from those copies and
// would wait for all of them before it, so the 8 reads are issued in one asm
// statement that also waits for them (lgkmcnt) before it ends.
template <int kM, int N>
__device__ __forceinline__ void pv_block_ring(const unsigned char *tile, const int (&voff)[4], const v8bf &pb,
                                              v4f (&acc)[N]) {
  static_assert(4 * kM + 3 < N, "accumulator block");
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  const uint32_t base = (uint32_t)(uintptr_t)(lds_u8 *)tile;
  v2u lo[4], hi[4];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:%13\n\t"
      "ds_read_b64_tr_b16 %2, %9 offset:%12\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
      "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:%13\n\t"
      "ds_read_b64_tr_b16 %6, %11 offset:%12\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:%13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]), "=&v"(lo[3]),
        "=&v"(hi[3])
      : "v"(base + voff[0]), "v"(base + voff[1]), "v"(base + voff[2]), "v"(base + voff[3]), "n"(kM * 128),
        "n"(kM * 128 + 16 * kRowChunks * 16)
      : "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v4bf l4 = __builtin_bit_cast(v4bf, lo[i]);
    const v4bf h4 = __builtin_bit_cast(v4bf, hi[i]);
    const v8bf va = {l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
    acc[4 * kM + i] = mfma_bf16(va, pb, acc[4 * kM + i]);
  }
}

// the cache row of position pos of the query's sequence (paged: through the
// block table)
template <bool kPaged>
__device__ __forceinline__ int32_t split_row(const MlaArgs &a, int b, int64_t start, int32_t pos) {
  return kPaged ? (int32_t)kv_row(a.meta, b, start, pos) : (int32_t)(start + pos);
}

// Workgroup b of a 1-D grid of S x T split workgroups -> (split, query).
// Workgroups are handed to the 8 XCDs round-robin (b mod 8); when the grid
// divides evenly, the mapping gives every XCD a run of consecutive (query,
// split) pairs, so that the splits of one query share an XCD and its L2:
// the query's 73.7 KB slice and its top-k candidates, which every split
// reads, are then fetched from memory once per query instead of once per
// XCD. Any other grid keeps the plain order.
constexpr int kXcds = 8;
__device__ __forceinline__ void split_of_block(int b, int S, int T, int *split, int *t) {
  const int total = S * T;
  int v = b;
  if (total % kXcds == 0) v = (b % kXcds) * (total / kXcds) + b / kXcds;
  *split = v % S;
  *t = v / S;
}

template <bool kMx, int R, bool kFuse, bool kPaged>
__global__ __launch_bounds__(512) void k_mla_split8(MlaArgs a, uint16_t *__restrict__ opart,
                                                    float2 *__restrict__ ml, int S) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // cache row of each selected row of the split (-1: none); int32 row ids
  // keep the gather's address batches small in registers
  __shared__ int32_t rows[R * kMlaRowsPerSplit];
  int split, t;
  split_of_block(blockIdx.x, S, a.T, &split, &t);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave & 3, set = wave >> 2, st = tid & 255;
  const int g = lane >> 4, c16 = lane & 15;
  // this split: R rounds of 128 selected rows
  const int r0 = split * R * kMlaRowsPerSplit;
  const int nrows = min(R * kMlaRowsPerSplit, a.k - r0);  // >= 1
  const int rounds = (nrows + kMlaRowsPerSplit - 1) / kMlaRowsPerSplit;
  // the query slice of this wave's 16 heads (B operands of S^T = rows . Q^T);
  // with the fused top-k finish it is requested right after the finish's
  // first candidates, so that it lands while the finish runs; elsewhere after
  // the row lookup, which keeps the many-round instances clear of register
  // spills
  const int head = hg * 16 + c16;
  const uint8_t *qh = (const uint8_t *)a.q + ((size_t)t * kH + head) * kD * 2;
  v8bf qreg[kKsteps];
  auto load_q = [&] {
#pragma unroll
    for (int ks = 0; ks < kKsteps; ++ks) qreg[ks] = as_v8bf(*(const v4i *)(qh + (ks * 32 + 8 * g) * 2));
  };
  int64_t start;
  if (!kFuse) {
    // the selected positions are requested first (clamped, unconditional) so
    // that their latency overlaps the sequence lookup; thread i takes row i
    const int my_row = min(tid, R * kMlaRowsPerSplit - 1);
    int32_t pos = a.topk_idx[(size_t)t * a.k + r0 + min(my_row, nrows - 1)];
    const int b = a.meta.q_seq[t];
    const int L = seq_len_clipped(a.meta, b, &start);
    if (tid < R * kMlaRowsPerSplit)
      rows[tid] = (tid < nrows && pos >= 0 && pos < L) ? split_row<kPaged>(a, b, start, pos) : -1;
  } else {
    // The top-k's last step, done here for the workgroup's own output slots
    // [r0, r0 + nrows) of the query (every split workgroup of the query
    // repeats it; that costs no time, since it replaces a kernel boundary and
    // the wait for the selected positions). n_t <= k: every candidate, in
    // position order, then -1. All the lookups are requested at once: the
    // finish's first candidates and totals (the fused finish runs only when
    // max_kv_len > k, so k_topk_select has written them), n_t with the row of
    // position 0 (recorded by the index pass) and, paged, the sequence; then
    // the query slice, so that waiting for any earlier load leaves it in
    // flight. Every candidate position is below n_t, which the sequence's
    // cached length bounds.
    FinishInput<512> fin;
    finish_request(a.sel, t, fin);
    const int2 nc = a.sel.ncand[t];
    const int b = kPaged ? a.meta.q_seq[t] : 0;
    asm volatile("" ::: "memory");
    if (set == 0) load_q();  // set 1 takes its copy from set 0 through LDS (below)
    const int n = nc.x;
    start = kPaged ? 0 : nc.y;
    if (tid < R * kMlaRowsPerSplit) {
      const int32_t pos = (n <= a.k && tid < nrows && r0 + tid < n) ? r0 + tid : -1;
      rows[tid] = pos >= 0 ? split_row<kPaged>(a, b, start, pos) : -1;
      if (n <= a.k && a.topk_out && tid < nrows) a.topk_out[(size_t)t * a.k + r0 + tid] = pos;
    }
    if (n > a.k) {  // uniform over the workgroup
      // (LDS for the histograms and scan at the start of the tile area; the
      // copies into it start after the barrier below)
      uint32_t *fh = (uint32_t *)smem;
      finish_query<512>(a.k, a.sel, t, fin, fh, fh + 2 * kHist12Bins, (int *)(fh + 2 * kHist12Bins + 8),
                        [&](uint32_t o, int32_t p) {
                          if (o >= (uint32_t)r0 && o < (uint32_t)(r0 + nrows)) {
                            rows[o - r0] = (p >= 0 && p < n) ? split_row<kPaged>(a, b, start, p) : -1;
                            if (a.topk_out) a.topk_out[(size_t)t * a.k + o] = p;
                          }
                        });
    }
  }
  // Fused: the two wave sets need the same query slice (waves w and w + 4
  // serve the same 16 heads). Set 0 loaded it; it writes it to 73,728 bytes
  // of LDS that no copy fills before the first tiles are under way (bf16:
  // the ring's tiles 2 and 3; MXFP8: the expanded tiles), and set 1 reads it
  // after the barrier below. One load of the slice per workgroup instead of
  // two: the finish's first loads share the memory system with half as many
  // bytes (split kernel 24.8-25.0 -> 24.3-24.5 us on 16 x 128K).
  unsigned char *qx = smem + (kMx ? kMaxTiles * kMxRawBytes : 2 * kTileBytes) + hg * (kKsteps * 1024) + lane * 16;
  static_assert(4 * kKsteps * 1024 == 2 * kTileBytes, "the query slice fills two tiles");
  if (kFuse && set == 0) {
#pragma unroll
    for (int ks = 0; ks < kKsteps; ++ks) *(v4i *)(qx + ks * 1024) = __builtin_bit_cast(v4i, qreg[ks]);
  }
  // rows[] ready, and (fused) set 0's slice in LDS (written through LDS only)
  if (kFuse) barrier_lds(); else __syncthreads();
  if (!kFuse) load_q();

  // MXFP8: raw tiles at smem, the set's expanded bf16 tile after them, then
  // the scales of the round's 128 rows
  unsigned char *cvt = smem + kMaxTiles * kMxRawBytes + set * kTileBytes;
  uint8_t *scl = (uint8_t *)(smem + kMaxTiles * kMxRawBytes + 2 * kTileBytes);
  constexpr int kSclPer = (kMlaRowsPerSplit * 9 + 511) / 512;  // two-byte scale words per thread

  v4f acc[kCt];
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) acc[ct] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  const float scale2 = a.tau * kLog2e;  // logits kept in the exp2 domain
  // V^T read bases: lane (g, c16) reads rows vr, vr + 16, chunk 2 ct + q at
  // sub-offset vsub; for ct = 4 m + i the address is base[i] + 128 m
  const int vr = 4 * g + (c16 >> 2);
  const int q = (c16 & 3) >> 1, vsub = (c16 & 1) * 8;

#pragma unroll
  for (int rd = 0; rd < R; ++rd) {
    if (rd >= rounds) break;  // uniform over the workgroup
    if (rd > 0) barrier_lds();  // every wave is done with the previous round's tiles
    const int32_t *rrows = rows + rd * kMlaRowsPerSplit;
    const int ntiles = (min(kMlaRowsPerSplit, nrows - rd * kMlaRowsPerSplit) + kTile - 1) / kTile;
    // validity of the round's 128 rows as two wave-wide bit masks (rows past
    // nrows are -1)
    const uint64_t valid01 = __ballot(rrows[lane] >= 0);
    const uint64_t valid23 = __ballot(rrows[64 + lane] >= 0);
    uint32_t sreg[kSclPer];
    if (kMx) {
      // scales as 9 two-byte words per row, loaded without branches (unselected
      // rows and padding read the zero block) and replaced by 2^0 afterwards
  #pragma unroll
      for (int j = 0; j < kSclPer; ++j) {
        const int i = tid + 512 * j;
        const int64_t gr = i < kMlaRowsPerSplit * 9 ? (int64_t)rrows[i / 9] : -1;
        const uint16_t *src = gr >= 0 ? (const uint16_t *)(a.kv_scale + gr * kScales + 2 * (i % 9))
                                      : (const uint16_t *)g_zero16;
        sreg[j] = *src;
        if (gr < 0) sreg[j] = 0x7F7Fu;
      }
    }
    // gather: the set's 256 threads copy its tiles set and set + 2 (tiles past
    // ntiles read the zero block, so every thread issues the same number of
    // copies a tile). bf16: rows land swizzled in their tile; MXFP8: the raw
    // 576-byte rows land in order (36 chunks each) and are expanded below.
    auto issue_tile = [&](const int32_t *rrows, int ntiles, int tt) {
      if (!kMx) {
        unsigned char *tbase = smem + tt * kTileBytes;
        int64_t gr[kBfDma];
  #pragma unroll
        for (int j = 0; j < kBfDma; ++j)
          gr[j] = tt < ntiles ? rrows[tt * kTile + (j * 256 + st) / kRowChunks] : -1;
  #pragma unroll
        for (int j = 0; j < kBfDma; ++j) {
          const int c = j * 256 + st;
          const int r = c / kRowChunks;
          const int col = (c - r * kRowChunks) ^ row_swz(r);
          const void *src = gr[j] >= 0 ? (const void *)((const uint8_t *)a.kv + (int64_t)gr[j] * (kD * 2) + col * 16)
                                       : (const void *)g_zero16;
          dma16(src, tbase + (j * 256 + (wave & 3) * 64) * 16);
        }
      } else {
        unsigned char *tbase = smem + tt * kMxRawBytes;
        int64_t gr[kMxDma];
  #pragma unroll
        for (int j = 0; j < kMxDma; ++j) {
          const int c = j * 256 + st;  // raw chunk slot: row c / 36, 16 values
          gr[j] = (c < kMxChunks && tt < ntiles) ? rrows[tt * kTile + c / 36] : -1;
        }
  #pragma unroll
        for (int j = 0; j < kMxDma; ++j) {
          const int c = j * 256 + st;
          const int r = c / 36;
          const void *src = gr[j] >= 0 ? (const void *)((const uint8_t *)a.kv + (int64_t)gr[j] * kD + (c - r * 36) * 16)
                                       : (const void *)g_zero16;
          dma16(src, tbase + (j * 256 + (wave & 3) * 64) * 16);
        }
      }
    };
    // both tiles of the set at once: with 8 waves issuing, the gather runs near
    // the random-row rate of the memory system. From the second round on, tile
    // `set` was requested during the previous round (see below).
    if (rd == 0) issue_tile(rrows, ntiles, set);
    if (kFuse && rd == 0) {
      if (set == 1) {
#pragma unroll
        for (int ks = 0; ks < kKsteps; ++ks) qreg[ks] = as_v8bf(*(const v4i *)(qx + ks * 1024));
      }
      barrier_lds();  // every wave is past the exchange area before tiles 2 and 3 (or their expansion) fill it
    }
    issue_tile(rrows, ntiles, set + 2);
    if (kMx) {
  #pragma unroll
      for (int j = 0; j < kSclPer; ++j) {
        const int i = tid + 512 * j;
        if (i < kMlaRowsPerSplit * 9) *(uint16_t *)(scl + (i / 9) * kScales + 2 * (i % 9)) = (uint16_t)sreg[j];
      }
    }

  #pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 0) wait_vmcnt<kMx ? kMxDma : kBfDma>(); else wait_vmcnt<0>();
      barrier_lds();  // tiles 2u and 2u + 1 have landed (MXFP8: and the scales; u = 1: the set's expanded tile is free)
      if (u == 1 && rd + 1 < rounds) {
        // every wave is past tile `set` of this round (its reads, and for
        // MXFP8 its expansion, came before this barrier): the next round's
        // tile `set` is requested now and lands during this tile's arithmetic
        const int32_t *nrows_ = rows + (rd + 1) * kMlaRowsPerSplit;
        issue_tile(nrows_, (min(kMlaRowsPerSplit, nrows - (rd + 1) * kMlaRowsPerSplit) + kTile - 1) / kTile, set);
      }
      const int tt = set + 2 * u;
      const unsigned char *tile = smem + tt * kTileBytes;
      if (kMx) {
        // the set's 256 threads expand raw tile tt into the set's bf16 tile,
        // each 16-value chunk with the E8M0 scale of its 32-channel block
        if (tt < ntiles) {
          const unsigned char *raw = smem + tt * kMxRawBytes;
          for (int c = st; c < kMxChunks; c += 256) {
            const int r = c / 36, blk = c - r * 36;  // 16 values = channels blk*16 ..
            const v4i v = *(const v4i *)(raw + c * 16);
            const float sc = e8m0_to_f32(scl[(tt * kTile + r) * kScales + (blk >> 1)]);
            const uint32_t w4[4] = {(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
            uint32_t o[8];
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              o[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w4[i], sc, false));
              o[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w4[i], sc, true));
            }
            *(v4i *)(cvt + swz(r, 2 * blk) * 16) = (v4i){(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
            *(v4i *)(cvt + swz(r, 2 * blk + 1) * 16) = (v4i){(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
          }
        }
        barrier_lds();  // the set's expanded tile is complete
        tile = cvt;
      }
      if (tt >= ntiles) continue;  // uniform over the wave; no barrier skipped
      const uint32_t tvalid = (uint32_t)((tt < 2 ? valid01 : valid23) >> (32 * (tt & 1)));
      if (tvalid == 0u) continue;  // no selected row in this tile (uniform)
      // the two 16-row halves are independent accumulation chains, interleaved
      // so that consecutive MFMAs do not wait on each other
      v4f sv[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  #pragma unroll
      for (int ks = 0; ks < kKsteps; ++ks)
  #pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          sv[rt] = mfma_bf16(as_v8bf(*(const v4i *)(tile + swz(rt * 16 + c16, 4 * ks + g) * 16)), qreg[ks], sv[rt]);
      float lg[8];
      float mt = -INFINITY;
  #pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool ok = (tvalid >> ((j >> 2) * 16 + 4 * g + (j & 3))) & 1u;
        lg[j] = ok ? sv[j >> 2][j & 3] * scale2 : -INFINITY;
        mt = fmaxf(mt, lg[j]);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      if (!(mt > -INFINITY)) continue;  // no selected row in this tile (uniform over heads)
      if (__any(mt > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = exp2f(m_run - m_new);
        l_run *= alpha;
  #pragma unroll
        for (int ct = 0; ct < kCt; ++ct) acc[ct] *= alpha;
        m_run = m_new;
      }
      float p[8], ps = 0.0f;
  #pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = exp2f(lg[j] - m_run);
        ps += p[j];
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      l_run += ps;
      v8bf pb;
  #pragma unroll
      for (int j = 0; j < 8; ++j) pb[j] = (__bf16)p[j];
      int voff[4];
  #pragma unroll
      for (int i = 0; i < 4; ++i) voff[i] = (vr * kRowChunks + ((2 * i + q) ^ row_swz(vr))) * 16 + vsub;
      {
        pv_block_b<0>(tile, voff, pb, acc);
        pv_block_b<1>(tile, voff, pb, acc);
        pv_block_b<2>(tile, voff, pb, acc);
        pv_block_b<3>(tile, voff, pb, acc);
        pv_block_b<4>(tile, voff, pb, acc);
        pv_block_b<5>(tile, voff, pb, acc);
        pv_block_b<6>(tile, voff, pb, acc);
        pv_block_b<7>(tile, voff, pb, acc);
      }
    }

  }  // rounds

  // merge the two sets through LDS (the tile area is free now): set 0 finishes
  // channel tiles 0..15 and set 1 channel tiles 16..31, each with the other
  // set's half of the accumulators
  barrier_lds();
  v4f *xch = (v4f *)smem;                              // [hg][ct][lane]
  float2 *mlx = (float2 *)(smem + 4 * kCt * 64 * 16);  // [set][hg][lane]
  // (register indices stay compile-time constants: one branch per set)
  if (set == 0) {
#pragma unroll
    for (int ct = kCt / 2; ct < kCt; ++ct) xch[(hg * kCt + ct) * 64 + lane] = acc[ct];
  } else {
#pragma unroll
    for (int ct = 0; ct < kCt / 2; ++ct) xch[(hg * kCt + ct) * 64 + lane] = acc[ct];
  }
  mlx[(set * 4 + hg) * 64 + lane] = make_float2(m_run, l_run);
  barrier_lds();
  const float2 other = mlx[((1 - set) * 4 + hg) * 64 + lane];
  const float m = fmaxf(m_run, other.x);
  const float sa = m > -INFINITY ? exp2f(m_run - m) : 0.0f;
  const float sb = m > -INFINITY ? exp2f(other.x - m) : 0.0f;
  const float l = l_run * sa + other.y * sb;
  uint2 *pdst = (uint2 *)opart + ((((size_t)t * S + split) * 4 + hg) * kCt) * 64 + lane;
  auto finish = [&](int ct) {
    const v4f b = xch[(hg * kCt + ct) * 64 + lane];
    const v4f o = acc[ct] * sa + b * sb;
    const uint32_t lo = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
    const uint32_t hi = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
    // streamed past the caches: the combine kernel reads the partials once,
    // from another XCD as often as not (measured: 1 us less per split pass)
    __builtin_nontemporal_store((v2u){lo, hi}, (v2u *)&pdst[ct * 64]);
  };
  if (set == 0) {
#pragma unroll
    for (int ct = 0; ct < kCt / 2; ++ct) finish(ct);
  } else {
#pragma unroll
    for (int ct = kCt / 2; ct < kCt; ++ct) finish(ct);
  }
  if (set == 0 && g == 0) ml[((size_t)t * S + split) * kH + head] = make_float2(m, l);
}

// --------------------------------------------------------------------------
// Whole-query kernel (bf16 rows, contiguous cache, many more queries than
// CUs, e.g. a prefill chunk). One workgroup per CU takes a run of whole
// queries and streams every 32-row tile of them through one ring of four LDS
// slots, across query boundaries, so the gather never restarts. All 8 waves
// work on the same tile: wave (hg, half) scores tile rows 16 half .. 16 half
// + 15 for heads 16 hg .. 16 hg + 15 over the full 576 dims and swaps the
// result with its partner wave through LDS, so both hold S for all 32 rows;
// both then run the same online softmax and accumulate O for channels
// 256 half .. 256 half + 255. A query's output is normalised, gated and
// written at its last tile: no partials and no combine pass.
//
// The ring is refilled two tiles at a time: at every even tile j all 512
// threads copy tiles j + 2 and j + 3 (9 16-byte copies per thread), so the
// number of copies in flight behind any tile is fixed and the waits are
// compile-time constants. The selected positions of each group of 128 rows
// (a "chunk", 4 tiles) are brought into LDS by two waves with the same kind
// of copy, two chunks ahead, and turned into cache rows one chunk ahead.
// --------------------------------------------------------------------------
constexpr int kWqSlots = 4;
constexpr int kWqMaxQ = 64;  // queries one workgroup takes
constexpr size_t kWqSmem = (size_t)kWqSlots * kTileBytes + 8 * 64 * 16;  // the ring, then the S exchange
static_assert(kWqSmem + 2 * 128 * 4 * 2 + kWqMaxQ * 8 <= 160 * 1024, "LDS of k_mla_wq");

template <bool kGateBf16>
__global__ __launch_bounds__(512) void k_mla_wq(MlaArgs a, int qpw) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];  // the tile ring
  __shared__ int32_t rowsbuf[2][128];                                   // cache rows of two chunks
  __shared__ __attribute__((aligned(16))) int32_t posbuf[2][128];       // positions of two chunks
  __shared__ int2 qmeta[kWqMaxQ];                                       // (row of position 0, length)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave & 3, half = wave >> 2;
  const int g = lane >> 4, c16 = lane & 15;
  const int t0 = blockIdx.x * qpw;
  const int nq = min(qpw, a.T - t0);
  const int k = a.k;
  const int C = (k + 127) / 128;  // chunks per query
  const int NT = 4 * C;           // tiles per query (tiles past k hold no row)
  const int N = nq * NT;          // tiles of the workgroup
  const int NC = nq * C;          // chunks of the workgroup
  const int head = hg * 16 + c16;
  v4f *xs = (v4f *)(smem + kWqSlots * kTileBytes);  // S of each wave's 16 rows, after the ring

  // chunk d -> query slot d / C, rows 128 (d % C) ..; the position of entry i
  auto pos_src = [&](int d, int i) {
    const int qi = d / C, c = d - qi * C;
    const int e = min(128 * c + i, k - 1);  // entries past k: any valid address (masked below)
    return a.topk_idx + (size_t)(t0 + qi) * k + e;
  };
  // positions -> cache rows for chunk d (threads 0..127), from posbuf[d & 1]
  auto convert = [&](int d) {
    if (tid < 128) {
      const int qi = d / C, c = d - qi * C;
      const int2 qm = qmeta[qi];
      const int32_t pos = posbuf[d & 1][tid];
      rowsbuf[d & 1][tid] = (128 * c + tid < k && pos >= 0 && pos < qm.y) ? qm.x + pos : -1;
    }
  };
  // copies of tiles j and j + 1 (both in the ring): chunk index c = u * 512 +
  // tid of the pair, c < 2304 in tile j; rows past the selection read zeros
  // (a wave's 64 chunks never straddle the two tiles: 2304 = 36 x 64, so
  // the tile and the LDS destination are uniform over the wave)
  static_assert((kTile * kRowChunks) % 64 == 0, "a wave's copies stay in one tile");
  auto issue_pair = [&](int j) {
    // (the lane index is made opaque here so that the compiler recomputes the
    // 9 addresses per call instead of keeping them in registers all along)
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int u = 0; u < 9; ++u) {
      const int cw = u * 512 + wave * 64;  // the wave's first chunk of the pair
      const int second = cw >= kTile * kRowChunks ? 1 : 0;
      const int tt = j + second;
      const int cb = cw - second * kTile * kRowChunks;  // ... within tile tt
      const int cc = cb + ln;
      const int r = cc / kRowChunks;
      const int col = (cc - r * kRowChunks) ^ row_swz(r);
      const int32_t gr = rowsbuf[(tt >> 2) & 1][(tt & 3) * kTile + r];
      const void *src = gr >= 0 ? (const void *)((const uint8_t *)a.kv + (int64_t)gr * (kD * 2) + col * 16)
                                : (const void *)g_zero16;
      dma16(src, smem + (tt & (kWqSlots - 1)) * kTileBytes + cb * 16);
    }
  };

  // ---- prologue: query metadata, rows of chunks 0 and 1, query slice of the
  // first query, copies of tiles 0 and 1
  int2 qm0 = make_int2(0, 0);
  if (tid < nq) {
    int64_t start;
    const int L = seq_len_clipped(a.meta, a.meta.q_seq[t0 + tid], &start);
    qm0 = make_int2((int32_t)start, L);
  }
  int32_t p0 = -1;
  if (tid < 256 && (tid >> 7) < NC) p0 = *pos_src(tid >> 7, tid & 127);
  if (tid < nq) qmeta[tid] = qm0;
  if (tid < 256) posbuf[tid >> 7][tid & 127] = p0;
  __syncthreads();
  convert(0);
  if (NC > 1) convert(1);
  v8bf qreg[kKsteps];
  auto load_q = [&](int qi) {
    const uint8_t *qh = (const uint8_t *)a.q + ((size_t)(t0 + qi) * kH + head) * kD * 2;
#pragma unroll
    for (int ks = 0; ks < kKsteps; ++ks) qreg[ks] = as_v8bf(*(const v4i *)(qh + (ks * 32 + 8 * g) * 2));
  };
  load_q(0);
  __syncthreads();  // rowsbuf of chunks 0 and 1
  // the slice is waited for here and after each reload below: a load still
  // in flight at the loop's first score MFMA would make the compiler wait for
  // every copy in flight there, in every iteration
  wait_vmcnt<0>();
  issue_pair(0);

  v4f acc[kCt / 2];
#pragma unroll
  for (int ct = 0; ct < kCt / 2; ++ct) acc[ct] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  const float scale2 = a.tau * kLog2e;
  const int vr = 4 * g + (c16 >> 2);
  const int qq = (c16 & 3) >> 1, vsub = (c16 & 1) * 8;
  int voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = (vr * kRowChunks + ((2 * i + qq) ^ row_swz(vr))) * 16 + vsub;
  const bool out_bf16 = a.out_dtype == SGA_BF16;

  for (int j = 0; j < N; ++j) {
    // tile j has landed: at even j it is the older tile of the newest pair
    // (5 or 4 of this thread's 9 copies of that pair belong to tile j + 1);
    // at odd j the pair of tiles j + 1, j + 2 was issued after it
    if (j & 1) {
      wait_vmcnt<9>();
    } else if (tid < 256) {
      wait_vmcnt<4>();
    } else {
      wait_vmcnt<5>();
    }
    barrier_lds();  // tile j (and the positions copied with it) visible; tile j - 1 and xs done
    if ((j & 1) == 0) {
      const int e = j >> 2;
      if ((j & 3) == 0 && j > 0 && e + 1 < NC) convert(e + 1);  // rows of chunk e + 1 (positions copied 2 tiles ago)
      if ((j & 3) == 2 && wave < 2 && e + 2 < NC) {
        // positions of chunk e + 2, two chunks ahead; older than the pair below
        __builtin_amdgcn_global_load_lds(pos_src(e + 2, wave * 64 + lane), (lds_void *)&posbuf[e & 1][wave * 64], 4,
                                         0, 0);
      }
      if (j + 2 < N) issue_pair(j + 2);
    }
    const int qi = j / NT, tt = j - qi * NT;
    const unsigned char *tile = smem + (j & (kWqSlots - 1)) * kTileBytes;
    const uint32_t tvalid = (uint32_t)__ballot(lane < kTile && rowsbuf[(j >> 2) & 1][(j & 3) * kTile + (lane & 31)] >= 0);
    const bool last = tt == NT - 1;
    if (tvalid != 0u) {  // uniform over the workgroup
      v4f sv[2];
      v4f own = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kKsteps; ++ks)
        own = mfma_bf16(as_v8bf(*(const v4i *)(tile + swz(16 * half + c16, 4 * ks + g) * 16)), qreg[ks], own);
      xs[wave * 64 + lane] = own;
      barrier_lds();
      const v4f other = xs[(wave ^ 4) * 64 + lane];
      sv[0] = half ? other : own;
      sv[1] = half ? own : other;
      float lg[8];
      float mt = -INFINITY;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const bool ok = (tvalid >> ((jj >> 2) * 16 + 4 * g + (jj & 3))) & 1u;
        lg[jj] = ok ? sv[jj >> 2][jj & 3] * scale2 : -INFINITY;
        mt = fmaxf(mt, lg[jj]);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      if (__any(mt > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int ct = 0; ct < kCt / 2; ++ct) acc[ct] *= alpha;
        m_run = m_new;
      }
      float p[8], ps = 0.0f;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        p[jj] = exp2f(lg[jj] - m_run);
        ps += p[jj];
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      l_run += ps;
      v8bf pb;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) pb[jj] = (__bf16)p[jj];
      const unsigned char *vt = tile + half * 512;  // this wave's 256 channels
      pv_block_ring<0>(vt, voff, pb, acc);
      pv_block_ring<1>(vt, voff, pb, acc);
      pv_block_ring<2>(vt, voff, pb, acc);
      pv_block_ring<3>(vt, voff, pb, acc);
    }
    if (last) {
      // the query's output: O / l, gated, and its log-sum-exp (R11: none
      // selected -> 0 and -inf)
      const int t = t0 + qi;
      const bool any = l_run > 0.0f;
      const float inv = any ? 1.0f / l_run : 0.0f;
      const size_t ob = ((size_t)t * kH + head) * kDc + (size_t)(256 * half + 4 * g);
      uint2 graw[kCt / 2];
      if (a.gate && kGateBf16) {
#pragma unroll
        for (int ct = 0; ct < kCt / 2; ++ct) graw[ct] = *(const uint2 *)((const uint16_t *)a.gate + ob + 16 * ct);
      }
      // (all outputs are formed in place first and stored afterwards)
#pragma unroll
      for (int ct = 0; ct < kCt / 2; ++ct) {
        float y[4] = {acc[ct][0] * inv, acc[ct][1] * inv, acc[ct][2] * inv, acc[ct][3] * inv};
        if (a.gate) {
          float gv[4];
          if (kGateBf16) {
            gv[0] = bf16_bits_to_f32(graw[ct].x & 0xFFFFu);
            gv[1] = bf16_bits_to_f32(graw[ct].x >> 16);
            gv[2] = bf16_bits_to_f32(graw[ct].y & 0xFFFFu);
            gv[3] = bf16_bits_to_f32(graw[ct].y >> 16);
          } else {
            const v4f gf = *(const v4f *)((const float *)a.gate + ob + 16 * ct);
#pragma unroll
            for (int i = 0; i < 4; ++i) gv[i] = gf[i];
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) y[i] *= sigmoidf_exact_ends(gv[i]);
        }
        acc[ct] = (v4f){y[0], y[1], y[2], y[3]};
      }
      if (out_bf16) {
#pragma unroll
        for (int ct = 0; ct < kCt / 2; ++ct) {
          const uint32_t lo = f32_to_bf16_bits(acc[ct][0]) | (f32_to_bf16_bits(acc[ct][1]) << 16);
          const uint32_t hi = f32_to_bf16_bits(acc[ct][2]) | (f32_to_bf16_bits(acc[ct][3]) << 16);
          *(uint2 *)((uint16_t *)a.out + ob + 16 * ct) = make_uint2(lo, hi);
        }
      } else {
#pragma unroll
        for (int ct = 0; ct < kCt / 2; ++ct) *(v4f *)((float *)a.out + ob + 16 * ct) = acc[ct];
      }
#pragma unroll
      for (int ct = 0; ct < kCt / 2; ++ct) acc[ct] = (v4f){0.f, 0.f, 0.f, 0.f};
      if (a.lse && half == 0 && g == 0) a.lse[(size_t)t * kH + head] = any ? m_run / kLog2e + __logf(l_run) : -INFINITY;
      m_run = -INFINITY;
      l_run = 0.0f;
      // the slice of the next query (loaded unconditionally, the last query's
      // again at the end, so that the old slice is dead during the output)
      asm volatile("" ::: "memory");
      load_q(min(qi + 1, nq - 1));
      wait_vmcnt<0>();
    }
  }
}

constexpr int kMaxSplits = 2048 / kMlaRowsPerSplit;
constexpr int kCombCt = 4;  // channel tiles per combine workgroup (256 threads)

// One workgroup per (query, head group of 16, 4 channel tiles); thread (ct,
// lane) owns the same register slot the split kernel stored, so every partial
// load of a wave is 512 contiguous bytes. kS > 0 fixes the split count at
// compile time (all loads issue before the first use); kS = 0 takes it from S.
template <int kS>
__global__ __launch_bounds__(64 * kCombCt) void k_mla_combine(MlaArgs a, const uint16_t *__restrict__ opart,
                                                              const float2 *__restrict__ ml, int S) {
  if (kS > 0) S = kS;
  const int ct = blockIdx.x * kCombCt + (threadIdx.x >> 6);
  const int wave = blockIdx.y, t = blockIdx.z;
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
  const int h = wave * 16 + c16;
  const int c = ct * 16 + 4 * g;
  const size_t oi = ((size_t)t * kH + h) * kDc + c;
  // gate logits first, raw: their loads overlap the partial loads below and
  // are only decoded after them
  const bool gate_bf16 = a.gate_dtype == SGA_BF16;
  v4i graw = {0, 0, 0, 0};
  if (a.gate) {
    if (gate_bf16) {
      const uint2 gb = *(const uint2 *)((const uint16_t *)a.gate + oi);
      graw.x = (int)gb.x;
      graw.y = (int)gb.y;
    } else {
      graw = *(const v4i *)((const float *)a.gate + oi);
    }
  }
  constexpr int kN = kS > 0 ? kS : kMaxSplits;
  float2 st[kN];
  uint2 xb[kN];
  const uint2 *src = (const uint2 *)opart + ((((size_t)t * S) * 4 + wave) * kCt + ct) * 64 + lane;
  const float2 *msrc = ml + (size_t)t * S * kH + h;
  if constexpr (kS > 0 && kS * 16 <= 64 * kCombCt) {
    // the (m, l) pairs of the workgroup's 16 heads are loaded once, one per
    // thread, and shared through LDS (every lane would otherwise load all kS)
    __shared__ float2 s_ml[kS * 16];
    const int tid = threadIdx.x;
    float2 mine = make_float2(0.f, 0.f);
    if (tid < kS * 16) mine = ml[((size_t)t * S + tid / 16) * kH + wave * 16 + (tid & 15)];
#pragma unroll
    for (int s = 0; s < kN; ++s) xb[s] = src[(size_t)s * 4 * kCt * 64];
    if (tid < kS * 16) s_ml[tid] = mine;
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kN; ++s) st[s] = s_ml[s * 16 + c16];
  } else {
#pragma unroll
    for (int s = 0; s < kN; ++s) {
      if (kS > 0 || s < S) {
        st[s] = msrc[(size_t)s * kH];
        xb[s] = src[(size_t)s * 4 * kCt * 64];
      }
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kN; ++s)
    if (kS > 0 || s < S) M = fmaxf(M, st[s].x);
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (M > -INFINITY) {
    float wsum = 0.0f;
#pragma unroll
    for (int s = 0; s < kN; ++s) {
      if ((kS > 0 || s < S) && st[s].x > -INFINITY) {
        const float wgt = exp2f(st[s].x - M);
        wsum = fmaf(wgt, st[s].y, wsum);
        o[0] = fmaf(wgt, bf16_bits_to_f32(xb[s].x & 0xFFFFu), o[0]);
        o[1] = fmaf(wgt, bf16_bits_to_f32(xb[s].x >> 16), o[1]);
        o[2] = fmaf(wgt, bf16_bits_to_f32(xb[s].y & 0xFFFFu), o[2]);
        o[3] = fmaf(wgt, bf16_bits_to_f32(xb[s].y >> 16), o[3]);
      }
    }
    const float inv = 1.0f / wsum;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] *= inv;
    lse = M / kLog2e + __logf(wsum);
  }
  float y[4] = {o[0], o[1], o[2], o[3]};
  if (a.gate) {
    float gv[4];
    if (gate_bf16) {
      gv[0] = bf16_bits_to_f32((uint32_t)graw.x & 0xFFFFu);
      gv[1] = bf16_bits_to_f32((uint32_t)graw.x >> 16);
      gv[2] = bf16_bits_to_f32((uint32_t)graw.y & 0xFFFFu);
      gv[3] = bf16_bits_to_f32((uint32_t)graw.y >> 16);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) gv[i] = __int_as_float(graw[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] *= sigmoidf_exact_ends(gv[i]);
  }
  if (a.out_dtype == SGA_BF16) {
    const uint32_t lo = f32_to_bf16_bits(y[0]) | (f32_to_bf16_bits(y[1]) << 16);
    const uint32_t hi = f32_to_bf16_bits(y[2]) | (f32_to_bf16_bits(y[3]) << 16);
    *(uint2 *)((uint16_t *)a.out + oi) = make_uint2(lo, hi);
  } else {
    *(v4f *)((float *)a.out + oi) = (v4f){y[0], y[1], y[2], y[3]};
  }
  if (a.lse && ct == 0 && g == 0) a.lse[(size_t)t * kH + h] = lse;
}

}  // namespace

hipError_t launch_mla_f32(const MlaArgs &a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_mla_f32, dim3(a.H, a.T), dim3(kF32Block), 0, s, a);
  return hipGetLastError();
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int mla_splits(int k) { return (k + kMlaRowsPerSplit - 1) / kMlaRowsPerSplit; }

// Rounds of 128 rows per split workgroup (R) and splits per query (S) of the
// 8-wave split kernel: the fewest rounds that fit all workgroups on the
// chip's CUs at once (one per CU: the tiles fill its LDS): 1, 2 or 4.
// More rounds mean fewer partials to write and combine, and no second wave of
// workgroups waiting for a CU.
static void mla_plan(int T, int k, int *R, int *S) {
  const int cus = device_cu_count();
  int r = 1;
  while (r < kMaxRounds && (int64_t)T * ((k + r * kMlaRowsPerSplit - 1) / (r * kMlaRowsPerSplit)) > cus) r *= 2;
  *R = r;
  *S = (k + *R * kMlaRowsPerSplit - 1) / (*R * kMlaRowsPerSplit);
}

size_t mla_split_ws_bytes(int T, int k) {
  size_t S = (size_t)mla_splits(k);
  return align256((size_t)T * S * kH * kDc * 2) + align256((size_t)T * S * kH * sizeof(float2));
}

bool mla_fuse_finish(int T, int k) {
  // With more split workgroups than CUs, the repeated top-k finish in every
  // split workgroup of a query costs more than the finish kernel it replaces
  // (prefill: 4,096 queries x 4 splits, 0.35 ms more).
  int R, S;
  mla_plan(T, k, &R, &S);
  return (int64_t)T * S <= device_cu_count();
}

template <bool kMx, int R, bool kFuse, bool kPaged>
static void launch_split8(const MlaArgs &a, uint16_t *opart, float2 *ml, int S, hipStream_t s) {
  const size_t smem = kMx ? kMx8Smem : kBfSmem;
  // one-time set-up per instance (a function-local static is initialised
  // exactly once, also when several host threads arrive together)
  static const bool attr = [smem] {
    (void)hipFuncSetAttribute((const void *)k_mla_split8<kMx, R, kFuse, kPaged>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    (void)hipGetLastError();
    return true;
  }();
  (void)attr;
  hipLaunchKernelGGL((k_mla_split8<kMx, R, kFuse, kPaged>), dim3(S * a.T), dim3(512), smem, s, a, opart, ml, S);
}

// The whole-query kernel takes bf16 rows in the contiguous layout when there
// are at least two queries per CU (and so no fused top-k finish).
bool mla_whole_query_path(int T, int kv_dtype, int page_shift) {
  return kv_dtype == SGA_BF16 && page_shift == 0 && (int64_t)T >= 2LL * device_cu_count();
}

static hipError_t launch_wq(const MlaArgs &a, hipStream_t s) {
  static const bool attr = [] {
    (void)hipFuncSetAttribute((const void *)k_mla_wq<true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kWqSmem);
    (void)hipFuncSetAttribute((const void *)k_mla_wq<false>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kWqSmem);
    (void)hipGetLastError();
    return true;
  }();
  (void)attr;
  const int cus = device_cu_count();
  const int qpw = std::min((a.T + cus - 1) / cus, kWqMaxQ);
  const dim3 grid((a.T + qpw - 1) / qpw);
  if (a.gate_dtype == SGA_BF16)
    hipLaunchKernelGGL(k_mla_wq<true>, grid, dim3(512), kWqSmem, s, a, qpw);
  else
    hipLaunchKernelGGL(k_mla_wq<false>, grid, dim3(512), kWqSmem, s, a, qpw);
  return hipGetLastError();
}

template <bool kMx, bool kFuse, bool kPaged>
static void launch_split8_rp(const MlaArgs &a, uint16_t *opart, float2 *ml, int R, int S, hipStream_t s) {
  if (R == 4)
    launch_split8<kMx, 4, kFuse, kPaged>(a, opart, ml, S, s);
  else if (R == 2)
    launch_split8<kMx, 2, kFuse, kPaged>(a, opart, ml, S, s);
  else
    launch_split8<kMx, 1, kFuse, kPaged>(a, opart, ml, S, s);
}

template <bool kMx, bool kFuse>
static void launch_split8_r(const MlaArgs &a, uint16_t *opart, float2 *ml, int R, int S, hipStream_t s) {
  if (a.meta.page_shift)
    launch_split8_rp<kMx, kFuse, true>(a, opart, ml, R, S, s);
  else
    launch_split8_rp<kMx, kFuse, false>(a, opart, ml, R, S, s);
}

hipError_t launch_mla_split(const MlaArgs &a, void *ws, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (!a.fuse && mla_whole_query_path(a.T, a.kv_dtype, a.meta.page_shift)) return launch_wq(a, s);
  int R, S;
  mla_plan(a.T, a.k, &R, &S);
  uint16_t *opart = (uint16_t *)ws;
  float2 *ml = (float2 *)((char *)ws + align256((size_t)a.T * S * kH * kDc * 2));
  const bool mx = a.kv_dtype == SGA_MXFP8_E4M3FN;
  if (mx && a.fuse)
    launch_split8_r<true, true>(a, opart, ml, R, S, s);
  else if (mx)
    launch_split8_r<true, false>(a, opart, ml, R, S, s);
  else if (a.fuse)
    launch_split8_r<false, true>(a, opart, ml, R, S, s);
  else
    launch_split8_r<false, false>(a, opart, ml, R, S, s);
  return hipGetLastError();
}

hipError_t launch_mla_combine(const MlaArgs &a, const void *ws, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (!a.fuse && mla_whole_query_path(a.T, a.kv_dtype, a.meta.page_shift)) return hipSuccess;  // written whole
  int R, S;
  mla_plan(a.T, a.k, &R, &S);
  const uint16_t *opart = (const uint16_t *)ws;
  const float2 *ml = (const float2 *)((const char *)ws + align256((size_t)a.T * S * kH * kDc * 2));
  const dim3 grid(kCt / kCombCt, 4, a.T), block(64 * kCombCt);
  if (S == kMaxSplits)
    hipLaunchKernelGGL(k_mla_combine<kMaxSplits>, grid, block, 0, s, a, opart, ml, S);
  else if (S == kMaxSplits / 2)
    hipLaunchKernelGGL(k_mla_combine<kMaxSplits / 2>, grid, block, 0, s, a, opart, ml, S);
  else if (S == kMaxSplits / 4)
    hipLaunchKernelGGL(k_mla_combine<kMaxSplits / 4>, grid, block, 0, s, a, opart, ml, S);
  else
    hipLaunchKernelGGL(k_mla_combine<0>, grid, block, 0, s, a, opart, ml, S);
  return hipGetLastError();
}

}  // namespace sga
