/*
 * sga.h -- C ABI of the Sparse Gated Attention (SGA) forward hot path on AMD
 * MI355X (gfx950).
 *
 * SGA is the attention sublayer described on the A.X K2 pages:
 *   - "A.X-K2: a sparse-attention upgrade that costs nothing, trained natively
 *     in FP8", section "Sparse Gated Attention": a small indexer rates each
 *     cached key, 2,048 single positions survive for each query (not
 *     blocks), attention reads only those latent rows, and a per-head
 *     learned gate multiplies the attention result ahead of Wo;
 *   - "SK Telecom Opens A.X K2: 688B Parameters and One Telling Benchmark",
 *     section "Sparse Gated Attention" and its block-diagram caption (the
 *     index scores pick the rows MLA reads; a sigmoid gate on the output);
 *   - "A.X K2 Technical Report", section 2 (an MLA backbone whose heads each
 *     gate their own output) and section 3.4 (Stage 3C: the indexer's selection holds
 *     2,048 positions for each query).
 * The pages print no formula. The operations below implement these readings:
 *   scores  I[t,s] = sum_h w[t,h] * max(0, qI[t,h,:] . kI[s,:])   for s <= p_t
 *   select  S_t    = the k positions of largest I[t,.], ties to the lowest
 *                    position; every position when p_t + 1 <= k
 *   attend  o[t,h] = sum_{s in S_t} softmax_s(tau * q[t,h,:] . kv[s,:]) * kv[s,:Dc]
 *   gate    y[t,h,c] = sigmoid(g[t,h,c]) * o[t,h,c]
 * (absorbed MLA: every head reads the same cached row kv[s] = [c_s | kR_s] of
 * Dc + Dr values; the value is its first Dc = d_latent entries).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers to contiguous row-major arrays,
 *     16-byte aligned. Pointers in sga_problem are device pointers too.
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *     enqueues work on it and returns without synchronising. Device faults, if
 *     any, surface at the caller's next synchronisation.
 *   - The caller owns all memory, including the workspace `ws` (size from
 *     sga_workspace_size). The library allocates no device memory and keeps
 *     no pointer after a call returns. Calls that share a workspace must not
 *     overlap in time.
 *   - Argument errors are returned synchronously as an sga_status before any
 *     work is enqueued; sga_last_error() gives this thread's detail message.
 *     No C++ exception crosses this boundary.
 *   - Sequence metadata lives on the device and is not checked on the host.
 *     Kernels stay inside every buffer whatever it holds: a query's candidate
 *     count is n_t = clamp(q_pos[t] + 1, 0, min(kv_len[b], max_kv_len,
 *     num_kv_rows - kv_start[b])), and a query with an out-of-range q_seq has
 *     n_t = 0. A query with n_t = 0 selects nothing and outputs y = 0 and
 *     lse = -inf.
 *
 * Supported shapes (anything else returns SGA_ERR_UNSUPPORTED)
 *   - fp32 path: q, kv, index q/k all SGA_F32; 1 <= heads <= 64,
 *     d_latent + d_rope <= 1024 (d_latent a multiple of 4), idx_heads * idx_dim
 *     <= 8192, topk <= 4096.
 *   - MI355X path: heads = 64, d_latent = 512, d_rope = 64 with q SGA_BF16 and
 *     kv SGA_BF16 or SGA_MXFP8_E4M3FN; index heads 64 x dim 128 in
 *     SGA_FP8_E4M3FN; 1 <= topk <= 2048.
 *   Gate and output may be SGA_F32 or SGA_BF16 on either path.
 */
#ifndef SGA_H
#define SGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SGA_ABI_VERSION 2

typedef enum sga_status {
  SGA_OK = 0,
  SGA_ERR_INVALID_ARGUMENT = 1, /* NULL pointer, bad size, bad dtype code          */
  SGA_ERR_UNSUPPORTED = 2,      /* valid, but no kernel for this shape/dtype mix   */
  SGA_ERR_WORKSPACE = 3,        /* ws NULL or smaller than sga_workspace_size()    */
  SGA_ERR_DEVICE = 4,           /* HIP runtime error before launching              */
  SGA_ERR_LAUNCH = 5            /* a kernel launch failed                          */
} sga_status;

typedef enum sga_dtype {
  SGA_F32 = 0,          /* IEEE binary32                                              */
  SGA_BF16 = 1,         /* bfloat16                                                   */
  SGA_FP8_E4M3FN = 2,   /* OCP FP8 E4M3FN bytes (bias 7, max 448, no inf)             */
  SGA_MXFP8_E4M3FN = 3  /* E4M3FN bytes + one E8M0 scale byte per 32 consecutive values */
} sga_dtype;

typedef enum sga_op {
  SGA_OP_INDEX = 0, /* sga_index_scores   */
  SGA_OP_TOPK = 1,  /* sga_topk_select    */
  SGA_OP_MLA = 2,   /* sga_sparse_mla_fwd */
  SGA_OP_LAYER = 3, /* sga_layer_fwd      */
  SGA_OP_INDEXER_KL = 4 /* sga_indexer_kl */
} sga_op;

/* Shapes, dtypes and sequence metadata of one call. */
typedef struct sga_problem {
  int32_t num_seqs;      /* B: sequences in the caches                                   */
  int32_t num_q;         /* T: query rows                                                */
  int32_t max_kv_len;    /* host bound on every kv_len[b]; row stride of the score buffer */
  int32_t page_size;     /* 0: contiguous rows (kv_start); else rows in pages (see below) */
  int64_t num_kv_rows;   /* rows in kv, kv_scale and k_idx (at most 2^31 - 1)            */
  int32_t heads;         /* H: attention heads (64)                                      */
  int32_t d_latent;      /* Dc: latent width = value width (512)                          */
  int32_t d_rope;        /* Dr: rotary key width (64)                                     */
  int32_t idx_heads;     /* HI: indexer heads (64)                                        */
  int32_t idx_dim;       /* DI: indexer head width (128)                                  */
  int32_t topk;          /* k: positions kept per query (2048)                            */
  float softmax_scale;   /* tau, applied to q . kv                                         */
  int32_t q_dtype;       /* sga_dtype of q                                                 */
  int32_t kv_dtype;      /* sga_dtype of kv                                                */
  int32_t idx_dtype;     /* sga_dtype of q_idx and k_idx                                   */
  int32_t gate_dtype;    /* sga_dtype of gate logits (ignored when gate is NULL)           */
  int32_t out_dtype;     /* sga_dtype of out                                               */
  const int32_t *q_seq;  /* [T] sequence of each query row                                 */
  const int32_t *q_pos;  /* [T] position of each query row within its sequence             */
  const int64_t *kv_start; /* [B] cache row holding position 0 of each sequence (contiguous
                              layout; ignored, may be NULL, when page_size > 0)          */
  const int32_t *kv_len;   /* [B] cached tokens of each sequence                           */
  const int32_t *block_table; /* [B, max_pages] page of each sequence's positions, or NULL  */
  int32_t max_pages;     /* row length of block_table (0 when page_size is 0)             */
  int32_t reserved0;     /* must be 0                                                    */
} sga_problem;

/*
 * Cache layouts (every entry point that reads kv, kv_scale or k_idx)
 *   - contiguous (page_size = 0): position s of sequence b is cache row
 *     kv_start[b] + s; the sequence's length is clipped to num_kv_rows -
 *     kv_start[b].
 *   - paged (page_size a power of two, 64 <= page_size <= 65536): the caches
 *     are num_kv_rows / page_size pages of page_size rows, and position s of
 *     sequence b is row block_table[b * max_pages + s / page_size] * page_size
 *     + s % page_size (the block table of a paged KV cache; the serving stack
 *     the pages deploy with keeps its cache this way). The sequence's length
 *     is clipped to max_pages * page_size. A page id outside
 *     [0, num_kv_rows / page_size) is an error the library does not detect:
 *     the kernels still read only rows inside the caches, but the results
 *     of every query of that sequence are unspecified. Queries of other
 *     sequences are unaffected. The block table lives on the device and is
 *     not checked on the host.
 */

/* ABI version of the loaded library (SGA_ABI_VERSION). */
int sga_abi_version(void);

/* Static text for a status code. */
const char *sga_status_string(int status);

/* Detail message of this thread's last non-OK return ("" if none). */
const char *sga_last_error(void);

/* Workspace bytes `op` needs for problem `p`, written to *bytes (0 when none is
 * needed). Pure host computation; validates `p` like the op itself. */
sga_status sga_workspace_size(const sga_problem *p, int op, size_t *bytes);

/*
 * Indexer score pass: one score per (query, visible cached key); see the
 * header comment for sources.
 *   q_idx  [T, HI, DI]   idx_dtype (SGA_F32 or SGA_FP8_E4M3FN)
 *   w      [T, HI]       fp32 per-(query, head) weights
 *   k_idx  [num_kv_rows, DI] idx_dtype, one key per cached token, shared by all
 *                        index heads; sequence b owns rows kv_start[b] + s
 *   scores [T, max_kv_len] fp32 output: scores[t, s] for s < n_t; entries with
 *                        s >= n_t are left untouched.
 * Arithmetic: fp32 accumulation (FP8 MFMA on the MI355X path). With integer
 * q/k and a dyadic w that keeps every partial sum below 2^24 units of its
 * finest bit, the result is the exact score in any evaluation order.
 * A -0.0 result is stored as +0.0. Needs no workspace.
 */
sga_status sga_index_scores(const sga_problem *p, const void *q_idx, const float *w,
                            const void *k_idx, float *scores, void *stream);

/*
 * Per-query top-k selection: the selector of the "Sparse Gated Attention"
 * section keeps k = 2,048 single positions per query, chosen one by one
 * rather than in blocks.
 *   scores   [T, max_kv_len] fp32, only s < n_t is read
 *   topk_idx [T, topk] int32 output: the selected positions within the
 *            sequence in ascending order; -1 fills the tail when n_t < topk.
 * Order: larger score first, ties to the lower position; -0.0 equals +0.0;
 * every NaN (either sign) orders above +inf and ties with the other NaNs.
 * Exact (radix select on the fp32 bit pattern), so the result is
 * deterministic.
 */
sga_status sga_topk_select(const sga_problem *p, const float *scores, int32_t *topk_idx,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * Sparse MLA over the selected latent rows plus the sigmoid output gate:
 * attention reads only the chosen rows, and each head's output is scaled by
 * its own gate ahead of the Wo projection ("Sparse Gated Attention" section;
 * technical report section 2).
 *   q        [T, H, Dc + Dr]  q_dtype (absorbed query: latent part then rope part)
 *   kv       [num_kv_rows, Dc + Dr] kv_dtype, row = [c_s | kR_s]
 *   kv_scale [num_kv_rows, (Dc + Dr) / 32] E8M0 bytes for SGA_MXFP8_E4M3FN, else NULL
 *   topk_idx [T, topk] int32 positions within the query's sequence; entries
 *            < 0 or >= n_t-clipped cache length are skipped (any order)
 *   gate     [T, H, Dc] gate_dtype logits, or NULL for no gate
 *   out      [T, H, Dc] out_dtype: sigmoid(gate) * softmax-weighted latent sum
 *   lse      [T, H] fp32 log-sum-exp of the scaled logits, or NULL
 * Arithmetic on the MI355X path: bf16 MFMA for q.kv and p.v with fp32
 * accumulation, fp32 online softmax, p rounded to bf16 for p.v; MXFP8 rows
 * are expanded exactly to bf16.
 */
sga_status sga_sparse_mla_fwd(const sga_problem *p, const void *q, const void *kv,
                              const uint8_t *kv_scale, const int32_t *topk_idx,
                              const void *gate, void *out, float *lse, void *ws,
                              size_t ws_bytes, void *stream);

/*
 * The whole path in one call: index scores -> top-k -> sparse MLA -> gate.
 * Arguments as in the three calls above. topk_idx_out [T, topk] and lse [T, H]
 * are optional outputs (NULL to skip). The scores live in the workspace.
 */
sga_status sga_layer_fwd(const sga_problem *p, const void *q_idx, const float *w,
                         const void *k_idx, const void *q, const void *kv,
                         const uint8_t *kv_scale, const void *gate, void *out,
                         int32_t *topk_idx_out, float *lse, void *ws, size_t ws_bytes,
                         void *stream);

/*
 * sga_layer_fwd without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation. Arguments and results are those of
 * sga_layer_fwd minus ws / ws_bytes. The workspace is the library's own
 * static device buffer of SGA_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU that
 * runs it, held until the process ends; the call allocates and frees no
 * device memory. A problem whose sga_workspace_size(p, SGA_OP_LAYER) exceeds
 * it returns SGA_ERR_WORKSPACE before any work is enqueued (16 x 128K and
 * 32 x 32K decode batches with k = 2048 fit; use sga_layer_fwd for larger
 * ones). Every call on one GPU shares that GPU's buffer: calls that overlap
 * in time on one GPU (on different streams or host threads) race, and the
 * caller must serialise them. Nothing in the buffer needs clearing between
 * calls (every kernel writes what it later reads).
 */
#define SGA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
sga_status sga_layer_fwd_noalloc(const sga_problem *p, const void *q_idx, const float *w,
                                 const void *k_idx, const void *q, const void *kv,
                                 const uint8_t *kv_scale, const void *gate, void *out,
                                 int32_t *topk_idx_out, float *lse, void *stream);

/*
 * Cache append: the step before the path in serving, which stores each new
 * token's latent row and index key in the caches' storage formats. MXFP8 is
 * the OCP microscaling FP8 that the A.X K2 Technical Report's FP8 section
 * names (E4M3 elements, one shared scale per 32 consecutive values); the
 * FP8 KV cache is the serving configuration of the inference sweep in the
 * "Sparse Gated Attention" section of "A.X-K2: a sparse-attention upgrade
 * that costs nothing, trained natively in FP8".
 *   p          only num_kv_rows, d_latent, d_rope, idx_dim, kv_dtype and
 *              idx_dtype are read (the sequence metadata may be NULL)
 *   num_tokens N >= 0 new tokens
 *   src_dtype  SGA_F32 or SGA_BF16: element type of kv_new and k_idx_new
 *   kv_new     [N, Dc + Dr] new rows [c | kR], or NULL to write no latent rows
 *   k_idx_new  [N, DI] new index keys, or NULL to write no index keys
 *   slots      [N] int64 cache row of each token. A slot outside
 *              [0, num_kv_rows) drops that token; valid slots must be
 *              distinct (two tokens writing one row race). With a paged
 *              cache the caller maps (sequence, position) to its slot.
 *   kv         [num_kv_rows, Dc + Dr] kv_dtype: SGA_F32, SGA_BF16 or
 *              SGA_MXFP8_E4M3FN (then kv_scale [num_kv_rows, (Dc + Dr) / 32])
 *   k_idx      [num_kv_rows, DI] idx_dtype: SGA_F32 or SGA_FP8_E4M3FN
 * Encodings: fp32 and bf16 sources are stored exactly in fp32 and a bf16
 * source is copied to bf16; fp32 -> bf16 rounds to nearest even (NaN becomes
 * the quiet NaN of its sign). FP8 E4M3FN rounds to nearest even and
 * saturates at +-448; a NaN becomes 0x7F / 0xFF by its sign. An MXFP8 block
 * of 32 values gets the scale 2^(floor(log2 max|v|) - 8), clamped to
 * 2^-127 .. 2^127 (all zeros: 2^-127), and stores v / scale as E4M3FN; a
 * block with an inf or NaN stores scale byte 0xFF and element bytes 0x7F.
 * Index keys are stored unscaled.
 * Requires Dc + Dr and DI to be multiples of 8 (Dc + Dr of 32 for MXFP8) and
 * N * (Dc + Dr + DI) / 8 < 2^31. Rows not named by a valid slot are left
 * untouched. Needs no workspace.
 */
sga_status sga_cache_append(const sga_problem *p, int64_t num_tokens, int src_dtype,
                            const void *kv_new, const void *k_idx_new, const int64_t *slots,
                            void *kv, uint8_t *kv_scale, void *k_idx, void *stream);

/*
 * Indexer KL loss and its gradients, the training side of the indexer ("A.X
 * K2 Technical Report" section 3.4: a KL objective pulls the indexer's
 * scores toward the attention weights, evaluated only on the sparse
 * selection from the first step of that stage; "A.X-K2: a sparse-attention
 * upgrade that costs nothing, trained natively in FP8", section "Sparse
 * Gated Attention"). For query t with the selected positions S_t of a forward pass:
 *   target_s = sum_h exp(tau q[t,h] . kv[s] - lse[t,h]), normalised over S_t
 *   I_s      = sum_h w[t,h] max(0, q_idx[t,h] . k_idx[s])
 *   loss[t]  = sum_s target_s (log target_s - log softmax_S(I)_s)
 *   g_s      = softmax_S(I)_s - target_s          (the target is a constant)
 *   d_w[t,h] = sum_s g_s max(0, z_hs);  d_q_idx[t,h] = sum_s g_s w[t,h] [z_hs > 0] k_idx[s]
 *   d_k_idx[s] += sum_h g_s w[t,h] [z_hs > 0] q_idx[t,h]   (z_hs = q_idx[t,h] . k_idx[s])
 * Arguments: q_idx, w, k_idx, q, kv, kv_scale as in sga_layer_fwd; topk_idx
 * [T, topk] and lse [T, H] are that forward's outputs (topk_idx_out, lse);
 * outputs loss [T], d_w [T, HI], d_q_idx [T, HI, DI] (fp32, written) and
 * d_k_idx [num_kv_rows, DI] (fp32, ADDED to: the caller clears it; the
 * order of the additions is not fixed; no other work may touch d_k_idx
 * while the call runs). Queries without candidates give
 * loss 0 and zero gradients.
 * Shapes: H, HI <= 64, HI * DI <= 8192, Dc + Dr and DI multiples of 8, topk
 * <= 4096, q in LDS (H * (Dc + Dr) bf16 or fp32) within 96 KiB; q SGA_F32 or
 * SGA_BF16, kv SGA_F32, SGA_BF16 or SGA_MXFP8_E4M3FN, index SGA_F32 or
 * SGA_FP8_E4M3FN. Arithmetic: fp32 accumulation throughout. For 64 heads
 * with bf16 q and 576-wide bf16 or MXFP8 rows, the attention logits q . kv
 * run on bf16 MFMA (MXFP8 rows expanded exactly to bf16); with 64 x 128 FP8
 * index tensors, z = q_idx . k_idx runs on bf16 MFMA too (E4M3FN values are
 * exact in bf16), and so do the gradient products d_q_idx and d_k_idx: their
 * fp32 factor g w [z > 0] enters as three bf16 parts whose sum carries its
 * 24 significant bits, so every product is exact and accumulates in fp32.
 * Every other shape, and the softmax, loss and reductions, use the fp32
 * vector ALUs. Workspace: sga_workspace_size(p, SGA_OP_INDEXER_KL).
 */
sga_status sga_indexer_kl(const sga_problem *p, const void *q_idx, const float *w,
                          const void *k_idx, const void *q, const void *kv,
                          const uint8_t *kv_scale, const int32_t *topk_idx, const float *lse,
                          float *loss, float *d_w, float *d_q_idx, float *d_k_idx, void *ws,
                          size_t ws_bytes, void *stream);

/*
 * Phase timing of sga_layer_fwd, for measurement. While enabled, each
 * sga_layer_fwd call on this thread records HIP events on its stream around
 * each phase (0 index scores, 1 top-k, 2 sparse MLA, 3 combine + gate), for up
 * to `max_calls` calls. sga_profile_collect waits for those events, writes the
 * summed milliseconds per phase into ms[0..nphase) and the number of timed
 * calls into *calls, then resets the record. Disable with max_calls = 0.
 */
sga_status sga_profile_enable(int max_calls);
sga_status sga_profile_collect(double *ms, int nphase, int *calls);

/*
 * Streaming-read reference, for measurement: reads `bytes` (a multiple of
 * 8192) from the device buffer `src` (16-byte aligned) with the decode
 * indexer's copy pattern (8 KiB tiles through an LDS ring by LDS-DMA, two
 * 256-thread workgroups per CU, each a contiguous share) and no arithmetic
 * beyond folding the bytes into one word per workgroup, written to `sink`
 * (device, sga_stream_read_sink_words() words). Its bandwidth is what the
 * indexer's copies alone reach on this device.
 */
sga_status sga_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream);
int sga_stream_read_sink_words(void);

#ifdef __cplusplus
}
#endif

#endif /* SGA_H */
