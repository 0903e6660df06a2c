// C ABI of the SGA hot path: argument checks, workspace layout and dispatch.
// The operations and their sources are described in include/sga.h.

#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"

using namespace sga;

namespace {

thread_local std::string g_err;

sga_status fail(sga_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool dtype_ok(int d) { return d >= SGA_F32 && d <= SGA_MXFP8_E4M3FN; }

enum class IdxPath { kF32, kFp8 };
enum class MlaPath { kF32, kBf16, kMx };

struct Plan {
  IdxPath idx = IdxPath::kF32;
  MlaPath mla = MlaPath::kF32;
};

constexpr int kMaxKvLen = 1024 * kTopkChunk;  // 4,194,304 positions per sequence

sga_status check_common(const sga_problem *p) {
  if (!p) return fail(SGA_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (p->reserved0 != 0) return fail(SGA_ERR_INVALID_ARGUMENT, "reserved0 must be 0");
  if (p->num_q < 0 || p->num_seqs < 0 || p->max_kv_len < 0 || p->num_kv_rows < 0)
    return fail(SGA_ERR_INVALID_ARGUMENT, "negative size (num_q=%d num_seqs=%d max_kv_len=%d)",
                p->num_q, p->num_seqs, p->max_kv_len);
  if (p->max_kv_len > kMaxKvLen)
    return fail(SGA_ERR_UNSUPPORTED, "max_kv_len %d exceeds %d", p->max_kv_len, kMaxKvLen);
  // cache rows are addressed with 32-bit ids on the device
  if (p->num_kv_rows > INT32_MAX)
    return fail(SGA_ERR_UNSUPPORTED, "num_kv_rows %lld exceeds 2^31 - 1", (long long)p->num_kv_rows);
  if (p->topk < 1) return fail(SGA_ERR_INVALID_ARGUMENT, "topk must be >= 1 (got %d)", p->topk);
  if (p->num_q > 0 && (!p->q_seq || !p->q_pos))
    return fail(SGA_ERR_INVALID_ARGUMENT, "q_seq / q_pos is NULL");
  if (p->num_seqs > 0 && (!p->kv_len || (p->page_size == 0 && !p->kv_start)))
    return fail(SGA_ERR_INVALID_ARGUMENT, "kv_start / kv_len is NULL");
  if (p->page_size != 0) {
    if (p->page_size < 64 || p->page_size > 65536 || (p->page_size & (p->page_size - 1)))
      return fail(SGA_ERR_INVALID_ARGUMENT, "page_size must be 0 or a power of two in [64, 65536] (got %d)",
                  p->page_size);
    if (p->max_pages < 1) return fail(SGA_ERR_INVALID_ARGUMENT, "max_pages must be >= 1 with pages");
    if (p->num_seqs > 0 && !p->block_table)
      return fail(SGA_ERR_INVALID_ARGUMENT, "block_table is NULL with page_size %d", p->page_size);
  } else if (p->max_pages != 0 || p->block_table) {
    return fail(SGA_ERR_INVALID_ARGUMENT, "block_table / max_pages given without page_size");
  }
  if (!dtype_ok(p->q_dtype) || !dtype_ok(p->kv_dtype) || !dtype_ok(p->idx_dtype) ||
      !dtype_ok(p->gate_dtype) || !dtype_ok(p->out_dtype))
    return fail(SGA_ERR_INVALID_ARGUMENT, "unknown dtype code");
  return SGA_OK;
}

sga_status check_index(const sga_problem *p, Plan *plan) {
  if (p->idx_heads < 1 || p->idx_dim < 1)
    return fail(SGA_ERR_INVALID_ARGUMENT, "idx_heads / idx_dim must be >= 1");
  if (p->idx_dtype == SGA_F32) {
    if (p->idx_heads > 64 || (int64_t)p->idx_heads * p->idx_dim > 8192)
      return fail(SGA_ERR_UNSUPPORTED, "fp32 indexer needs idx_heads <= 64 and heads*dim <= 8192");
    plan->idx = IdxPath::kF32;
    return SGA_OK;
  }
  if (p->idx_dtype == SGA_FP8_E4M3FN) {
    if (p->idx_heads != 64 || p->idx_dim != 128)
      return fail(SGA_ERR_UNSUPPORTED, "FP8 indexer is built for 64 heads x 128 dims (got %d x %d)",
                  p->idx_heads, p->idx_dim);
    plan->idx = IdxPath::kFp8;
    return SGA_OK;
  }
  return fail(SGA_ERR_UNSUPPORTED, "indexer dtype must be SGA_F32 or SGA_FP8_E4M3FN");
}

sga_status check_mla(const sga_problem *p, Plan *plan) {
  if (p->heads < 1 || p->d_latent < 1 || p->d_rope < 0)
    return fail(SGA_ERR_INVALID_ARGUMENT, "heads / d_latent must be >= 1, d_rope >= 0");
  if (!(p->softmax_scale == p->softmax_scale) || p->softmax_scale > 3.0e38f ||
      p->softmax_scale < -3.0e38f)
    return fail(SGA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  if (p->gate_dtype != SGA_F32 && p->gate_dtype != SGA_BF16)
    return fail(SGA_ERR_UNSUPPORTED, "gate dtype must be SGA_F32 or SGA_BF16");
  if (p->out_dtype != SGA_F32 && p->out_dtype != SGA_BF16)
    return fail(SGA_ERR_UNSUPPORTED, "out dtype must be SGA_F32 or SGA_BF16");
  if (p->q_dtype == SGA_F32 && p->kv_dtype == SGA_F32) {
    if (p->heads > 64 || p->d_latent + p->d_rope > 1024 || p->topk > 4096)
      return fail(SGA_ERR_UNSUPPORTED,
                  "fp32 MLA needs heads <= 64, d_latent + d_rope <= 1024, topk <= 4096");
    plan->mla = MlaPath::kF32;
    return SGA_OK;
  }
  if (p->q_dtype == SGA_BF16 && (p->kv_dtype == SGA_BF16 || p->kv_dtype == SGA_MXFP8_E4M3FN)) {
    if (p->heads != 64 || p->d_latent != 512 || p->d_rope != 64)
      return fail(SGA_ERR_UNSUPPORTED, "bf16 MLA is built for 64 heads, d_latent 512, d_rope 64");
    if (p->topk > 2048) return fail(SGA_ERR_UNSUPPORTED, "bf16 MLA supports topk <= 2048");
    plan->mla = p->kv_dtype == SGA_BF16 ? MlaPath::kBf16 : MlaPath::kMx;
    return SGA_OK;
  }
  return fail(SGA_ERR_UNSUPPORTED, "q/kv dtype pair not supported (q=%d kv=%d)", p->q_dtype,
              p->kv_dtype);
}

sga_status check_kl(const sga_problem *p) {
  if (p->heads < 1 || p->heads > 64 || p->idx_heads < 1 || p->idx_heads > 64 || p->idx_dim < 8 ||
      p->idx_heads * p->idx_dim > 8192)
    return fail(SGA_ERR_UNSUPPORTED, "indexer KL needs heads, idx_heads <= 64 and idx_heads*idx_dim <= 8192");
  const int D = p->d_latent + p->d_rope;
  if (p->d_latent < 1 || p->d_rope < 0 || D % 8 || p->idx_dim % 8)
    return fail(SGA_ERR_UNSUPPORTED, "indexer KL needs d_latent + d_rope and idx_dim multiples of 8");
  if (p->topk > 4096) return fail(SGA_ERR_UNSUPPORTED, "indexer KL supports topk <= 4096");
  if (!(p->softmax_scale == p->softmax_scale) || p->softmax_scale > 3.0e38f || p->softmax_scale < -3.0e38f)
    return fail(SGA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  if (p->q_dtype != SGA_F32 && p->q_dtype != SGA_BF16)
    return fail(SGA_ERR_UNSUPPORTED, "indexer KL: q must be SGA_F32 or SGA_BF16");
  if (p->kv_dtype != SGA_F32 && p->kv_dtype != SGA_BF16 && p->kv_dtype != SGA_MXFP8_E4M3FN)
    return fail(SGA_ERR_UNSUPPORTED, "indexer KL: kv must be SGA_F32, SGA_BF16 or SGA_MXFP8_E4M3FN");
  if (p->kv_dtype == SGA_MXFP8_E4M3FN && D % 32)
    return fail(SGA_ERR_UNSUPPORTED, "MXFP8 rows need a multiple of 32 values");
  if (p->idx_dtype != SGA_F32 && p->idx_dtype != SGA_FP8_E4M3FN)
    return fail(SGA_ERR_UNSUPPORTED, "indexer KL: index tensors must be SGA_F32 or SGA_FP8_E4M3FN");
  if ((int64_t)p->heads * D * (p->q_dtype == SGA_BF16 ? 2 : 4) > 96 * 1024 ||
      indexer_kl_smem(p->heads, D, p->idx_heads, p->idx_dim, p->q_dtype) > 160 * 1024)
    return fail(SGA_ERR_UNSUPPORTED, "indexer KL: q of one query must fit 96 KiB");
  return SGA_OK;
}

int64_t score_stride(const sga_problem *p) { return ((int64_t)p->max_kv_len + 63) / 64 * 64; }

sga_status plan_for(const sga_problem *p, int op, Plan *plan) {
  sga_status st = check_common(p);
  if (st != SGA_OK) return st;
  switch (op) {
    case SGA_OP_INDEX:
      return check_index(p, plan);
    case SGA_OP_TOPK:
      return SGA_OK;
    case SGA_OP_MLA:
      return check_mla(p, plan);
    case SGA_OP_LAYER:
      st = check_index(p, plan);
      if (st != SGA_OK) return st;
      return check_mla(p, plan);
    case SGA_OP_INDEXER_KL:
      return check_kl(p);
    default:
      return fail(SGA_ERR_INVALID_ARGUMENT, "unknown op %d", op);
  }
}

size_t mla_ws(const sga_problem *p, const Plan &plan) {
  if (plan.mla == MlaPath::kF32) return 0;
  const int shift = p->page_size ? __builtin_ctz((unsigned)p->page_size) : 0;
  return mla_whole_query_path(p->num_q, p->kv_dtype, shift) ? 0 : mla_split_ws_bytes(p->num_q, p->topk);
}

size_t ws_bytes(const sga_problem *p, int op, const Plan &plan) {
  switch (op) {
    case SGA_OP_INDEX:
      return 0;
    case SGA_OP_TOPK:
      return topk_ws_bytes(p->num_q, p->max_kv_len);
    case SGA_OP_MLA:
      return mla_ws(p, plan);
    case SGA_OP_LAYER:
      return align256((size_t)p->num_q * score_stride(p) * 4) +
             align256((size_t)p->num_q * p->topk * 4) +
             align256(topk_ws_bytes(p->num_q, p->max_kv_len)) + mla_ws(p, plan);
    case SGA_OP_INDEXER_KL:
      return indexer_kl_ws_bytes(p->num_q, p->topk, p->idx_heads, p->idx_dim);
  }
  return 0;
}

SeqMeta meta_of(const sga_problem *p) {
  SeqMeta m;
  m.q_seq = p->q_seq;
  m.q_pos = p->q_pos;
  m.kv_start = p->kv_start;
  m.kv_len = p->kv_len;
  m.num_seqs = p->num_seqs;
  m.max_kv_len = p->max_kv_len;
  m.num_kv_rows = p->num_kv_rows;
  m.block_table = p->page_size ? p->block_table : nullptr;
  m.page_shift = p->page_size ? __builtin_ctz((unsigned)p->page_size) : 0;
  m.max_pages = p->page_size ? p->max_pages : 0;
  return m;
}

sga_status launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(SGA_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return SGA_OK;
}

#define SGA_TRY(expr)               \
  do {                              \
    sga_status _st = (expr);        \
    if (_st != SGA_OK) return _st;  \
  } while (0)

// --------------------------------------------------------------------------
// phase timing
// --------------------------------------------------------------------------
constexpr int kPhases = 4;
struct Profile {
  int max_calls = 0;
  int used = 0;
  std::vector<hipEvent_t> ev;  // (kPhases + 1) per call
};
thread_local Profile g_prof;

void prof_mark(hipStream_t s, int phase_boundary) {
  if (g_prof.used >= g_prof.max_calls) return;
  (void)hipEventRecord(g_prof.ev[(size_t)g_prof.used * (kPhases + 1) + phase_boundary], s);
}

MlaArgs mla_args(const sga_problem *p, const void *q, const void *kv, const uint8_t *kv_scale,
                 const int32_t *topk_idx, const void *gate, void *out, float *lse) {
  MlaArgs a;
  a.meta = meta_of(p);
  a.T = p->num_q;
  a.H = p->heads;
  a.Dc = p->d_latent;
  a.Dr = p->d_rope;
  a.k = p->topk;
  a.tau = p->softmax_scale;
  a.q = q;
  a.q_dtype = p->q_dtype;
  a.kv = kv;
  a.kv_dtype = p->kv_dtype;
  a.kv_scale = kv_scale;
  a.topk_idx = topk_idx;
  a.fuse = false;
  a.sel = TopkWs{};
  a.topk_out = nullptr;
  a.gate = gate;
  a.gate_dtype = p->gate_dtype;
  a.out = out;
  a.out_dtype = p->out_dtype;
  a.lse = lse;
  return a;
}

sga_status run_index(const sga_problem *p, const Plan &plan, const void *q_idx, const float *w,
                     const void *k_idx, float *scores, int64_t stride, TopkWs *sel,
                     hipStream_t s) {
  const SeqMeta m = meta_of(p);
  if (plan.idx == IdxPath::kFp8)
    return launched(launch_index_fp8(m, p->num_q, p->topk, (const uint8_t *)q_idx, w,
                                     (const uint8_t *)k_idx, scores, stride, sel, s),
                    "index scores (fp8)");
  return launched(launch_index_f32(m, p->num_q, p->topk, p->idx_heads, p->idx_dim,
                                   (const float *)q_idx, w, (const float *)k_idx, scores, stride,
                                   sel, s),
                  "index scores (fp32)");
}

sga_status run_mla(const MlaArgs &a, const Plan &plan, void *ws, hipStream_t s, bool prof) {
  if (plan.mla == MlaPath::kF32) {
    SGA_TRY(launched(launch_mla_f32(a, s), "sparse mla (fp32)"));
    if (prof) prof_mark(s, 3);
    return SGA_OK;
  }
  SGA_TRY(launched(launch_mla_split(a, ws, s), "sparse mla split"));
  if (prof) prof_mark(s, 3);
  return launched(launch_mla_combine(a, ws, s), "sparse mla combine");
}

// Argument checks of sga_layer_fwd and its allocation-free variant; *need
// receives the workspace bytes.
sga_status layer_check(const sga_problem *p, const void *q_idx, const float *w, const void *k_idx,
                       const void *q, const void *kv, const uint8_t *kv_scale, void *out, Plan *plan,
                       size_t *need) {
  SGA_TRY(plan_for(p, SGA_OP_LAYER, plan));
  *need = 0;
  if (p->num_q == 0) return SGA_OK;
  if (!q || !kv || !out) return fail(SGA_ERR_INVALID_ARGUMENT, "q / kv / out is NULL");
  if (p->max_kv_len > 0 && (!q_idx || !w || !k_idx))
    return fail(SGA_ERR_INVALID_ARGUMENT, "q_idx / w / k_idx is NULL");
  if (plan->mla == MlaPath::kMx && !kv_scale)
    return fail(SGA_ERR_INVALID_ARGUMENT, "MXFP8 rows need kv_scale");
  *need = ws_bytes(p, SGA_OP_LAYER, *plan);
  return SGA_OK;
}

// The a1 -> a4 launch sequence of one layer call on workspace `ws` (already
// checked to be large enough).
sga_status layer_launch(const sga_problem *p, const Plan &plan, const void *q_idx, const float *w,
                        const void *k_idx, const void *q, const void *kv, const uint8_t *kv_scale,
                        const void *gate, void *out, int32_t *topk_idx_out, float *lse, void *ws,
                        hipStream_t stream) {
  hipStream_t s = stream;
  const int T = p->num_q;
  const int64_t stride = score_stride(p);
  char *c = (char *)ws;
  float *scores = (float *)c;
  c += align256((size_t)T * stride * 4);
  int32_t *idx = (int32_t *)c;
  c += align256((size_t)T * p->topk * 4);
  if (topk_idx_out) idx = topk_idx_out;
  void *tws = c;
  c += align256(topk_ws_bytes(T, p->max_kv_len));
  void *mws = c;
  const SeqMeta m = meta_of(p);
  TopkWs tw = topk_ws_carve(tws, T, p->max_kv_len);
  const bool prof = g_prof.used < g_prof.max_calls;

  if (prof) prof_mark(s, 0);
  SGA_TRY(run_index(p, plan, q_idx, w, k_idx, scores, stride, &tw, s));
  if (prof) prof_mark(s, 1);
  // The MI355X MLA path can do the top-k's last step itself (MlaArgs::fuse)
  // when its grid fits the CUs at once: only the select kernel runs here,
  // and the split kernel derives its rows from the select's candidates and
  // writes topk_idx_out.
  const bool fuse = plan.mla != MlaPath::kF32 && p->max_kv_len > p->topk && mla_fuse_finish(T, p->topk);
  SGA_TRY(launched(launch_topk_select(m, T, p->topk, scores, stride, tw, idx, s, !fuse), "topk select"));
  if (prof) prof_mark(s, 2);
  MlaArgs a = mla_args(p, q, kv, kv_scale, idx, gate, out, lse);
  if (fuse) {
    a.fuse = true;
    a.sel = tw;
    a.topk_out = topk_idx_out;
  }
  SGA_TRY(run_mla(a, plan, mws, s, prof));
  if (prof) {
    prof_mark(s, 4);
    ++g_prof.used;
  }
  return SGA_OK;
}

// --------------------------------------------------------------------------
// static scratch of the allocation-free layer call
// --------------------------------------------------------------------------
// One buffer per GPU, part of this library's device code: the runtime places
// it on each device that loads the library and keeps it until the process
// ends. In host code the array's name is only a stand-in; its device address
// comes from hipGetSymbolAddress, once per device with that device current,
// and only that address is ever handed to kernels.
constexpr size_t kScratchBytes = SGA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

sga_status scratch_device_ptr(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SGA_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SGA_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::call_once(g_scratch_once[dev], [dev] {
    void *ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev])
    return fail(SGA_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                hipGetErrorString(g_scratch_err[dev]));
  *out = g_scratch_ptr[dev];
  return SGA_OK;
}

}  // namespace

extern "C" {

int sga_abi_version(void) { return SGA_ABI_VERSION; }

const char *sga_status_string(int status) {
  switch (status) {
    case SGA_OK: return "ok";
    case SGA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SGA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case SGA_ERR_WORKSPACE: return "workspace missing or too small";
    case SGA_ERR_DEVICE: return "device error";
    case SGA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char *sga_last_error(void) { return g_err.c_str(); }

sga_status sga_workspace_size(const sga_problem *p, int op, size_t *bytes) {
  try {
    if (!bytes) return fail(SGA_ERR_INVALID_ARGUMENT, "bytes is NULL");
    Plan plan;
    SGA_TRY(plan_for(p, op, &plan));
    *bytes = ws_bytes(p, op, plan);
    return SGA_OK;
  } catch (...) {
    return fail(SGA_ERR_DEVICE, "internal error");
  }
}

sga_status sga_index_scores(const sga_problem *p, const void *q_idx, const float *w,
                            const void *k_idx, float *scores, void *stream) {
  try {
    Plan plan;
    SGA_TRY(plan_for(p, SGA_OP_INDEX, &plan));
    if (p->num_q == 0 || p->max_kv_len == 0) return SGA_OK;
    if (!q_idx || !w || !k_idx || !scores)
      return fail(SGA_ERR_INVALID_ARGUMENT, "q_idx / w / k_idx / scores is NULL");
    return run_index(p, plan, q_idx, w, k_idx, scores, p->max_kv_len, nullptr,
                     (hipStream_t)stream);
  } catch (...) {
    return fail(SGA_ERR_DEVICE, "internal error");
  }
}

sga_status sga_topk_select(const sga_problem *p, const float *scores, int32_t *topk_idx,
                           void *ws, size_t ws_size, void *stream) {
  try {
    Plan plan;
    SGA_TRY(plan_for(p, SGA_OP_TOPK, &plan));
    if (p->num_q == 0) return SGA_OK;
    if (!topk_idx || (!scores && p->max_kv_len > 0))
      return fail(SGA_ERR_INVALID_ARGUMENT, "scores / topk_idx is NULL");
    const size_t need = ws_bytes(p, SGA_OP_TOPK, plan);
    if (need && (!ws || ws_size < need))
      return fail(SGA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_size);
    hipStream_t s = (hipStream_t)stream;
    const SeqMeta m = meta_of(p);
    TopkWs w = topk_ws_carve(ws, p->num_q, p->max_kv_len);
    SGA_TRY(launched(launch_topk_hist0(m, p->num_q, scores, p->max_kv_len, &w, s), "hist0"));
    return launched(launch_topk_select(m, p->num_q, p->topk, scores, p->max_kv_len, w, topk_idx, s),
                    "topk select");
  } catch (...) {
    return fail(SGA_ERR_DEVICE, "internal error");
  }
}

sga_status sga_sparse_mla_fwd(const sga_problem *p, const void *q, const void *kv,
                              const uint8_t *kv_scale, const int32_t *topk_idx, const void *gate,
                              void *out, float *lse, void *ws, size_t ws_size, void *stream) {
  try {
    Plan plan;
    SGA_TRY(plan_for(p, SGA_OP_MLA, &plan));
    if (p->num_q == 0) return SGA_OK;
    if (!q || !kv || !topk_idx || !out)
      return fail(SGA_ERR_INVALID_ARGUMENT, "q / kv / topk_idx / out is NULL");
    if (plan.mla == MlaPath::kMx && !kv_scale)
      return fail(SGA_ERR_INVALID_ARGUMENT, "MXFP8 rows need kv_scale");
    const size_t need = ws_bytes(p, SGA_OP_MLA, plan);
    if (need && (!ws || ws_size < need))
      return fail(SGA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_size);
    MlaArgs a = mla_args(p, q, kv, kv_scale, topk_idx, gate, out, lse);
    return run_mla(a, plan, ws, (hipStream_t)stream, false);
  } catch (...) {
    return fail(SGA_ERR_DEVICE, "internal error");
  }
}

sga_status sga_layer_fwd(const sga_problem *p, const void *q_idx, const float *w,
                         const void *k_idx, const void *q, const void *kv,
                         const uint8_t *kv_scale, const void *gate, void *out,
                         int32_t *topk_idx_out, float *lse, void *ws, size_t ws_size,
                         void *stream) {
  try {
    Plan plan;
    size_t need = 0;
    SGA_TRY(layer_check(p, q_idx, w, k_idx, q, kv, kv_scale, out, &plan, &need));
    if (p->num_q == 0) return SGA_OK;
    if (!ws || ws_size < need)
      return fail(SGA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_size);
    return layer_launch(p, plan, q_idx, w, k_idx, q, kv, kv_scale, gate, out, topk_idx_out, lse, ws,
                        (hipStream_t)stream);
  } catch (...) {
    return fail(SGA_ERR_DEVICE, "internal error");
  }
}

sga_status sga_layer_fwd_noalloc(const sga_problem *p, const void *q_idx, const float *w,
                                 const void *k_idx, const void *q, const void *kv,
                                 const uint8_t *kv_scale, const void *gate, void *out,
                                 int32_t *topk_idx_out, float *lse, void *stream) {
  try {
    Plan plan;
    size_t need = 0;
    SGA_TRY(layer_check(p, q_idx, w, k_idx, q, kv, kv_scale, out, &plan, &need));
    if (p->num_q == 0) return SGA_OK;
    if (need > kScratchBytes)
      return fail(SGA_ERR_WORKSPACE,
                  "this problem needs %zu bytes of workspace; the static scratch holds %zu "
                  "(call sga_layer_fwd with a caller workspace instead)",
                  need, kScratchBytes);
    void *ws = nullptr;
    SGA_TRY(scratch_device_ptr(&ws));
    return layer_launch(p, plan, q_idx, w, k_idx, q, kv, kv_scale, gate, out, topk_idx_out, lse, ws,
                        (hipStream_t)stream);
  } catch (...) {
    return fail(SGA_ERR_DEVICE, "internal error");
  }
}

sga_status sga_cache_append(const sga_problem *p, int64_t num_tokens, int src_dtype,
                            const void *kv_new, const void *k_idx_new, const int64_t *slots,
                            void *kv, uint8_t *kv_scale, void *k_idx, void *stream) {
  try {
    if (!p) return fail(SGA_ERR_INVALID_ARGUMENT, "problem is NULL");
    if (num_tokens < 0 || p->num_kv_rows < 0)
      return fail(SGA_ERR_INVALID_ARGUMENT, "negative size (num_tokens=%lld num_kv_rows=%lld)",
                  (long long)num_tokens, (long long)p->num_kv_rows);
    if (src_dtype != SGA_F32 && src_dtype != SGA_BF16)
      return fail(SGA_ERR_UNSUPPORTED, "source dtype must be SGA_F32 or SGA_BF16");
    const int64_t D = (int64_t)p->d_latent + p->d_rope;
    const int64_t DI = p->idx_dim;
    if (kv_new) {
      if (p->d_latent < 1 || p->d_rope < 0)
        return fail(SGA_ERR_INVALID_ARGUMENT, "d_latent must be >= 1, d_rope >= 0");
      if (p->kv_dtype != SGA_F32 && p->kv_dtype != SGA_BF16 && p->kv_dtype != SGA_MXFP8_E4M3FN)
        return fail(SGA_ERR_UNSUPPORTED, "kv dtype must be SGA_F32, SGA_BF16 or SGA_MXFP8_E4M3FN");
      if (D % (p->kv_dtype == SGA_MXFP8_E4M3FN ? 32 : 8))
        return fail(SGA_ERR_UNSUPPORTED, "row width %lld must be a multiple of %d", (long long)D,
                    p->kv_dtype == SGA_MXFP8_E4M3FN ? 32 : 8);
      if (num_tokens > 0 && !kv) return fail(SGA_ERR_INVALID_ARGUMENT, "kv is NULL");
      if (num_tokens > 0 && p->kv_dtype == SGA_MXFP8_E4M3FN && !kv_scale)
        return fail(SGA_ERR_INVALID_ARGUMENT, "MXFP8 rows need kv_scale");
    }
    if (k_idx_new) {
      if (DI < 1 || DI % 8)
        return fail(SGA_ERR_UNSUPPORTED, "idx_dim %lld must be a positive multiple of 8",
                    (long long)DI);
      if (p->idx_dtype != SGA_F32 && p->idx_dtype != SGA_FP8_E4M3FN)
        return fail(SGA_ERR_UNSUPPORTED, "index key dtype must be SGA_F32 or SGA_FP8_E4M3FN");
      if (num_tokens > 0 && !k_idx) return fail(SGA_ERR_INVALID_ARGUMENT, "k_idx is NULL");
    }
    const int64_t units = num_tokens * ((kv_new ? D : 0) + (k_idx_new ? DI : 0)) / 8;
    if (units >= ((int64_t)1 << 31))
      return fail(SGA_ERR_UNSUPPORTED, "%lld tokens are more than one call takes",
                  (long long)num_tokens);
    if (num_tokens == 0 || (!kv_new && !k_idx_new)) return SGA_OK;
    if (!slots) return fail(SGA_ERR_INVALID_ARGUMENT, "slots is NULL");
    return launched(launch_cache_append(num_tokens, (int)D, (int)DI, src_dtype, kv_new, k_idx_new,
                                        slots, p->num_kv_rows, p->kv_dtype, kv, kv_scale,
                                        p->idx_dtype, k_idx, (hipStream_t)stream),
                    "cache append");
  } catch (...) {
    return fail(SGA_ERR_DEVICE, "internal error");
  }
}

sga_status sga_indexer_kl(const sga_problem *p, const void *q_idx, const float *w,
                          const void *k_idx, const void *q, const void *kv,
                          const uint8_t *kv_scale, const int32_t *topk_idx, const float *lse,
                          float *loss, float *d_w, float *d_q_idx, float *d_k_idx, void *ws,
                          size_t ws_size, void *stream) {
  try {
    Plan plan;
    SGA_TRY(plan_for(p, SGA_OP_INDEXER_KL, &plan));
    if (p->num_q == 0) return SGA_OK;
    if (!q_idx || !w || !k_idx || !q || !kv || !topk_idx || !lse || !loss || !d_w || !d_q_idx || !d_k_idx)
      return fail(SGA_ERR_INVALID_ARGUMENT, "a tensor argument is NULL");
    if (p->kv_dtype == SGA_MXFP8_E4M3FN && !kv_scale)
      return fail(SGA_ERR_INVALID_ARGUMENT, "MXFP8 rows need kv_scale");
    const size_t need = ws_bytes(p, SGA_OP_INDEXER_KL, plan);
    if (!ws || ws_size < need)
      return fail(SGA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_size);
    return launched(launch_indexer_kl(meta_of(p), p->num_q, p->heads, p->d_latent + p->d_rope,
                                      p->idx_heads, p->idx_dim, p->topk, p->softmax_scale, q, p->q_dtype,
                                      kv, p->kv_dtype, kv_scale, q_idx, w, k_idx, p->idx_dtype, topk_idx,
                                      lse, loss, d_w, d_q_idx, d_k_idx, ws, (hipStream_t)stream),
                    "indexer KL");
  } catch (...) {
    return fail(SGA_ERR_DEVICE, "internal error");
  }
}

sga_status sga_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
  try {
    if (!src || !sink) return fail(SGA_ERR_INVALID_ARGUMENT, "src / sink is NULL");
    if (bytes % 8192 || ((uintptr_t)src & 15))
      return fail(SGA_ERR_INVALID_ARGUMENT, "bytes must be a multiple of 8192 and src 16-byte aligned");
    return launched(launch_stream_read((const uint8_t *)src, (int64_t)bytes, sink, (hipStream_t)stream),
                    "stream read");
  } catch (...) {
    return fail(SGA_ERR_DEVICE, "internal error");
  }
}

int sga_stream_read_sink_words(void) { return kStreamReadBlocksPerCu * device_cu_count(); }

sga_status sga_profile_enable(int max_calls) {
  try {
    for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
    g_prof.ev.clear();
    g_prof.used = 0;
    g_prof.max_calls = max_calls > 0 ? max_calls : 0;
    for (size_t i = 0; i < (size_t)g_prof.max_calls * (kPhases + 1); ++i) {
      hipEvent_t e;
      hipError_t err = hipEventCreate(&e);
      if (err != hipSuccess) {
        g_prof.max_calls = 0;
        return fail(SGA_ERR_DEVICE, "hipEventCreate: %s", hipGetErrorString(err));
      }
      g_prof.ev.push_back(e);
    }
    return SGA_OK;
  } catch (...) {
    return fail(SGA_ERR_DEVICE, "internal error");
  }
}

sga_status sga_profile_collect(double *ms, int nphase, int *calls) {
  try {
    if (!ms || !calls || nphase < 0) return fail(SGA_ERR_INVALID_ARGUMENT, "bad arguments");
    for (int i = 0; i < nphase; ++i) ms[i] = 0.0;
    *calls = g_prof.used;
    for (int c = 0; c < g_prof.used; ++c) {
      hipEvent_t *e = &g_prof.ev[(size_t)c * (kPhases + 1)];
      hipError_t err = hipEventSynchronize(e[kPhases]);
      if (err != hipSuccess)
        return fail(SGA_ERR_DEVICE, "hipEventSynchronize: %s", hipGetErrorString(err));
      for (int ph = 0; ph < kPhases && ph < nphase; ++ph) {
        float t = 0.0f;
        err = hipEventElapsedTime(&t, e[ph], e[ph + 1]);
        if (err != hipSuccess)
          return fail(SGA_ERR_DEVICE, "hipEventElapsedTime: %s", hipGetErrorString(err));
        ms[ph] += t;
      }
    }
    g_prof.used = 0;
    return SGA_OK;
  } catch (...) {
    return fail(SGA_ERR_DEVICE, "internal error");
  }
}

}  // extern "C"
