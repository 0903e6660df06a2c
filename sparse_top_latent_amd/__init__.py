"""Python binding of the SGA hot-path library (libsga.so, HIP for gfx950).

The functions below carry the names of the C ABI in include/sga.h and only
marshal arguments: they check device, dtype, contiguity and size of torch
tensors, then pass raw pointers and the current HIP stream. Every step of the
computation runs in the library's kernels; there is no fallback. PyTorch
provides device memory and streams.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _ffi
from ._ffi import (  # noqa: F401
    SGA_BF16,
    SGA_F32,
    SGA_FP8_E4M3FN,
    SGA_MXFP8_E4M3FN,
    SGA_OP_INDEX,
    SGA_NOALLOC_SCRATCH_BYTES,
    SGA_OP_INDEXER_KL,
    SGA_OP_LAYER,
    SGA_OP_MLA,
    SGA_OP_TOPK,
    SgaError,
    SgaProblem,
)

_DTYPE_CODES = {"f32": SGA_F32, "bf16": SGA_BF16, "fp8": SGA_FP8_E4M3FN, "mxfp8": SGA_MXFP8_E4M3FN}
_ELEM = {SGA_F32: (torch.float32,), SGA_BF16: (torch.bfloat16,),
         SGA_FP8_E4M3FN: (torch.uint8, torch.float8_e4m3fn),
         SGA_MXFP8_E4M3FN: (torch.uint8, torch.float8_e4m3fn)}


def lib():
    return _ffi.load()


def abi_version() -> int:
    return lib().sga_abi_version()


class Problem:
    """An sga_problem plus references to its device metadata tensors."""

    def __init__(self, *, q_seq, q_pos, kv_start, kv_len, max_kv_len, num_kv_rows, heads,
                 d_latent, d_rope, idx_heads, idx_dim, topk, softmax_scale, q_dtype="bf16",
                 kv_dtype="bf16", idx_dtype="fp8", gate_dtype="bf16", out_dtype="bf16",
                 page_size=0, block_table=None):
        """Contiguous caches (kv_start) or, with page_size > 0, paged caches
        addressed through block_table [num_seqs, max_pages] (int32)."""
        metas = [("q_seq", q_seq, torch.int32), ("q_pos", q_pos, torch.int32),
                 ("kv_len", kv_len, torch.int32)]
        if page_size:
            if block_table is None or block_table.dim() != 2 or block_table.shape[0] != kv_len.numel():
                raise ValueError("paged caches need block_table [num_seqs, max_pages]")
            metas.append(("block_table", block_table, torch.int32))
        else:
            metas.append(("kv_start", kv_start, torch.int64))
        for name, t, dt in metas:
            if t.dtype != dt or not t.is_contiguous() or t.device.type != "cuda":
                raise ValueError(f"{name} must be a contiguous {dt} CUDA tensor")
        if q_seq.numel() != q_pos.numel() or (not page_size and kv_start.numel() != kv_len.numel()):
            raise ValueError("metadata lengths disagree")
        self._keep = (q_seq, q_pos, kv_start, kv_len, block_table)
        code = lambda d: d if isinstance(d, int) else _DTYPE_CODES[d]  # noqa: E731
        self.c = SgaProblem(
            num_seqs=kv_len.numel(), num_q=q_pos.numel(), max_kv_len=int(max_kv_len),
            num_kv_rows=int(num_kv_rows), heads=heads, d_latent=d_latent, d_rope=d_rope,
            idx_heads=idx_heads, idx_dim=idx_dim, topk=topk, softmax_scale=float(softmax_scale),
            q_dtype=code(q_dtype), kv_dtype=code(kv_dtype), idx_dtype=code(idx_dtype),
            gate_dtype=code(gate_dtype or "f32"), out_dtype=code(out_dtype),
            q_seq=q_seq.data_ptr(), q_pos=q_pos.data_ptr(),
            kv_start=None if page_size else kv_start.data_ptr(), kv_len=kv_len.data_ptr(),
            page_size=int(page_size), block_table=block_table.data_ptr() if page_size else None,
            max_pages=int(block_table.shape[1]) if page_size else 0, reserved0=0)

    @classmethod
    def from_case(cls, case, *, topk: Optional[int] = None, out_dtype: Optional[str] = None,
                  max_kv_len: Optional[int] = None) -> "Problem":
        """Problem for an sga_inputs.SgaCase whose tensors already live on the GPU."""
        return cls(q_seq=case.q_seq, q_pos=case.q_pos, kv_start=case.kv_start, kv_len=case.kv_len,
                   max_kv_len=case.max_kv_len if max_kv_len is None else max_kv_len,
                   num_kv_rows=case.num_kv_rows, heads=case.heads, d_latent=case.d_latent,
                   d_rope=case.d_rope, idx_heads=case.idx_heads, idx_dim=case.idx_dim,
                   topk=case.topk if topk is None else topk, softmax_scale=case.softmax_scale,
                   q_dtype=case.q_dtype, kv_dtype=case.kv_dtype, idx_dtype=case.idx_dtype,
                   gate_dtype=case.gate_dtype, out_dtype=out_dtype or case.out_dtype,
                   page_size=case.page_size, block_table=case.block_table)

    @classmethod
    def for_cache(cls, *, num_kv_rows, d_latent, d_rope, idx_dim, kv_dtype, idx_dtype,
                  device="cuda") -> "Problem":
        """Problem for sga_cache_append, which reads only the cache geometry and dtypes."""
        e32 = torch.empty(0, dtype=torch.int32, device=device)
        e64 = torch.empty(0, dtype=torch.int64, device=device)
        return cls(q_seq=e32, q_pos=e32, kv_start=e64, kv_len=e32, max_kv_len=0,
                   num_kv_rows=num_kv_rows, heads=1, d_latent=d_latent, d_rope=d_rope,
                   idx_heads=1, idx_dim=idx_dim, topk=1, softmax_scale=1.0, q_dtype="bf16",
                   kv_dtype=kv_dtype, idx_dtype=idx_dtype)

    @property
    def ptr(self):
        return ctypes.byref(self.c)

    def __getattr__(self, name):
        if name in ("c", "_keep"):
            raise AttributeError(name)
        return getattr(self.c, name)


def _ptr(t: Optional[torch.Tensor], name: str, codes=None, numel: Optional[int] = None):
    if t is None:
        return None
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if codes is not None:
        ok = tuple(d for c in codes for d in _ELEM[c])
        if t.dtype not in ok:
            raise ValueError(f"{name} has dtype {t.dtype}, expected one of {ok}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def sga_workspace_size(prob: Problem, op: int) -> int:
    n = ctypes.c_size_t(0)
    _ffi.check(lib().sga_workspace_size(prob.ptr, op, ctypes.byref(n)))
    return int(n.value)


def workspace(prob: Problem, op: int, device="cuda") -> torch.Tensor:
    """A uint8 device buffer of the size `op` needs (at least 1 byte)."""
    return torch.empty(max(1, sga_workspace_size(prob, op)), dtype=torch.uint8, device=device)


def sga_index_scores(prob: Problem, q_idx, w, k_idx, scores, stream=None) -> None:
    c = prob.c
    T, HI, DI = c.num_q, c.idx_heads, c.idx_dim
    _ffi.check(lib().sga_index_scores(
        prob.ptr,
        _ptr(q_idx, "q_idx", (c.idx_dtype,), T * HI * DI),
        _ptr(w, "w", (SGA_F32,), T * HI),
        _ptr(k_idx, "k_idx", (c.idx_dtype,), c.num_kv_rows * DI),
        _ptr(scores, "scores", (SGA_F32,), T * c.max_kv_len),
        _stream(stream)))


def sga_topk_select(prob: Problem, scores, topk_idx, ws, stream=None) -> None:
    c = prob.c
    _ffi.check(lib().sga_topk_select(
        prob.ptr,
        _ptr(scores, "scores", (SGA_F32,), c.num_q * c.max_kv_len),
        _ptr(topk_idx, "topk_idx", None, c.num_q * c.topk),
        _ptr(ws, "ws"), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))


def _mla_ptrs(c, q, kv, kv_scale, gate, out, lse):
    T, H, Dc, D = c.num_q, c.heads, c.d_latent, c.d_latent + c.d_rope
    return (
        _ptr(q, "q", (c.q_dtype,), T * H * D),
        _ptr(kv, "kv", (c.kv_dtype,), c.num_kv_rows * D),
        _ptr(kv_scale, "kv_scale", (SGA_FP8_E4M3FN,),
             c.num_kv_rows * (D // 32) if kv_scale is not None else None),
        _ptr(gate, "gate", (c.gate_dtype,), T * H * Dc),
        _ptr(out, "out", (c.out_dtype,), T * H * Dc),
        _ptr(lse, "lse", (SGA_F32,), T * H),
    )


def sga_sparse_mla_fwd(prob: Problem, q, kv, kv_scale, topk_idx, gate, out, lse=None, ws=None,
                       stream=None) -> None:
    c = prob.c
    pq, pkv, psc, pg, po, pl = _mla_ptrs(c, q, kv, kv_scale, gate, out, lse)
    if topk_idx is not None and topk_idx.dtype != torch.int32:
        raise ValueError("topk_idx must be int32")
    _ffi.check(lib().sga_sparse_mla_fwd(
        prob.ptr, pq, pkv, psc, _ptr(topk_idx, "topk_idx", None, c.num_q * c.topk), pg, po, pl,
        _ptr(ws, "ws"), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def sga_layer_fwd(prob: Problem, q_idx, w, k_idx, q, kv, kv_scale, gate, out, topk_idx_out=None,
                  lse=None, ws=None, stream=None) -> None:
    c = prob.c
    T, HI, DI = c.num_q, c.idx_heads, c.idx_dim
    pq, pkv, psc, pg, po, pl = _mla_ptrs(c, q, kv, kv_scale, gate, out, lse)
    if topk_idx_out is not None and topk_idx_out.dtype != torch.int32:
        raise ValueError("topk_idx_out must be int32")
    _ffi.check(lib().sga_layer_fwd(
        prob.ptr,
        _ptr(q_idx, "q_idx", (c.idx_dtype,), T * HI * DI),
        _ptr(w, "w", (SGA_F32,), T * HI),
        _ptr(k_idx, "k_idx", (c.idx_dtype,), c.num_kv_rows * DI),
        pq, pkv, psc, pg, po,
        _ptr(topk_idx_out, "topk_idx_out", None, T * c.topk),
        pl,
        _ptr(ws, "ws"), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))


def sga_layer_fwd_noalloc(prob: Problem, q_idx, w, k_idx, q, kv, kv_scale, gate, out,
                          topk_idx_out=None, lse=None, stream=None) -> None:
    """sga_layer_fwd on the library's static per-GPU scratch (no workspace
    argument, no allocation); calls on one GPU must not overlap in time."""
    c = prob.c
    T, HI, DI = c.num_q, c.idx_heads, c.idx_dim
    pq, pkv, psc, pg, po, pl = _mla_ptrs(c, q, kv, kv_scale, gate, out, lse)
    if topk_idx_out is not None and topk_idx_out.dtype != torch.int32:
        raise ValueError("topk_idx_out must be int32")
    _ffi.check(lib().sga_layer_fwd_noalloc(
        prob.ptr,
        _ptr(q_idx, "q_idx", (c.idx_dtype,), T * HI * DI),
        _ptr(w, "w", (SGA_F32,), T * HI),
        _ptr(k_idx, "k_idx", (c.idx_dtype,), c.num_kv_rows * DI),
        pq, pkv, psc, pg, po,
        _ptr(topk_idx_out, "topk_idx_out", None, T * c.topk),
        pl,
        _stream(stream)))


def sga_stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """The library's streaming-read reference over a device tensor (see sga.h)."""
    nbytes = src.numel() * src.element_size()
    if sink.dtype != torch.int32 or sink.numel() < lib().sga_stream_read_sink_words():
        raise ValueError("sink must be an int32 tensor of sga_stream_read_sink_words() words")
    _ffi.check(lib().sga_stream_read(_ptr(src, "src"), nbytes - nbytes % 8192, _ptr(sink, "sink"),
                                     _stream(stream)))


def sga_cache_append(prob: Problem, kv_new, k_idx_new, slots, kv, kv_scale, k_idx,
                     stream=None) -> None:
    """Quantise new tokens into cache rows `slots` (see sga_cache_append in sga.h).

    kv_new [N, Dc + Dr] and k_idx_new [N, DI] share one source dtype (float32
    or bfloat16); either may be None to skip that part.
    """
    c = prob.c
    D, DI = c.d_latent + c.d_rope, c.idx_dim
    if slots.dtype != torch.int64:
        raise ValueError("slots must be int64")
    N = slots.numel()
    srcs = [t for t in (kv_new, k_idx_new) if t is not None]
    if any(t.dtype != srcs[0].dtype for t in srcs):
        raise ValueError("kv_new and k_idx_new must share a dtype")
    src = SGA_BF16 if srcs and srcs[0].dtype == torch.bfloat16 else SGA_F32
    _ffi.check(lib().sga_cache_append(
        prob.ptr, N, src,
        _ptr(kv_new, "kv_new", (src,), N * D),
        _ptr(k_idx_new, "k_idx_new", (src,), N * DI),
        _ptr(slots, "slots", None, N),
        _ptr(kv, "kv", (c.kv_dtype,), c.num_kv_rows * D if kv_new is not None else None),
        _ptr(kv_scale, "kv_scale", (SGA_FP8_E4M3FN,),
             c.num_kv_rows * (D // 32) if kv_scale is not None else None),
        _ptr(k_idx, "k_idx", (c.idx_dtype,), c.num_kv_rows * DI if k_idx_new is not None else None),
        _stream(stream)))


def sga_indexer_kl(prob: Problem, q_idx, w, k_idx, q, kv, kv_scale, topk_idx, lse, loss, d_w,
                   d_q_idx, d_k_idx, ws, stream=None) -> None:
    """Indexer KL loss and gradients (see sga_indexer_kl in sga.h); d_k_idx is added to."""
    c = prob.c
    T, H, HI, DI, D = c.num_q, c.heads, c.idx_heads, c.idx_dim, c.d_latent + c.d_rope
    for name, t in (("topk_idx", topk_idx),):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    _ffi.check(lib().sga_indexer_kl(
        prob.ptr,
        _ptr(q_idx, "q_idx", (c.idx_dtype,), T * HI * DI),
        _ptr(w, "w", (SGA_F32,), T * HI),
        _ptr(k_idx, "k_idx", (c.idx_dtype,), c.num_kv_rows * DI),
        _ptr(q, "q", (c.q_dtype,), T * H * D),
        _ptr(kv, "kv", (c.kv_dtype,), c.num_kv_rows * D),
        _ptr(kv_scale, "kv_scale", (SGA_FP8_E4M3FN,),
             c.num_kv_rows * (D // 32) if kv_scale is not None else None),
        _ptr(topk_idx, "topk_idx", None, T * c.topk),
        _ptr(lse, "lse", (SGA_F32,), T * H),
        _ptr(loss, "loss", (SGA_F32,), T),
        _ptr(d_w, "d_w", (SGA_F32,), T * HI),
        _ptr(d_q_idx, "d_q_idx", (SGA_F32,), T * HI * DI),
        _ptr(d_k_idx, "d_k_idx", (SGA_F32,), c.num_kv_rows * DI),
        _ptr(ws, "ws"), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def sga_profile_enable(max_calls: int) -> None:
    _ffi.check(lib().sga_profile_enable(int(max_calls)))


def sga_profile_collect(nphase: int = 4):
    """(summed ms per phase, number of timed calls) since sga_profile_enable."""
    ms = (ctypes.c_double * nphase)()
    calls = ctypes.c_int(0)
    _ffi.check(lib().sga_profile_collect(ms, nphase, ctypes.byref(calls)))
    return list(ms), calls.value


def out_torch_dtype(code: int):
    return torch.float32 if code == SGA_F32 else torch.bfloat16
