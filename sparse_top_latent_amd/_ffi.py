"""ctypes view of include/sga.h (argument marshalling only)."""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; SGA_LIBRARY names another build of the same library
# (for side-by-side measurements of build variants)
LIB_PATH = os.environ.get("SGA_LIBRARY") or os.path.join(HERE, "libsga.so")

SGA_OK = 0
SGA_ERR_INVALID_ARGUMENT = 1
SGA_ERR_UNSUPPORTED = 2
SGA_ERR_WORKSPACE = 3
SGA_ERR_DEVICE = 4
SGA_ERR_LAUNCH = 5

SGA_F32 = 0
SGA_BF16 = 1
SGA_FP8_E4M3FN = 2
SGA_MXFP8_E4M3FN = 3

SGA_OP_INDEX = 0
SGA_OP_TOPK = 1
SGA_OP_MLA = 2
SGA_OP_LAYER = 3
SGA_OP_INDEXER_KL = 4
SGA_NOALLOC_SCRATCH_BYTES = 64 << 20

# every symbol include/sga.h declares
EXPORTS = (
    "sga_abi_version",
    "sga_status_string",
    "sga_last_error",
    "sga_workspace_size",
    "sga_index_scores",
    "sga_topk_select",
    "sga_sparse_mla_fwd",
    "sga_layer_fwd",
    "sga_layer_fwd_noalloc",
    "sga_cache_append",
    "sga_indexer_kl",
    "sga_profile_enable",
    "sga_profile_collect",
    "sga_stream_read",
    "sga_stream_read_sink_words",
)


class SgaProblem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q", ctypes.c_int32),
        ("max_kv_len", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_kv_rows", ctypes.c_int64),
        ("heads", ctypes.c_int32),
        ("d_latent", ctypes.c_int32),
        ("d_rope", ctypes.c_int32),
        ("idx_heads", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("idx_dtype", ctypes.c_int32),
        ("gate_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("q_seq", ctypes.c_void_p),
        ("q_pos", ctypes.c_void_p),
        ("kv_start", ctypes.c_void_p),
        ("kv_len", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("max_pages", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
    ]


class SgaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libsga.so from this package directory; raise if it was never built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m sparse_top_latent_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(SgaProblem)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    sigs = {
        "sga_abi_version": ([], ctypes.c_int),
        "sga_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "sga_last_error": ([], ctypes.c_char_p),
        "sga_workspace_size": ([P, ctypes.c_int, ctypes.POINTER(sz)], ctypes.c_int),
        "sga_index_scores": ([P, vp, vp, vp, vp, vp], ctypes.c_int),
        "sga_topk_select": ([P, vp, vp, vp, sz, vp], ctypes.c_int),
        "sga_sparse_mla_fwd": ([P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "sga_layer_fwd": ([P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "sga_layer_fwd_noalloc": ([P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
        "sga_cache_append": ([P, ctypes.c_int64, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp],
                             ctypes.c_int),
        "sga_indexer_kl": ([P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "sga_profile_enable": ([ctypes.c_int], ctypes.c_int),
        "sga_profile_collect": ([ctypes.POINTER(ctypes.c_double), ctypes.c_int,
                                 ctypes.POINTER(ctypes.c_int)], ctypes.c_int),
        "sga_stream_read": ([vp, sz, vp, vp], ctypes.c_int),
        "sga_stream_read_sink_words": ([], ctypes.c_int),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != SGA_OK:
        lib = load()
        detail = lib.sga_last_error().decode()
        raise SgaError(status, f"{lib.sga_status_string(status).decode()}: {detail}")
