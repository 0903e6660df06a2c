"""The C ABI without a GPU: exports, versions, workspace sizing and every
argument error path (all of which return before any HIP call)."""

import ctypes
import re
import os

import pytest

from sparse_top_latent_amd import _ffi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return _ffi.load()


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "sga.h")).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(sga_\w+)\s*\(", src, flags=re.M)))


def test_header_and_exports_agree(lib):
    declared = _declared_functions()
    assert declared == sorted(_ffi.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert lib.sga_abi_version() == 2
    for code in range(6):
        assert lib.sga_status_string(code)
    assert lib.sga_status_string(99) == b"unknown status"


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _problem(**kw):
    base = dict(num_seqs=16, num_q=16, max_kv_len=131072, page_size=0, num_kv_rows=16 * 131072,
                heads=64, d_latent=512, d_rope=64, idx_heads=64, idx_dim=128, topk=2048,
                softmax_scale=1 / 24, q_dtype=1, kv_dtype=1, idx_dtype=2, gate_dtype=1,
                out_dtype=1, q_seq=FAKE, q_pos=FAKE, kv_start=FAKE, kv_len=FAKE, block_table=None,
                max_pages=0, reserved0=0)
    base.update(kw)
    return _ffi.SgaProblem(**base)


def _ws(lib, p, op):
    n = ctypes.c_size_t(123)
    st = lib.sga_workspace_size(ctypes.byref(p), op, ctypes.byref(n))
    return st, n.value


def test_workspace_sizes(lib):
    p = _problem()
    st, idx = _ws(lib, p, _ffi.SGA_OP_INDEX)
    assert st == 0 and idx == 0
    sizes = {}
    for op in (_ffi.SGA_OP_TOPK, _ffi.SGA_OP_MLA, _ffi.SGA_OP_LAYER):
        st, sizes[op] = _ws(lib, p, op)
        assert st == 0 and sizes[op] > 0
    assert sizes[_ffi.SGA_OP_LAYER] >= sizes[_ffi.SGA_OP_TOPK] + sizes[_ffi.SGA_OP_MLA]
    # monotone in T, k and context
    for field, bigger in (("num_q", 32), ("topk", 1024), ("max_kv_len", 262144)):
        q = _problem(**{field: bigger, "num_seqs": 32, "num_kv_rows": 32 * 262144})
        for op in (_ffi.SGA_OP_TOPK, _ffi.SGA_OP_MLA, _ffi.SGA_OP_LAYER):
            st, n = _ws(lib, q, op)
            ref_p = _problem(num_seqs=32, num_kv_rows=32 * 262144)
            _, ref = _ws(lib, ref_p, op)
            assert st == 0
            if field == "topk":
                assert n <= ref
            else:
                assert n >= ref
    # the fp32 path needs no MLA workspace
    f = _problem(heads=8, d_latent=64, d_rope=16, idx_heads=2, idx_dim=32, topk=64, q_dtype=0,
                 kv_dtype=0, idx_dtype=0, gate_dtype=0, out_dtype=0)
    assert _ws(lib, f, _ffi.SGA_OP_MLA) == (0, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(reserved0=1), 1),
    (dict(num_q=-1), 1),
    (dict(topk=0), 1),
    (dict(q_seq=None), 1),
    (dict(kv_len=None), 1),
    (dict(q_dtype=7), 1),
    (dict(max_kv_len=5_000_000), 2),
    (dict(idx_heads=32), 2),
    (dict(idx_dtype=1), 2),
    (dict(heads=32), 2),
    (dict(topk=4096), 2),
    (dict(q_dtype=0), 2),
    (dict(out_dtype=2), 2),
    (dict(softmax_scale=float("nan")), 1),
    (dict(page_size=32, block_table=FAKE, max_pages=4), 1),      # pages below 64 rows
    (dict(page_size=96, block_table=FAKE, max_pages=4), 1),      # not a power of two
    (dict(page_size=1 << 17, block_table=FAKE, max_pages=4), 1),
    (dict(page_size=64, block_table=None, max_pages=4), 1),      # no block table
    (dict(page_size=64, block_table=FAKE, max_pages=0), 1),
    (dict(block_table=FAKE, max_pages=4), 1),                    # a table without pages
    (dict(kv_start=None), 1),                                    # contiguous needs kv_start
])
def test_invalid_problems(lib, kw, status):
    p = _problem(**kw)
    st, _ = _ws(lib, p, _ffi.SGA_OP_LAYER)
    assert st == status, lib.sga_last_error()
    assert lib.sga_last_error()
    st = lib.sga_layer_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None,
                           None, FAKE, 1 << 40, None)
    assert st == status


def test_paged_problem_is_valid_without_kv_start(lib):
    p = _problem(page_size=64, block_table=FAKE, max_pages=2048, kv_start=None)
    st, n = _ws(lib, p, _ffi.SGA_OP_LAYER)
    assert st == 0 and n > 0, lib.sga_last_error()


def test_null_problem_and_null_buffers(lib):
    n = ctypes.c_size_t()
    assert lib.sga_workspace_size(None, 0, ctypes.byref(n)) == 1
    p = _problem()
    assert lib.sga_workspace_size(ctypes.byref(p), 9, ctypes.byref(n)) == 1
    assert lib.sga_index_scores(ctypes.byref(p), None, FAKE, FAKE, FAKE, None) == 1
    assert lib.sga_topk_select(ctypes.byref(p), FAKE, None, FAKE, 1 << 40, None) == 1
    assert lib.sga_sparse_mla_fwd(ctypes.byref(p), FAKE, FAKE, None, FAKE, None, None, None, FAKE,
                                  1 << 40, None) == 1
    mx = _problem(kv_dtype=3)
    assert lib.sga_sparse_mla_fwd(ctypes.byref(mx), FAKE, FAKE, None, FAKE, None, FAKE, None,
                                  FAKE, 1 << 40, None) == 1
    assert b"kv_scale" in lib.sga_last_error()


def test_workspace_too_small(lib):
    p = _problem()
    _, need = _ws(lib, p, _ffi.SGA_OP_LAYER)
    st = lib.sga_layer_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None,
                           None, FAKE, need - 1, None)
    assert st == 3
    _, need = _ws(lib, p, _ffi.SGA_OP_TOPK)
    assert lib.sga_topk_select(ctypes.byref(p), FAKE, FAKE, FAKE, need - 1, None) == 3
    assert lib.sga_topk_select(ctypes.byref(p), FAKE, FAKE, None, 0, None) == 3


def test_empty_problems_enqueue_nothing(lib):
    p = _problem(num_q=0)
    assert lib.sga_index_scores(ctypes.byref(p), None, None, None, None, None) == 0
    assert lib.sga_topk_select(ctypes.byref(p), None, None, None, 0, None) == 0
    assert lib.sga_layer_fwd(ctypes.byref(p), None, None, None, None, None, None, None, None, None,
                             None, None, 0, None) == 0


def test_profile_collect_without_calls(lib):
    ms = (ctypes.c_double * 4)()
    calls = ctypes.c_int(5)
    assert lib.sga_profile_collect(ms, 4, ctypes.byref(calls)) == 0
    assert calls.value == 0 and list(ms) == [0.0] * 4
    assert lib.sga_profile_collect(None, 4, ctypes.byref(calls)) == 1


@pytest.mark.parametrize("kw,args,status", [
    (dict(), dict(src=7), 2),                                     # source dtype
    (dict(kv_dtype=2), dict(), 2),                                # FP8 latent rows: not a cache format
    (dict(d_rope=48, kv_dtype=3), dict(), 2),                     # MXFP8 row not a multiple of 32
    (dict(d_rope=60, kv_dtype=1), dict(), 2),                     # row not a multiple of 8
    (dict(idx_dim=100), dict(), 2),                               # key not a multiple of 8
    (dict(idx_dtype=1), dict(), 2),                               # bf16 keys: not a cache format
    (dict(), dict(n=-1), 1),
    (dict(), dict(slots=None), 1),
    (dict(), dict(kv=None), 1),
    (dict(kv_dtype=3), dict(kv_scale=None), 1),
    (dict(), dict(k_idx=None), 1),
    (dict(), dict(n=1 << 30), 2),                                 # more units than one launch takes
])
def test_cache_append_argument_errors(lib, kw, args, status):
    p = _problem(**kw)
    a = dict(n=16, src=1, kv_new=FAKE, k_idx_new=FAKE, slots=FAKE, kv=FAKE, kv_scale=FAKE,
             k_idx=FAKE)
    a.update(args)
    st = lib.sga_cache_append(ctypes.byref(p), a["n"], a["src"], a["kv_new"], a["k_idx_new"],
                              a["slots"], a["kv"], a["kv_scale"], a["k_idx"], None)
    assert st == status, lib.sga_last_error()
    assert lib.sga_last_error()


def test_cache_append_nothing_to_do(lib):
    p = _problem()
    # no tokens, or neither part given: returns before touching any pointer
    assert lib.sga_cache_append(ctypes.byref(p), 0, 1, FAKE, FAKE, None, None, None, None, None) == 0
    assert lib.sga_cache_append(ctypes.byref(p), 16, 1, None, None, None, None, None, None, None) == 0
    assert lib.sga_cache_append(None, 16, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1


@pytest.mark.parametrize("kw,status", [
    (dict(heads=80), 2),
    (dict(idx_dim=100), 2),
    (dict(topk=5000), 2),
    (dict(q_dtype=2), 2),
    (dict(kv_dtype=2), 2),
    (dict(idx_dtype=1), 2),
    (dict(d_latent=1000, d_rope=24), 2),   # q of one query past 96 KiB
    (dict(num_q=-1), 1),
])
def test_indexer_kl_argument_errors(lib, kw, status):
    p = _problem(**kw)
    st, _ = _ws(lib, p, _ffi.SGA_OP_INDEXER_KL)
    assert st == status, lib.sga_last_error()
    st = lib.sga_indexer_kl(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == status


def test_indexer_kl_null_buffers_and_workspace(lib):
    p = _problem()
    st, n = _ws(lib, p, _ffi.SGA_OP_INDEXER_KL)
    assert st == 0 and n > 16 * 2048 * 12
    args = [FAKE] * 12
    for i in range(12):
        if i == 5:  # kv_scale may be NULL for bf16 rows
            continue
        a = list(args)
        a[i] = None
        assert lib.sga_indexer_kl(ctypes.byref(p), *a, FAKE, 1 << 40, None) == 1
    assert lib.sga_indexer_kl(ctypes.byref(p), *args, FAKE, 16, None) == 3


def test_noalloc_layer_rejects_problems_beyond_its_scratch(lib):
    # checked on the host before any HIP call: 64 queries at 128K need about
    # 196 MiB of workspace, more than the 64 MiB static scratch
    big = _problem(num_q=64)
    _, need = _ws(lib, big, _ffi.SGA_OP_LAYER)
    assert need > _ffi.SGA_NOALLOC_SCRATCH_BYTES
    st = lib.sga_layer_fwd_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                                   None, None, None)
    assert st == 3 and b"static scratch" in lib.sga_last_error()
    # the headline batch (16 x 128K) fits
    _, need16 = _ws(lib, _problem(), _ffi.SGA_OP_LAYER)
    assert need16 <= _ffi.SGA_NOALLOC_SCRATCH_BYTES
    # argument errors come first, as in sga_layer_fwd
    bad = _problem(reserved0=1)
    assert lib.sga_layer_fwd_noalloc(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                                     None, None, None) == 1
    assert lib.sga_layer_fwd_noalloc(ctypes.byref(_problem()), None, None, None, FAKE, FAKE, None,
                                     None, FAKE, None, None, None) == 1


def test_stream_read_reference_argument_checks(lib):
    # measurement utility: rejected before any HIP call
    assert lib.sga_stream_read(None, 8192, FAKE, None) == 1
    assert lib.sga_stream_read(FAKE, 8192, None, None) == 1
    assert lib.sga_stream_read(FAKE, 8000, FAKE, None) == 1        # not whole 8 KiB tiles
    assert lib.sga_stream_read(FAKE + 8, 8192, FAKE, None) == 1    # not 16-byte aligned
