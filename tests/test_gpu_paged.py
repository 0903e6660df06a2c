"""GPU parity of the paged cache layout (block table).

Each case is run twice through the C ABI: on contiguous caches, and on a
copy whose rows sit in pages of page_size rows in a seeded random page order
with a block table (sga_inputs.paged_copy). The same logical rows must give
bit-identical scores, top-k lists, outputs and log-sum-exps, and sampled
queries of the paged run are compared with the oracle reading the caches
through the same table.
"""

import numpy as np
import pytest
import torch

import sparse_top_latent_amd as sga
from gpu_util import compare_layer, run_layer, run_scores, say
from sga_inputs import make_case, make_custom, paged_copy
from sga_inputs.gen import FULL_DIMS

pytestmark = pytest.mark.gpu


def _same(a, b, what):
    if a is None:
        return
    if a.dtype in (torch.float32, torch.bfloat16):
        x, y = a.float().cpu().numpy(), b.float().cpu().numpy()
        ok = np.array_equal(x.view(np.uint32), y.view(np.uint32))
    else:
        ok = torch.equal(a.cpu(), b.cpu())
    assert ok, f"{what} differs between contiguous and paged caches"


def _check_paged(case, page_size, sample, label):
    paged = paged_copy(case, page_size, seed=page_size)
    say(f"case paged {label}: page_size={page_size}, {paged.num_kv_rows} rows in pages, "
        f"T={case.num_q}")
    o0, i0, l0 = run_layer(case)
    o1, i1, l1 = run_layer(paged)
    _same(i0, i1, "top-k")
    _same(o0, o1, "y")
    _same(l0, l1, "lse")
    s0, s1 = run_scores(case), run_scores(paged)
    n = (case.q_pos.long() + 1).clamp(max=case.max_kv_len)
    for t in range(case.num_q):
        _same(s0[t, : n[t]], s1[t, : n[t]], f"scores of query {t}")
    compare_layer(paged, sample, out=o1, idx=i1, lse=l1, label=label)


@pytest.mark.parametrize("page_size", [64, 256])
def test_paged_decode_ragged(page_size):
    # one query per sequence (the per-query indexer kernel), ragged lengths,
    # a one-page and a one-key sequence
    lens = [20000, 4097, 64, 1, 9000, 12345, 2048, 30001]
    qs = [(b, n - 1) for b, n in enumerate(lens)] + [(0, 777), (5, 4096)]
    case = make_custom(lens, qs, dims=FULL_DIMS, precision="bf16", seed=51, device="cuda")
    _check_paged(case, page_size, [0, 2, 3, 7, 8], f"decode ragged p{page_size}")


def test_paged_prefill_groups_and_multi_query():
    # 8-row groups inside one sequence and groups that straddle a boundary
    # (query-tiled kernel, both paths), then 4-row groups (multi-query decode)
    lens = [9000, 20000, 3000]
    qs = [(0, 8999 - i) for i in range(37)] + [(1, 19999 - 7 * i) for i in range(45)] + \
         [(2, 2999 - i) for i in range(14)]
    case = make_custom(lens, qs, dims=FULL_DIMS, precision="bf16", seed=52, device="cuda")
    _check_paged(case, 128, [0, 36, 37, 60, 95], "prefill groups p128")
    lens = [9000, 20000, 3000, 4097, 12000, 5000, 64, 8191, 16385, 2048]
    qs = [(b, n - 4 + j) for b, n in enumerate(lens) for j in range(4)]
    case = make_custom(lens, qs, dims=FULL_DIMS, precision="bf16", seed=53, device="cuda")
    _check_paged(case, 64, [0, 5, 26, 39], "multi-query p64")


def test_paged_mxfp8_and_fp32_paths():
    lens = [7000, 33000, 129, 16384]
    case = make_custom(lens, [(b, n - 1) for b, n in enumerate(lens)], dims=FULL_DIMS,
                       precision="mxfp8", seed=54, device="cuda")
    _check_paged(case, 512, [0, 1, 2, 3], "mxfp8 p512")
    _check_paged(make_case("tiny_fp32_L512", device="cuda"), 64, [0, 63, 64, 200, 511], "fp32 tiny p64")


def test_paged_decode_b16_n128k_sampled():
    # the bench's workload in 64-row pages
    case = make_case("decode_b16_n128k", device="cuda")
    _check_paged(case, 64, [0, 9, 15], "decode_b16_n128k p64")


def test_paged_large_pages_and_bad_page_ids():
    # pages larger than a workgroup's key range; then a block table with ids
    # outside the cache for sequence 0. The results of sequence 0's query are
    # unspecified (only: the run completes and its list names positions of
    # the sequence); the queries of sequence 1 must be exactly what they are
    # with a valid table, and match the oracle.
    lens = [40000, 70000]
    case = make_custom(lens, [(0, 39999), (1, 69999), (1, 5000)], dims=FULL_DIMS, precision="bf16",
                       seed=55, device="cuda")
    _check_paged(case, 8192, [0, 1, 2], "pages of 8192")
    paged = paged_copy(case, 1024, seed=3)
    o0, i0, l0 = run_layer(paged)
    paged.block_table[0, 3] = 1 << 20
    paged.block_table[0, 5] = -2
    say("case paged: out-of-range page ids")
    o1, i1, l1 = run_layer(paged)
    _same(i0[1:], i1[1:], "top-k of sequence 1")
    _same(o0[1:], o1[1:], "y of sequence 1")
    _same(l0[1:], l1[1:], "lse of sequence 1")
    sel = i1[0]
    assert bool(torch.all((sel == -1) | ((sel >= 0) & (sel < lens[0]))))
    compare_layer(paged, [1, 2], out=o1, idx=i1, lse=l1, label="sequence 1 beside bad page ids")
