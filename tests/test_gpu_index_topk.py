"""GPU parity of the indexer score pass and the top-k select (bit-exact)."""

import numpy as np
import pytest
import torch

import sparse_top_latent_amd as sga
from gpu_util import run_scores, say
from oracle import case as ocase
from oracle import sga as osga
from sga_inputs import make_case, make_custom
from sga_inputs.gen import FULL_DIMS

pytestmark = pytest.mark.gpu


def _check_scores(case, queries=None):
    # fp32 scores compared as bit patterns; only the compared rows leave the GPU
    scores = run_scores(case)
    ref = ocase.run_queries(case, queries)
    assert all(ref["scores_exact"])
    rows = torch.as_tensor(ref["queries"], device=scores.device)
    got = scores.index_select(0, rows).cpu().numpy()
    del scores
    for i, t in enumerate(ref["queries"]):
        r = ref["scores"][i]
        g = got[i, : r.size]
        assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), \
            f"query {t}: {np.count_nonzero(g != r)} scores differ"


def test_index_scores_tiny_fp32_all_queries():
    say("case tiny_fp32_L512 index scores")
    _check_scores(make_case("tiny_fp32_L512", device="cuda"))


def test_index_scores_fp8_ragged():
    # several 2048-key workgroups, ragged tails, one-key and empty sequences
    lens = [5000, 2049, 2048, 63, 1, 0, 4100]
    qs = [(0, 4999), (0, 1234), (1, 2048), (2, 2047), (3, 62), (4, 0), (5, 0), (6, 4099), (6, 64)]
    case = make_custom(lens, qs, dims=FULL_DIMS, precision="bf16", seed=11, device="cuda")
    say("case fp8 ragged index scores")
    _check_scores(case)


def test_index_scores_fp8_full_decode_b32_n32k():
    case = make_case("decode_b32_n32k", device="cuda")
    say("case decode_b32_n32k index scores, all 32 queries")
    _check_scores(case)


def test_index_scores_fp8_full_decode_b16_n128k():
    case = make_case("decode_b16_n128k", device="cuda")
    say("case decode_b16_n128k index scores, all 16 queries")
    _check_scores(case)


def test_index_scores_fp8_prefill_q4096_n128k_sampled():
    # first and last rows of spread 8-row groups of the query-tiled kernel
    case = make_case("prefill_q4096_n128k", device="cuda")
    qs = [0, 7, 8, 1023, 1024, 2047, 2048, 3071, 3072, 4088, 4095]
    say(f"case prefill_q4096_n128k index scores, {len(qs)} sampled queries")
    _check_scores(case, qs)


# --------------------------------------------------------------------------
# top-k select on adversarial score rows
# --------------------------------------------------------------------------
def _topk_case(rows, k):
    """Problem whose query t owns sequence t with n_t = len(rows[t])."""
    T = len(rows)
    lens = [len(r) for r in rows]
    L = max(max(lens), 1)
    scores = torch.full((T, L), float("nan"))
    for t, r in enumerate(rows):
        scores[t, : len(r)] = torch.as_tensor(r, dtype=torch.float32)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    prob = sga.Problem(
        q_seq=torch.arange(T, dtype=torch.int32, device="cuda"),
        q_pos=torch.as_tensor([max(n - 1, 0) if n else -1 for n in lens], dtype=torch.int32,
                              device="cuda"),
        kv_start=torch.as_tensor(starts, device="cuda"),
        kv_len=torch.as_tensor(lens, dtype=torch.int32, device="cuda"),
        max_kv_len=L, num_kv_rows=int(sum(lens)), heads=64, d_latent=512, d_rope=64,
        idx_heads=64, idx_dim=128, topk=k, softmax_scale=1.0)
    return prob, scores.cuda()


def _check_topk(rows, k, label):
    prob, scores = _topk_case(rows, k)
    out = torch.full((len(rows), k), -7, dtype=torch.int32, device="cuda")
    ws = sga.workspace(prob, sga.SGA_OP_TOPK)
    say(f"case topk {label}: T={len(rows)} k={k} max_n={scores.shape[1]}")
    sga.sga_topk_select(prob, scores, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for t, r in enumerate(rows):
        ref = osga.select_topk(np.asarray(r, dtype=np.float32), k)
        assert np.array_equal(got[t], ref), f"{label}: query {t} (n={len(r)}) differs"


def test_topk_ties_and_short_rows():
    g = torch.Generator().manual_seed(0)
    rows = []
    for n in (0, 1, 5, 2047, 2048, 2049, 4096, 4097, 9000, 30000):
        rows.append((torch.randint(-3, 4, (n,), generator=g).float() * 0.5).tolist())
    _check_topk(rows, 2048, "integer ties")


def test_topk_all_equal_signed_zero_and_negative():
    n = 20000
    zeros = [0.0] * n
    signed = [(-0.0 if i % 3 else 0.0) for i in range(n)]
    neg = (-torch.arange(n, dtype=torch.float32) / 7).tolist()
    _check_topk([zeros, signed, neg], 2048, "equal / signed zero / negative")


def test_topk_one_dense_bin_beyond_lds_staging():
    # 100k distinct scores that share their top 12 key bits: the refinement walks
    # more pairs than fit in LDS
    g = torch.Generator().manual_seed(1)
    n = 100_000
    vals = (1.0 + torch.rand(n, generator=g) * 0.12).tolist()
    _check_topk([vals, vals[: n // 2]], 2048, "dense level-0 bin")


def test_topk_many_slots_block_path():
    # 74 and 269 level-0 slots of 4,096 positions: more slots than one wave
    # merges, and more than one slot per thread of the block-wide merge
    g = torch.Generator().manual_seed(3)
    a = (torch.randint(-50, 50, (300_000,), generator=g).float() * 0.25).numpy()
    b = torch.randn(1_100_000, generator=g).numpy()
    _check_topk([a, b], 2048, "many slots")


def test_topk_small_k_and_continuous_scores():
    g = torch.Generator().manual_seed(2)
    rows = [torch.randn(n, generator=g).tolist() for n in (3, 100, 5000, 70000)]
    for k in (1, 7, 64):
        _check_topk(rows, k, f"k={k}")


def test_index_scores_prefill_groups_mixed():
    # 96 query rows over three sequences: 8-row groups that lie inside one
    # sequence go through the query-tiled prefill kernel, the two groups that
    # straddle a sequence boundary (rows 32-39 and 80-87) through the
    # per-query kernel
    lens = [9000, 20000, 3000]
    qs = [(0, 8999 - i) for i in range(37)] + [(1, 19999 - 7 * i) for i in range(45)] + \
         [(2, 2999 - i) for i in range(14)]
    case = make_custom(lens, qs, dims=FULL_DIMS, precision="bf16", seed=41, device="cuda")
    say("case prefill index scores, mixed groups")
    _check_scores(case)


def test_index_scores_prefill_single_sequence_chunk():
    # a prefill chunk: 200 consecutive positions at the end of a 40,000-token
    # sequence (a ragged last group and a ragged causal edge)
    n = 40000
    case = make_custom([n], [(0, n - 200 + i) for i in range(200)], dims=FULL_DIMS,
                       precision="bf16", seed=42, device="cuda")
    say("case prefill index scores, one sequence")
    _check_scores(case, [0, 1, 17, 100, 150, 199])


def test_index_scores_multi_query_groups_of_four():
    # a few queries per sequence (speculative verification): 4-row groups
    # share each key tile. Sequence 5 holds 5 queries, so every later group
    # straddles a sequence boundary and takes the per-query path; ragged
    # lengths give ragged last chunks and a 64-key sequence.
    lens = [9000, 20000, 3000, 4097, 12000, 5000, 64, 8191, 16385, 2048, 7000, 30000]
    qs = []
    for b, n in enumerate(lens):
        q = 5 if b == 5 else 4
        qs += [(b, n - q + j) for j in range(q)]
    case = make_custom(lens, qs, dims=FULL_DIMS, precision="bf16", seed=43, device="cuda")
    say(f"case multi-query index scores, {len(qs)} queries over {len(lens)} sequences")
    _check_scores(case)


def test_topk_threshold_deep_in_wide_histograms():
    # scores spread over hundreds of level-0 bins per 4096-position chunk and
    # k near n / 2: the threshold lies far below the 15 highest bins of every
    # chunk's list, so the select must read the lists in full
    g = torch.Generator().manual_seed(3)
    rows = []
    for n in (5000, 9000, 20000):
        x = torch.randn(n, generator=g) * torch.exp(3 * torch.randn(n, generator=g))
        rows.append(x.tolist())
    _check_topk(rows, 2048, "wide histograms, k ~ n/2 and below")
    _check_topk([r[:4100] for r in rows], 2048, "wide histograms, k = n/2")


def test_topk_nan_ranks_above_inf_and_ties_by_position():
    # every NaN, either sign and any payload, ranks above +inf; NaNs tie with
    # each other (lower position first). Row 0: a few NaNs and infs among
    # normal scores; row 1: more NaNs than k, so the selection is the first k
    # NaN positions.
    g = np.random.default_rng(7)
    a = g.standard_normal(9000).astype(np.float32)
    bits = a.view(np.uint32)
    nan_pos = g.choice(9000, 60, replace=False)
    bits[nan_pos] = np.where(np.arange(60) % 2 == 0, 0x7FC00000, 0xFFC00001) + np.arange(60, dtype=np.uint32)
    a[g.choice(np.setdiff1d(np.arange(9000), nan_pos), 10, replace=False)] = np.inf
    b = g.standard_normal(12000).astype(np.float32)
    bb = b.view(np.uint32)
    many = g.choice(12000, 3000, replace=False)
    bb[many] = np.where(many % 3 == 0, 0xFF800001, 0x7F800005).astype(np.uint32)
    _check_topk([a, b], 2048, "NaN scores")
