"""End-to-end GPU parity of sga_layer_fwd against the oracle, on the five
named workloads (full sizes, sampled queries where the oracle would be slow)
and on ragged / degenerate cases."""

import numpy as np
import pytest
import torch

import sparse_top_latent_amd as sga
from gpu_util import compare_layer, run_layer, say
from oracle import sga as osga
from sga_inputs import make_case, make_custom
from sga_inputs.gen import FULL_DIMS, TINY_DIMS

pytestmark = pytest.mark.gpu


def test_layer_tiny_fp32_all_queries():
    case = make_case("tiny_fp32_L512", device="cuda")
    say("case layer tiny_fp32_L512")
    compare_layer(case, label="tiny")


def test_layer_tiny_dims_k_at_least_n_is_dense():
    # k >= n: every query keeps its whole causal prefix, i.e. dense causal MLA
    case = make_custom([300], [(0, p) for p in range(0, 300, 7)],
                       dims=dict(TINY_DIMS, topk=512), precision="f32", seed=2, device="cuda")
    say("case layer tiny k>=n")
    out, idx, lse = run_layer(case)
    from oracle import case as ocase
    d = ocase.decode_all(case)
    o, _ = osga.dense_causal_mla(d["q"], d["kv"], d["q_pos"], case.softmax_scale, case.d_latent)
    y = osga.output_gate(o, d["gate"])
    err = np.max(np.abs(out.cpu().numpy() - y))
    assert err <= 1e-5 * np.max(np.abs(y))
    for i, p in enumerate(d["q_pos"]):
        assert list(idx[i, : p + 1].cpu().numpy()) == list(range(p + 1))
        assert bool(torch.all(idx[i, p + 1:] == -1))


def test_layer_full_dims_ragged_and_degenerate():
    lens = [2047, 2048, 2049, 4097, 9000, 1, 0, 130]
    qs = [(0, 2046), (1, 2047), (2, 2048), (3, 4096), (4, 8999), (4, 3000), (5, 0), (3, 2000),
          (7, 129)]
    case = make_custom(lens, qs, dims=FULL_DIMS, precision="bf16", seed=21, device="cuda",
                       softmax_scale=1 / 24)
    say("case layer ragged full dims")
    compare_layer(case, label="ragged")


def test_layer_workgroups_with_partial_load_batches():
    # 10 queries over sequences up to 30,001 keys: the decode indexer then
    # gives each workgroup 12 steps of 64 keys, not a multiple of the groups
    # a wave keeps in flight, and every query but the short ones spans
    # several workgroups (the keys past a workgroup's last step belong to the
    # next one and must not enter its scores or level-0 counts)
    lens = [20000, 4097, 64, 1, 9000, 12345, 2048, 30001]
    qs = [(b, n - 1) for b, n in enumerate(lens)] + [(0, 777), (5, 4096)]
    case = make_custom(lens, qs, dims=FULL_DIMS, precision="bf16", seed=51, device="cuda",
                       softmax_scale=1 / 24)
    say("case layer partial load batches")
    compare_layer(case, label="partial batches")


def test_layer_out_of_range_metadata_is_empty():
    # a query on an empty sequence, a bad sequence id, and a position past the cache
    case = make_custom([5000, 0], [(0, 4999), (1, 0), (0, 4999), (0, 4999)], dims=FULL_DIMS,
                       precision="bf16", seed=22, device="cuda", softmax_scale=1 / 24)
    case.q_seq[2] = 7          # no such sequence
    case.q_pos[3] = 10**6      # clipped to the cached length
    say("case layer metadata edges")
    out, idx, lse = run_layer(case)
    for t in (1, 2):
        assert torch.count_nonzero(out[t].float()) == 0
        assert bool(torch.all(idx[t] == -1))
        assert bool(torch.all(torch.isneginf(lse[t])))
    # query 3 sits past the end of its cache: it sees the whole sequence, like query 0
    assert bool(torch.all(idx[3] >= 0)) and int(idx[3].max()) <= 4999
    compare_layer(case, [0, 3], out=out, idx=idx, lse=lse, label="clip")


def test_layer_small_k_not_multiple_of_tiles():
    case = make_custom([3000, 800], [(0, 2999), (1, 799), (0, 99)], dims=dict(FULL_DIMS, topk=100),
                       precision="mxfp8", seed=23, device="cuda", softmax_scale=1 / 24)
    say("case layer k=100 mxfp8")
    compare_layer(case, label="k=100")


def test_layer_decode_b32_n32k_all_queries():
    case = make_case("decode_b32_n32k", device="cuda")
    say("case layer decode_b32_n32k")
    compare_layer(case, label="decode_b32_n32k")


def test_layer_decode_b16_n128k_all_queries_and_deterministic():
    case = make_case("decode_b16_n128k", device="cuda")
    say("case layer decode_b16_n128k (all 16 queries)")
    out1, idx1, lse1 = run_layer(case)
    out2, idx2, _ = run_layer(case)
    assert torch.equal(idx1, idx2) and torch.equal(out1, out2)
    compare_layer(case, out=out1, idx=idx1, lse=lse1, label="decode_b16_n128k")


def test_layer_decode_b16_n128k_mq4_all_queries():
    # 4 queries per sequence at its last 4 positions share one index scan
    case = make_case("decode_b16_n128k_mq4", device="cuda")
    say("case layer decode_b16_n128k_mq4 (all 64 queries)")
    compare_layer(case, label="decode_b16_n128k_mq4")


def test_layer_varlen_mxfp8_b64_all_queries():
    case = make_case("varlen_mxfp8_b64", device="cuda")
    say("case layer varlen_mxfp8_b64 (all 64 queries)")
    compare_layer(case, label="varlen_mxfp8_b64")


def prefill_sample(T=4096, group=8, groups=34):
    """The first and last query row of evenly spaced 8-row groups of the
    prefill chunk (both chunk ends included)."""
    g = np.unique(np.linspace(0, T // group - 1, groups).round().astype(int))
    return sorted({int(x) for gi in g for x in (gi * group, gi * group + group - 1)})


def test_layer_prefill_q4096_n128k_sampled():
    case = make_case("prefill_q4096_n128k", device="cuda")
    qs = prefill_sample()
    assert len(qs) >= 64 and qs[0] == 0 and qs[-1] == 4095
    say(f"case layer prefill_q4096_n128k ({len(qs)} sampled queries)")
    compare_layer(case, qs, label="prefill")


def heavy_tail_index(case, seed):
    """Index inputs whose top scores spread over many level-0 bins with ties.

    One index head scores each key by its first channel alone (w one-hot, the
    query's index matrix a unit vector), so a key's score is its first channel.
    That channel takes exact E4M3FN integers: each of the 53 largest (18 ..
    448) with probability 33/65536, the value 1 otherwise. Every score is then
    an exact integer, each value in its own level-0 bin (3 mantissa bits), and
    the 2,048 largest of a 128K-key query spread over about 30 bins with some
    65 keys each: a slot's 15-entry list head no longer reaches the threshold
    bin, and the k-th key has ties of which only the lowest positions are kept.
    """
    from sga_inputs.gen import uniform_int
    vals = [v for v in range(1, 449) if float(torch.tensor(float(v)).to(torch.float8_e4m3fn).float()) == v]
    top = torch.tensor(vals[::-1][:53], dtype=torch.float32, device="cuda")
    codes = torch.cat([top, torch.ones(1, device="cuda")]).to(torch.float8_e4m3fn).view(torch.uint8)
    rows = case.k_idx.shape[0]
    r = uniform_int((rows,), seed, "heavy_hi", 0, 255, device="cuda").to(torch.int64) * 256 + \
        uniform_int((rows,), seed, "heavy_lo", 0, 255, device="cuda").to(torch.int64)
    j = torch.where(r < 53 * 33, r // 33, torch.full_like(r, 53))
    case.k_idx[:, 0] = codes[j]
    case.q_idx.zero_()
    case.q_idx[:, 0, 0] = int(torch.tensor(1.0).to(torch.float8_e4m3fn).view(torch.uint8))
    case.w.zero_()
    case.w[:, 0] = 1.0


@pytest.mark.parametrize("precision", ["bf16", "mxfp8"])
def test_layer_heavy_tail_scores_whole_lists_and_partial_ties(precision):
    # the top-k select takes its threshold from the whole level-0 lists (the
    # list heads stop above it), and the k-th key has ties of which only the
    # lowest positions are kept
    lens = [131072, 50000, 262144, 3000]
    qs = [(0, 131071), (1, 49999), (2, 262143), (2, 100000), (0, 4095), (3, 2999), (1, 2047)]
    case = make_custom(lens, qs, dims=FULL_DIMS, precision=precision, seed=61, device="cuda",
                       softmax_scale=1 / 24)
    heavy_tail_index(case, 61)
    say(f"case layer heavy-tail scores ({precision})")
    compare_layer(case, label=f"heavy tail {precision}")
