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


def test_layer_decode_b16_n128k_sampled_and_deterministic():
    case = make_case("decode_b16_n128k", device="cuda")
    say("case layer decode_b16_n128k")
    out1, idx1, lse1 = run_layer(case)
    out2, idx2, _ = run_layer(case)
    assert torch.equal(idx1, idx2) and torch.equal(out1, out2)
    compare_layer(case, [0, 5, 10, 15], out=out1, idx=idx1, lse=lse1, label="decode_b16_n128k")


def test_layer_decode_b16_n128k_mq4_sampled():
    # 4 queries per sequence at its last 4 positions share one index scan
    case = make_case("decode_b16_n128k_mq4", device="cuda")
    say("case layer decode_b16_n128k_mq4")
    compare_layer(case, [0, 1, 2, 3, 22, 63], label="decode_b16_n128k_mq4")


def test_layer_varlen_mxfp8_b64_sampled():
    case = make_case("varlen_mxfp8_b64", device="cuda")
    lens = np.array(case.lens)
    pick = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 3, 17, 40, 63})
    say(f"case layer varlen_mxfp8_b64 queries {pick}")
    compare_layer(case, pick, label="varlen_mxfp8_b64")


def test_layer_prefill_q4096_n128k_sampled():
    case = make_case("prefill_q4096_n128k", device="cuda")
    say("case layer prefill_q4096_n128k")
    compare_layer(case, [0, 1, 2048, 4095], label="prefill")
