"""GPU parity of the sparse MLA + gate, fed with index lists from the oracle,
plus the method's invariants on the device."""

import math

import numpy as np
import pytest
import torch

import sparse_top_latent_amd as sga
from gpu_util import check_close, say, to_np
from oracle import case as ocase
from oracle import sga as osga
from sga_inputs import make_case, make_custom
from sga_inputs.gen import FULL_DIMS

pytestmark = pytest.mark.gpu


def _run_mla(case, idx, *, gate=..., out_dtype=None):
    prob = sga.Problem.from_case(case, out_dtype=out_dtype)
    T, H, Dc = case.num_q, case.heads, case.d_latent
    out = torch.empty((T, H, Dc), dtype=sga.out_torch_dtype(prob.c.out_dtype), device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = sga.workspace(prob, sga.SGA_OP_MLA)
    g = case.gate if gate is ... else gate
    sga.sga_sparse_mla_fwd(prob, case.q, case.kv, case.kv_scale, idx, g, out, lse, ws)
    torch.cuda.synchronize()
    return out, lse


def _oracle(case):
    ref = ocase.run_queries(case, keep_scores=False)
    idx = torch.as_tensor(ref["topk_idx"], dtype=torch.int32, device="cuda")
    return ref, idx


def _compare(case, out, lse, ref, label):
    check_close(to_np(out), ref["y"], case, label)
    lr = ref["lse"]
    lg = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(lr)
    assert np.array_equal(fin, np.isfinite(lg))
    if fin.any():
        assert np.max(np.abs(lg[fin] - lr[fin])) <= 1e-3 * max(1.0, np.max(np.abs(lr[fin])))


def test_mla_tiny_fp32():
    case = make_case("tiny_fp32_L512", device="cuda")
    ref, idx = _oracle(case)
    say("case mla tiny fp32")
    out, lse = _run_mla(case, idx)
    _compare(case, out, lse, ref, "tiny")


SMALL_LENS = [3000, 2048, 5000, 700, 2049]
SMALL_Q = [(0, 2999), (1, 2047), (2, 4999), (2, 2500), (3, 699), (4, 2048), (0, 10)]


@pytest.mark.parametrize("precision", ["bf16", "mxfp8"])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_mla_full_dims_small(precision, out_dtype):
    case = make_custom(SMALL_LENS, SMALL_Q, dims=FULL_DIMS, precision=precision, seed=5,
                       device="cuda", out_dtype=out_dtype, softmax_scale=1 / 24)
    ref, idx = _oracle(case)
    say(f"case mla {precision} out={out_dtype}")
    out, lse = _run_mla(case, idx)
    _compare(case, out, lse, ref, f"{precision}/{out_dtype}")


# Enough queries that one split workgroup takes several rounds of 128 rows
# (40 x 16 groups of 128 exceed the CU count, so 4 rounds of 4 splits), with
# queries short of k (padded lists) among them.
ROUND_LENS = [2600, 3100, 2300, 4000]
ROUND_Q = [(b, p) for b, (L, ps) in enumerate(zip(ROUND_LENS, [(0.3, 0.8, 0.99), (0.5, 0.7, 0.9, 0.999),
                                                              (0.2, 0.6, 0.95), (0.1, 0.4, 0.55, 0.999)]))
           for p in [int(L * f) for f in ps]]
ROUND_Q = (ROUND_Q * 3)[:40]


@pytest.mark.parametrize("precision", ["bf16", "mxfp8"])
def test_mla_split_rounds(precision):
    case = make_custom(ROUND_LENS, ROUND_Q, dims=FULL_DIMS, precision=precision, seed=9,
                       device="cuda", softmax_scale=1 / 24)
    ref, idx = _oracle(case)
    say(f"case mla rounds {precision}, {case.num_q} queries")
    out, lse = _run_mla(case, idx)
    _compare(case, out, lse, ref, f"rounds/{precision}")


def test_mla_order_invariance_and_invalid_entries():
    case = make_custom(SMALL_LENS, SMALL_Q, dims=FULL_DIMS, precision="bf16", seed=6,
                       device="cuda", softmax_scale=1 / 24)
    ref, idx = _oracle(case)
    g = torch.Generator(device="cpu").manual_seed(3)
    perm = torch.stack([torch.randperm(idx.shape[1], generator=g) for _ in range(idx.shape[0])])
    shuffled = torch.gather(idx.cpu(), 1, perm).cuda()
    # entries past the cache end are skipped like -1 padding
    bad = shuffled.clone()
    bad[bad < 0] = 1 << 30
    say("case mla order invariance")
    o1, l1 = _run_mla(case, idx)
    o2, l2 = _run_mla(case, shuffled)
    o3, _ = _run_mla(case, bad)
    _compare(case, o2, l2, ref, "shuffled")
    check_close(to_np(o2), to_np(o1), case, "shuffled vs sorted")
    assert torch.equal(o2, o3)


def test_mla_gate_plus_inf_is_ungated_and_minus_inf_is_zero():
    case = make_custom(SMALL_LENS, SMALL_Q, dims=FULL_DIMS, precision="bf16", seed=7,
                       device="cuda", softmax_scale=1 / 24)
    _, idx = _oracle(case)
    say("case mla gate limits")
    ungated, _ = _run_mla(case, idx, gate=None)
    pinf, _ = _run_mla(case, idx, gate=torch.full_like(case.gate, float("inf")))
    ninf, _ = _run_mla(case, idx, gate=torch.full_like(case.gate, float("-inf")))
    half, _ = _run_mla(case, idx, gate=torch.zeros_like(case.gate), out_dtype="f32")
    ungated32, _ = _run_mla(case, idx, gate=None, out_dtype="f32")
    assert torch.equal(pinf, ungated)
    assert torch.count_nonzero(ninf.float()) == 0
    assert torch.equal(half, ungated32 * 0.5)


def test_mla_constant_channel_sums_to_one():
    case = make_custom(SMALL_LENS, SMALL_Q, dims=FULL_DIMS, precision="bf16", seed=8,
                       device="cuda", softmax_scale=1 / 24)
    case.kv[:, 5] = 1.0
    case.kv[:, 300] = 1.0
    _, idx = _oracle(case)
    say("case mla constant channel")
    out, _ = _run_mla(case, idx, gate=None, out_dtype="f32")
    for c in (5, 300):
        assert float((out[:, :, c] - 1.0).abs().max()) <= 1e-2


def test_mla_no_valid_rows():
    case = make_custom([100, 50], [(0, 99), (1, 49)], dims=FULL_DIMS, precision="bf16", seed=9,
                       device="cuda", softmax_scale=1 / 24)
    idx = torch.full((2, 2048), -1, dtype=torch.int32, device="cuda")
    idx[1, :10] = 5000  # beyond the sequence: skipped
    say("case mla no valid rows")
    out, lse = _run_mla(case, idx)
    assert torch.count_nonzero(out.float()) == 0
    assert bool(torch.all(torch.isneginf(lse)))


# More than twice as many queries as CUs: the whole-query kernel (bf16 rows,
# contiguous cache) takes several queries per workgroup and writes outputs
# directly. Short index lists keep the oracle cheap while every workgroup
# crosses many query and 128-row chunk boundaries; k = 200 leaves a partial
# chunk and a partial tile; some queries see fewer than k positions (padded
# lists) and one has no valid entry at all.
WQ_LENS = [700, 300, 1000, 450, 2500]


def _wq_case(k, seed, gated=True, out_dtype=None):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    T = 2 * cus + 37
    rng = np.random.default_rng(seed)
    queries = []
    for i in range(T):
        b = i % len(WQ_LENS)
        queries.append((b, int(rng.integers(0, WQ_LENS[b]))))
    return make_custom(WQ_LENS, queries, dims=dict(FULL_DIMS, topk=k), precision="bf16", seed=seed,
                       device="cuda", gated=gated, out_dtype=out_dtype, softmax_scale=1 / 24)


@pytest.mark.parametrize("k,out_dtype", [(256, "bf16"), (200, "f32")])
def test_mla_whole_queries(k, out_dtype):
    case = _wq_case(k, 13 + k, out_dtype=out_dtype)
    ref, idx = _oracle(case)
    empty = 7
    idx[empty] = -1
    say(f"case mla whole queries k={k} out={out_dtype}, {case.num_q} queries")
    out, lse = _run_mla(case, idx)
    keep = np.array([t for t in range(case.num_q) if t != empty])
    kt = torch.as_tensor(keep, device="cuda")
    sub = {"y": ref["y"][keep], "lse": ref["lse"][keep]}
    _compare(case, out[kt], lse[kt], sub, f"whole/{k}")
    assert torch.count_nonzero(out[empty].float()) == 0
    assert bool(torch.all(torch.isneginf(lse[empty])))


def test_mla_whole_queries_ungated():
    case = _wq_case(256, 21, gated=False)
    ref, idx = _oracle(case)
    say(f"case mla whole queries ungated, {case.num_q} queries")
    out, lse = _run_mla(case, idx, gate=None)
    _compare(case, out, lse, ref, "whole/ungated")
