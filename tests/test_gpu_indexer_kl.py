"""GPU parity of the indexer KL loss and its gradients (sga_indexer_kl).

The forward pass (sga_layer_fwd) supplies the selection and the per-head
log-sum-exp; the oracle (oracle.case.kl_queries) recomputes everything in
float64 from the same inputs. The loss and the gradients are fp32 results
of long sums (attention logits over 576 values, 2,048 selected keys), so they
are compared within 2e-4 of the largest reference magnitude of each tensor
(plus 1e-7 absolute); the selection itself is bit-exact (the layer tests
cover it).
"""

import numpy as np
import pytest
import torch

import sparse_top_latent_amd as sga
from gpu_util import run_layer, say
from oracle import case as ocase
from sga_inputs import make_case, make_custom, paged_copy
from sga_inputs.gen import FULL_DIMS

pytestmark = pytest.mark.gpu

TOL = 2e-4


def _close(got, ref, what):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    bound = TOL * float(np.max(np.abs(ref))) + 1e-7 if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert err <= bound, f"{what}: max|diff| {err:.3e} > {bound:.3e}"


def run_kl(case):
    prob = sga.Problem.from_case(case)
    _, idx, lse = run_layer(case, prob)
    T, HI, DI = case.num_q, case.idx_heads, case.idx_dim
    loss = torch.full((T,), float("nan"), device="cuda")
    d_w = torch.full((T, HI), float("nan"), device="cuda")
    d_q = torch.full((T, HI, DI), float("nan"), device="cuda")
    d_k = torch.zeros((case.num_kv_rows, DI), device="cuda")
    ws = sga.workspace(prob, sga.SGA_OP_INDEXER_KL)
    sga.sga_indexer_kl(prob, case.q_idx, case.w, case.k_idx, case.q, case.kv, case.kv_scale, idx, lse,
                       loss, d_w, d_q, d_k, ws)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), d_w.cpu().numpy(), d_q.cpu().numpy(), d_k


def _check(case, label):
    say(f"case indexer KL {label}: T={case.num_q} rows={case.num_kv_rows}")
    loss, d_w, d_q, d_k = run_kl(case)
    ref = ocase.kl_queries(case)
    _close(loss, ref["loss"], f"{label} loss")
    for i in range(case.num_q):
        _close(d_w[i], ref["dw"][i], f"{label} d_w[{i}]")
        _close(d_q[i], ref["dq_idx"][i], f"{label} d_q_idx[{i}]")
    rows = np.array(sorted(ref["dk_idx"]), dtype=np.int64)
    dk_ref = np.stack([ref["dk_idx"][r] for r in rows]) if rows.size else np.zeros((0, case.idx_dim))
    got = d_k.index_select(0, torch.as_tensor(rows, device="cuda")).cpu().numpy()
    _close(got, dk_ref, f"{label} d_k_idx (selected rows)")
    other = torch.ones(case.num_kv_rows, dtype=torch.bool, device="cuda")
    other[torch.as_tensor(rows, device="cuda")] = False
    assert float(d_k[other].abs().max()) == 0.0 if bool(other.any()) else True, f"{label}: rows outside the selections changed"
    assert np.all(loss >= -1e-4)


def test_indexer_kl_decode_ragged():
    lens = [20000, 4097, 64, 9000, 3000, 2048, 1]
    qs = [(b, n - 1) for b, n in enumerate(lens)] + [(0, 1500), (3, 8000)]
    case = make_custom(lens, qs, dims=FULL_DIMS, precision="bf16", seed=61, device="cuda")
    _check(case, "decode ragged")


def test_indexer_kl_tiny_fp32_all_queries():
    # 512 queries of one sequence: the selected rows overlap, so d_k_idx sums
    # many queries' contributions through the atomics
    _check(make_case("tiny_fp32_L512", device="cuda"), "tiny fp32")


def test_indexer_kl_mxfp8_paged():
    lens = [7000, 15000, 129]
    case = make_custom(lens, [(b, n - 1) for b, n in enumerate(lens)] + [(1, 9000)], dims=FULL_DIMS,
                       precision="mxfp8", seed=62, device="cuda")
    _check(paged_copy(case, 256, seed=5), "mxfp8 paged")
