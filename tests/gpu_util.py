"""Helpers for the GPU parity tests: run the HIP path on a generated case and
compare with the oracle. Tolerances are the acceptance bars of the method:
index sets bit-exact; outputs within 1e-5 * max|ref| (fp32) or
2e-2 * max|ref| + 1e-3 (bf16 / FP8 / MXFP8)."""

from __future__ import annotations

import sys
from typing import Dict, Optional, Sequence

import numpy as np
import torch

import sparse_top_latent_amd as sga
from oracle import case as ocase


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tol(case) -> float:
    return 1e-5 if case.q_dtype == "f32" else 2e-2


def check_close(y_gpu: np.ndarray, y_ref: np.ndarray, case, what: str = "y") -> float:
    scale = float(np.max(np.abs(y_ref))) if y_ref.size else 0.0
    bound = tol(case) * scale + (0.0 if case.q_dtype == "f32" else 1e-3)
    err = float(np.max(np.abs(y_gpu - y_ref))) if y_ref.size else 0.0
    assert err <= bound, f"{what}: max|diff| {err:.3e} > bound {bound:.3e} (max|ref| {scale:.3e})"
    return err


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_layer(case, prob: Optional[sga.Problem] = None, *, lse=True, want_idx=True):
    prob = prob or sga.Problem.from_case(case)
    T, H, Dc = case.num_q, case.heads, case.d_latent
    out = torch.empty((T, H, Dc), dtype=sga.out_torch_dtype(prob.c.out_dtype), device="cuda")
    idx = torch.empty((T, prob.c.topk), dtype=torch.int32, device="cuda") if want_idx else None
    lse_t = torch.empty((T, H), dtype=torch.float32, device="cuda") if lse else None
    ws = sga.workspace(prob, sga.SGA_OP_LAYER)
    sga.sga_layer_fwd(prob, case.q_idx, case.w, case.k_idx, case.q, case.kv, case.kv_scale,
                      case.gate, out, idx, lse_t, ws)
    torch.cuda.synchronize()
    return out, idx, lse_t


def run_scores(case, prob: Optional[sga.Problem] = None):
    prob = prob or sga.Problem.from_case(case)
    scores = torch.full((case.num_q, prob.c.max_kv_len), float("nan"), device="cuda")
    sga.sga_index_scores(prob, case.q_idx, case.w, case.k_idx, scores)
    torch.cuda.synchronize()
    return scores


def compare_layer(case, queries: Optional[Sequence[int]] = None, *, out=None, idx=None, lse=None,
                  label="") -> Dict[str, float]:
    """Run (or take) the layer outputs and compare the listed queries with the oracle."""
    if out is None:
        out, idx, lse = run_layer(case)
    qs = list(range(case.num_q)) if queries is None else list(queries)
    ref = ocase.run_queries(case, qs, keep_scores=False)
    assert all(ref["scores_exact"]), "score exactness bound violated by the inputs"
    got_idx = idx[qs].cpu().numpy().astype(np.int64)
    bad = np.nonzero(np.any(got_idx != ref["topk_idx"], axis=1))[0]
    assert bad.size == 0, f"{label}: top-k differs for queries {[qs[i] for i in bad[:8]]}"
    err = check_close(to_np(out[qs]), ref["y"], case, f"{label} y")
    lerr = 0.0
    if lse is not None:
        lg, lr = lse[qs].cpu().numpy().astype(np.float64), ref["lse"]
        fin = np.isfinite(lr)
        assert np.array_equal(fin, np.isfinite(lg)), f"{label}: lse finiteness differs"
        if fin.any():
            lerr = float(np.max(np.abs(lg[fin] - lr[fin])))
            assert lerr <= (1e-5 if case.q_dtype == "f32" else 2e-2) * max(1.0, float(np.max(np.abs(lr[fin])))), \
                f"{label}: lse max|diff| {lerr:.3e}"
    return {"y_err": err, "lse_err": lerr}
