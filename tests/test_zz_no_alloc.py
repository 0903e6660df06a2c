"""GPU check of sga_layer_fwd_noalloc (the layer call on the library's static
per-GPU scratch) against sga_layer_fwd with a caller workspace: the same
kernels on the same inputs, so outputs, top-k lists and log-sum-exps must be
bit-identical. Two calls in a row, the second with a smaller problem, so the
second runs on scratch the first left behind."""

import numpy as np
import pytest
import torch

import sparse_top_latent_amd as sga
from gpu_util import compare_layer, say
from sga_inputs import make_case, make_custom
from sga_inputs.gen import FULL_DIMS

pytestmark = pytest.mark.gpu


def _outputs(case, prob):
    T, H, Dc = case.num_q, case.heads, case.d_latent
    out = torch.full((T, H, Dc), float("nan"), dtype=sga.out_torch_dtype(prob.c.out_dtype), device="cuda")
    idx = torch.full((T, prob.c.topk), -7, dtype=torch.int32, device="cuda")
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    return out, idx, lse


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else (t.view(torch.int32) if t.dtype == torch.float32 else t)


def _run_both(case, label):
    prob = sga.Problem.from_case(case)
    ref = _outputs(case, prob)
    ws = sga.workspace(prob, sga.SGA_OP_LAYER)
    sga.sga_layer_fwd(prob, case.q_idx, case.w, case.k_idx, case.q, case.kv, case.kv_scale, case.gate,
                      *ref, ws)
    got = _outputs(case, prob)
    say(f"case no-alloc layer {label}: T={case.num_q}, workspace {ws.numel() / 2**20:.1f} MiB")
    sga.sga_layer_fwd_noalloc(prob, case.q_idx, case.w, case.k_idx, case.q, case.kv, case.kv_scale,
                              case.gate, *got)
    torch.cuda.synchronize()
    for a, b, what in zip(ref, got, ("y", "top-k", "lse")):
        assert torch.equal(_bits(a), _bits(b)), f"{label}: {what} differs from sga_layer_fwd"
    return got


def test_noalloc_layer_matches_workspace_layer_twice():
    # first call: the 16 x 128K decode batch (48.9 MiB of scratch)
    big = make_case("decode_b16_n128k", device="cuda")
    out, idx, lse = _run_both(big, "decode_b16_n128k")
    compare_layer(big, [0, 15], out=out, idx=idx, lse=lse, label="no-alloc decode_b16_n128k")
    del big
    # second call, smaller and ragged (MXFP8 rows, one short sequence)
    lens = [9000, 3000, 2048, 70]
    small = make_custom(lens, [(0, 8999), (1, 2999), (2, 2047), (3, 69), (0, 4000)], dims=FULL_DIMS,
                        precision="mxfp8", seed=71, device="cuda")
    out, idx, lse = _run_both(small, "ragged mxfp8")
    compare_layer(small, out=out, idx=idx, lse=lse, label="no-alloc ragged")


def test_noalloc_layer_rejects_oversized_problem():
    case = make_case("decode_b16_n128k_mq4", device="cuda")  # 64 queries: about 196 MiB
    prob = sga.Problem.from_case(case)
    out, idx, lse = _outputs(case, prob)
    with pytest.raises(sga.SgaError) as e:
        sga.sga_layer_fwd_noalloc(prob, case.q_idx, case.w, case.k_idx, case.q, case.kv, case.kv_scale,
                                  case.gate, out, idx, lse)
    assert e.value.status == 3
