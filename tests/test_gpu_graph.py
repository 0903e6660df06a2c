"""The layer captured in a HIP graph: every replay must reproduce the eager
result bit for bit, also with other eager GPU work between replays."""

import pytest
import torch

import sparse_top_latent_amd as sga
from gpu_util import say
from sga_inputs import make_custom
from sga_inputs.gen import FULL_DIMS

pytestmark = pytest.mark.gpu


def _layer(case, prob, out, idx, lse, ws):
    sga.sga_layer_fwd(prob, case.q_idx, case.w, case.k_idx, case.q, case.kv, case.kv_scale,
                      case.gate, out, idx, lse, ws)


@pytest.mark.parametrize("precision", ["bf16", "mxfp8"])
def test_graph_replays_match_eager(precision):
    case = make_custom([20000, 9000, 1500], [(0, 19999), (1, 8999), (2, 1499), (0, 5000)],
                       dims=FULL_DIMS, precision=precision, seed=31, device="cuda",
                       softmax_scale=1 / 24)
    other = make_custom([12000], [(0, 11999)], dims=FULL_DIMS, precision="bf16", seed=32,
                        device="cuda", softmax_scale=1 / 24)
    say(f"case graph replay {precision}")
    prob = sga.Problem.from_case(case)
    oprob = sga.Problem.from_case(other)
    T = case.num_q
    out = torch.empty((T, 64, 512), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((T, 2048), dtype=torch.int32, device="cuda")
    lse = torch.empty((T, 64), dtype=torch.float32, device="cuda")
    ws = sga.workspace(prob, sga.SGA_OP_LAYER)
    oout = torch.empty((1, 64, 512), dtype=torch.bfloat16, device="cuda")
    ows = sga.workspace(oprob, sga.SGA_OP_LAYER)
    _layer(case, prob, out, idx, lse, ws)
    torch.cuda.synchronize()
    ref = (out.clone(), idx.clone(), lse.clone())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _layer(case, prob, out, idx, lse, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _layer(case, prob, out, idx, lse, ws)
    for rep in range(4):
        out.zero_()
        idx.fill_(-5)
        lse.zero_()
        # unrelated eager work between replays (its own workspace)
        _layer(other, oprob, oout, None, None, ows)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[1]), f"replay {rep}: top-k differs"
        assert torch.equal(out, ref[0]), f"replay {rep}: output differs"
        assert torch.equal(lse, ref[2]), f"replay {rep}: lse differs"
