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


def test_graph_decode_step_with_cache_append():
    # a serving decode step in one graph: the new token's latent row and index
    # key are appended (bf16 -> MXFP8 / FP8) at its slot, then the layer
    # attends with the new token as the last position; replays must match the
    # eager step bit for bit
    from sga_inputs import block_scaled_rows

    lens = [9000, 20000]
    case = make_custom(lens, [(0, 8999), (1, 19999)], dims=FULL_DIMS, precision="mxfp8", seed=33,
                       device="cuda", softmax_scale=1 / 24)
    say("case graph replay: cache append + layer")
    prob = sga.Problem.from_case(case)
    new_kv = block_scaled_rows(2, 576, 34, "graph.kv", spread=2, device="cuda")
    new_ki = (torch.randint(-8, 9, (2, 128), device="cuda").float()).to(torch.bfloat16)
    slots = (case.kv_start + case.kv_len.long() - 1).contiguous()
    T = case.num_q
    out = torch.empty((T, 64, 512), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((T, 2048), dtype=torch.int32, device="cuda")
    lse = torch.empty((T, 64), dtype=torch.float32, device="cuda")
    ws = sga.workspace(prob, sga.SGA_OP_LAYER)
    kv0, sc0, ki0 = case.kv.clone(), case.kv_scale.clone(), case.k_idx.clone()

    def step():
        sga.sga_cache_append(prob, new_kv, new_ki, slots, case.kv, case.kv_scale, case.k_idx)
        _layer(case, prob, out, idx, lse, ws)

    step()
    torch.cuda.synchronize()
    ref = (out.clone(), idx.clone(), lse.clone(), case.kv.clone(), case.kv_scale.clone(), case.k_idx.clone())
    assert not torch.equal(case.kv, kv0) and not torch.equal(case.k_idx, ki0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        # restore the caches eagerly, then replay
        case.kv.copy_(kv0)
        case.kv_scale.copy_(sc0)
        case.k_idx.copy_(ki0)
        out.zero_()
        idx.fill_(-5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (out, idx, lse, case.kv, case.kv_scale, case.k_idx)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {r} differs from the eager step"
