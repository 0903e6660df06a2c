"""Generator determinism and the oracle glue on generated cases (CPU only)."""

import math

import numpy as np
import torch

from oracle import case as ocase
from oracle import sga
from sga_inputs import make_case, make_custom
from sga_inputs.gen import FULL_DIMS, hash32, varlen_lengths


def test_hash_is_deterministic_and_spread():
    a = hash32(0, "x", torch.arange(1 << 16))
    b = hash32(0, "x", torch.arange(1 << 16))
    c = hash32(1, "x", torch.arange(1 << 16))
    assert torch.equal(a, b) and not torch.equal(a, c)
    assert 0 <= int(a.min()) and int(a.max()) < 2 ** 32
    # each bit is close to fair
    bits = torch.stack([(a >> i) & 1 for i in range(32)]).float().mean(dim=1)
    assert float((bits - 0.5).abs().max()) < 0.01
    # counters >= 2^32 differ from their low halves
    big = torch.tensor([5, 5 + (1 << 32)], dtype=torch.int64)
    h = hash32(0, "x", big)
    assert int(h[0]) != int(h[1])


def test_tiny_config_shapes_and_dyadic_weights():
    c = make_case("tiny_fp32_L512")
    assert c.q.shape == (512, 8, 80) and c.kv.shape == (512, 80)
    assert c.q_idx.shape == (512, 2, 32) and c.k_idx.shape == (512, 32)
    assert c.gate.shape == (512, 8, 64) and c.topk == 64
    assert math.isclose(c.softmax_scale, 1 / math.sqrt(80))
    assert torch.equal(c.q_idx, c.q_idx.round()) and float(c.q_idx.abs().max()) <= 4
    assert torch.equal(c.w * 1024, (c.w * 1024).round())
    assert torch.equal(c.q_pos, torch.arange(512, dtype=torch.int32))


def test_same_seed_same_bytes():
    a = make_custom([100, 37], [(0, 99), (1, 20)], dims=FULL_DIMS, precision="mxfp8", seed=3)
    b = make_custom([100, 37], [(0, 99), (1, 20)], dims=FULL_DIMS, precision="mxfp8", seed=3)
    for k in ("q", "kv", "kv_scale", "q_idx", "k_idx", "w", "gate"):
        assert torch.equal(getattr(a, k).view(torch.uint8) if getattr(a, k).dtype == torch.bfloat16
                           else getattr(a, k),
                           getattr(b, k).view(torch.uint8) if getattr(b, k).dtype == torch.bfloat16
                           else getattr(b, k))
    sc = a.kv_scale.int() - 127
    assert int(sc.min()) == -4 and int(sc.max()) == 4


def test_varlen_lengths_range():
    L = varlen_lengths(0)
    assert len(L) == 64 and min(L) >= 4096 and max(L) <= 262144
    logs = np.log(L)
    assert abs(np.mean((logs - math.log(4096)) / (math.log(262144) - math.log(4096))) - 0.5) < 0.15


def test_tiny_scores_exact_in_fp32_for_every_query():
    c = make_case("tiny_fp32_L512")
    res = ocase.run_queries(c, keep_scores=False)
    assert all(res["scores_exact"])


def test_full_shape_scores_exact_in_fp32():
    # a 4,096-key sequence with the decode dtypes: the dyadic w keeps fp32 exact
    c = make_custom([4096], [(0, 4095)], dims=FULL_DIMS, precision="bf16", seed=0)
    res = ocase.run_queries(c)
    assert res["scores_exact"] == [True]
    assert float(res["scores"][0].max()) < 2 ** 16


def test_case_glue_matches_direct_oracle_call():
    c = make_custom([70, 9], [(0, 69), (0, 30), (1, 8), (1, 0)], dims=dict(
        heads=2, d_latent=32, d_rope=32, idx_heads=3, idx_dim=8, topk=16), precision="mxfp8")
    res = ocase.run_queries(c)
    d = ocase.decode_all(c)
    ref = sga.sga_forward(**d, topk=16, tau=c.softmax_scale, d_latent=32)
    assert np.array_equal(res["topk_idx"], ref["topk_idx"])
    assert np.max(np.abs(res["y"] - ref["y"])) == 0.0


def test_paged_copy_keeps_every_logical_row_and_the_oracle_agrees():
    from oracle import case as ocase
    from sga_inputs import make_case, paged_copy

    c = make_case("tiny_fp32_L512")
    for P in (64, 128):
        p = paged_copy(c, P, seed=P)
        table = p.block_table.numpy()
        assert table.shape == (1, 512 // P)
        assert sorted(table[0].tolist()) == sorted(set(table[0].tolist()))  # distinct pages
        assert p.num_kv_rows == (512 // P + 3) * P
        rows = ocase.cache_rows(p, 0, np.arange(512), None, table)
        assert torch.equal(p.kv[torch.as_tensor(rows)], c.kv)
        assert torch.equal(p.k_idx[torch.as_tensor(rows)], c.k_idx)
        ref, got = ocase.run_queries(c, [0, 100, 511]), ocase.run_queries(p, [0, 100, 511])
        assert np.array_equal(ref["topk_idx"], got["topk_idx"])
        assert np.array_equal(ref["y"], got["y"])
