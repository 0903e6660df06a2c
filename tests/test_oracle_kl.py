"""Pins for the oracle's indexer KL loss and gradients (CPU only).

The loss is checked against torch's kl_div on log_softmax (a library
routine); every gradient against central finite differences of the oracle's
own loss, which does not share the closed forms; plus the invariants of a
KL divergence.
"""

import numpy as np
import torch

from oracle import kl


def _loss_of(I, target):
    return kl.indexer_kl(I, target)[0]


def test_loss_matches_torch_kl_div():
    g = np.random.default_rng(0)
    for m in (1, 5, 300):
        I = g.standard_normal(m) * 3
        p = g.random((4, m))
        p /= p.sum(axis=1, keepdims=True)
        t = kl.attention_target(p)
        ref = torch.nn.functional.kl_div(torch.log_softmax(torch.tensor(I), 0), torch.tensor(t),
                                         reduction="sum").item()
        assert abs(_loss_of(I, t) - ref) <= 1e-12 * max(1.0, abs(ref))


def test_gradient_wrt_scores_by_finite_differences():
    g = np.random.default_rng(1)
    I = g.standard_normal(40) * 2
    t = g.random(40)
    t[3] = 0.0  # a zero-target term
    t /= t.sum()
    _, grad = kl.indexer_kl(I, t)
    h = 1e-6
    for s in range(40):
        e = np.zeros(40)
        e[s] = h
        fd = (_loss_of(I + e, t) - _loss_of(I - e, t)) / (2 * h)
        assert abs(fd - grad[s]) < 1e-7


def test_kl_invariants():
    g = np.random.default_rng(2)
    t = g.random(50)
    t /= t.sum()
    for _ in range(5):
        I = g.standard_normal(50) * 4
        loss, grad = kl.indexer_kl(I, t)
        assert loss >= 0 and abs(grad.sum()) < 1e-12
    loss, grad = kl.indexer_kl(np.log(t) + 7.25, t)  # the indexer already matches the target
    assert abs(loss) < 1e-12 and np.abs(grad).max() < 1e-12
    assert kl.indexer_kl(np.zeros(0), np.zeros(0))[0] == 0.0


def test_attention_target():
    g = np.random.default_rng(3)
    p = g.random((8, 30))
    p /= p.sum(axis=1, keepdims=True)
    t = kl.attention_target(p)
    assert abs(t.sum() - 1) < 1e-12
    assert np.allclose(kl.attention_target(p[:1]), p[0])
    assert np.allclose(t, p.mean(axis=0))


def test_indexer_gradients_by_finite_differences():
    g = np.random.default_rng(4)
    HI, DI, m = 3, 5, 7
    q = g.standard_normal((HI, DI))
    w = g.standard_normal(HI)
    k = g.standard_normal((m, DI))
    t = g.random(m)
    t /= t.sum()

    def loss(q, w, k):
        z = q @ k.T
        return _loss_of(np.maximum(z, 0).T @ w, t)

    z = q @ k.T
    assert np.abs(z).min() > 1e-3  # no ReLU kink within the step
    I = np.maximum(z, 0).T @ w
    _, gI = kl.indexer_kl(I, t)
    dw, dq, dk = kl.indexer_backward(q, w, k, gI)
    h = 1e-7
    for arr, grad in ((w, dw), (q, dq), (k, dk)):
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            up = loss(q, w, k)
            arr[idx] = old - h
            dn = loss(q, w, k)
            arr[idx] = old
            assert abs((up - dn) / (2 * h) - grad[idx]) < 1e-6, (idx, grad[idx])


def test_case_level_kl_on_the_tiny_case():
    # the case glue against the step functions run by hand on one query
    from oracle import case as ocase
    from oracle import sga
    from sga_inputs import make_case

    c = make_case("tiny_fp32_L512")
    r = ocase.kl_queries(c, [300, 511])
    assert r["loss"].shape == (2,) and np.all(r["loss"] >= 0)
    t = 511
    d = ocase.decode_all(c)
    s = sga.index_scores(d["q_idx"][t], d["w"][t], d["k_idx"][:512])
    sel = sga.select_topk(sga.to_fp32(s), c.topk)
    _, _, p = sga.attend(d["q"][t], d["kv"][sel], c.softmax_scale, c.d_latent)
    loss, g = kl.indexer_kl(s[sel], kl.attention_target(p))
    dw, dq, _ = kl.indexer_backward(d["q_idx"][t], d["w"][t], d["k_idx"][sel], g)
    assert abs(r["loss"][1] - loss) < 1e-12 and np.allclose(r["dw"][1], dw) and np.allclose(r["dq_idx"][1], dq)
    # rows selected by both queries collect both contributions
    assert len(r["dk_idx"]) >= c.topk


def _golden_case(layout):
    """The hand-worked two-query case of tests/golden/kl_two_queries_shared_row.json
    as a case object (contiguous or paged caches); cache rows that hold no
    position carry other keys, so keying by the wrong row changes the result."""
    import json
    import os
    from types import SimpleNamespace

    with open(os.path.join(os.path.dirname(__file__), "golden", "kl_two_queries_shared_row.json")) as f:
        gold = json.load(f)
    c = gold["case"]
    lay = c[layout]
    rows = lay["rows_by_position"]
    n_rows = lay["num_kv_rows"]
    k_idx = torch.full((n_rows, c["index_dim"]), 5.0)
    for pos, r in enumerate(rows):
        k_idx[r] = torch.tensor(c["keys_by_position"][pos], dtype=torch.float32)
    H, Dc, Dr = 2, 2, 1
    case = SimpleNamespace(
        num_q=2, q_seq=torch.zeros(2, dtype=torch.int32),
        q_pos=torch.tensor([q["position"] for q in c["queries"]], dtype=torch.int32),
        kv_start=torch.tensor([lay.get("kv_start", 0)], dtype=torch.int64),
        kv_len=torch.tensor([3], dtype=torch.int32),
        page_size=lay.get("page_size", 0),
        block_table=torch.tensor([lay["block_table"]], dtype=torch.int32) if "block_table" in lay else None,
        num_kv_rows=n_rows, idx_dtype="f32", idx_heads=c["index_heads"], idx_dim=c["index_dim"],
        q_idx=torch.tensor([[q["q_idx"]] for q in c["queries"]], dtype=torch.float32),
        w=torch.tensor([c["w"], c["w"]], dtype=torch.float32), k_idx=k_idx,
        kv=torch.randn(n_rows, Dc + Dr, generator=torch.Generator().manual_seed(0)),
        kv_dtype="f32", kv_scale=None, q=torch.zeros(2, H, Dc + Dr), q_dtype="f32",
        heads=H, d_latent=Dc, d_rope=Dr, softmax_scale=1.0, topk=c["topk"])
    return case, rows, gold["expected"]


def test_kl_case_golden_two_queries_share_a_row():
    # d_k_idx sums the contributions of every query that selects a cache row,
    # keyed by the cache row (not the position), in both cache layouts
    import math

    from oracle import case as ocase

    for layout in ("contiguous", "paged"):
        case, rows, exp = _golden_case(layout)
        assert abs(exp["tau"] - math.tanh(0.5)) < 1e-15
        r = ocase.kl_queries(case)
        assert np.allclose(r["loss"], exp["loss"], rtol=0, atol=1e-12), layout
        assert np.allclose(r["dw"], exp["d_w"], rtol=0, atol=1e-12), layout
        assert np.allclose(r["dq_idx"], exp["d_q_idx"], rtol=0, atol=1e-12), layout
        want = {rows[int(p)]: np.array(v) for p, v in exp["d_k_by_position"].items()}
        assert set(r["dk_idx"]) == set(want), (layout, sorted(r["dk_idx"]), sorted(want))
        for row, v in want.items():
            assert np.allclose(r["dk_idx"][row], v, rtol=0, atol=1e-12), (layout, row)


def test_kl_case_refuses_page_ids_outside_the_cache():
    import pytest

    from oracle import case as ocase

    case, _, _ = _golden_case("paged")
    case.block_table[0, 1] = 4  # 8 rows in pages of 2: ids 0..3 exist
    with pytest.raises(ValueError):
        ocase.kl_queries(case)
