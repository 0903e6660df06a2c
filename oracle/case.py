"""Glue: run the oracle on a generated case (test infrastructure).

A case is any object with the attributes of sga_inputs.SgaCase (torch
tensors in storage form, possibly on a GPU). Only the slices a query needs
are copied to the host and decoded, so sampled queries of multi-GB caches
stay cheap. No SGA arithmetic lives here; it all happens in `sga`.
"""

from __future__ import annotations

from typing import Dict, Iterable, Optional

import numpy as np

from . import formats, sga


def raw(t) -> np.ndarray:
    """A torch tensor in storage form -> NumPy array of its raw storage."""
    import torch

    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _dec(t, dtype: str, scales=None) -> np.ndarray:
    return formats.decode(raw(t), dtype, None if scales is None else raw(scales))


def cache_rows(case, b: int, positions: np.ndarray, kv_start: np.ndarray, table) -> np.ndarray:
    """Cache rows of positions of sequence b: kv_start[b] + s, or, in the paged
    layout, table[b, s // P] * P + s % P.

    A page id outside the cache has no defined meaning (the library leaves
    the result of such a query unspecified), so the oracle refuses it.
    """
    positions = np.asarray(positions, dtype=np.int64)
    if not case.page_size:
        return int(kv_start[b]) + positions
    P = int(case.page_size)
    pg = table[b, positions // P].astype(np.int64)
    if np.any((pg < 0) | (pg >= case.num_kv_rows // P)):
        raise ValueError(f"sequence {b}: a page id outside the cache; the result is undefined")
    return pg * P + positions % P


def seq_capacity(case, b: int, kv_len: np.ndarray) -> int:
    """Cached length of sequence b as the caches hold it (the paged layout
    holds at most max_pages * page_size positions)."""
    n = int(kv_len[b])
    if case.page_size:
        n = min(n, case.block_table.shape[1] * int(case.page_size))
    return n


def run_queries(case, queries: Optional[Iterable[int]] = None, *, keep_scores: bool = True,
                topk: Optional[int] = None) -> Dict[str, object]:
    """Oracle SGA forward on the listed queries of `case` (all by default)."""
    T = case.num_q
    qs = list(range(T)) if queries is None else [int(t) for t in queries]
    k = case.topk if topk is None else int(topk)
    q_seq = raw(case.q_seq).astype(np.int64)
    q_pos = raw(case.q_pos).astype(np.int64)
    kv_start = raw(case.kv_start).astype(np.int64)
    kv_len = raw(case.kv_len).astype(np.int64)
    table = raw(case.block_table).astype(np.int64) if case.page_size else None
    idx_dt = "fp8" if case.idx_dtype == "fp8" else "f32"
    H, Dc = case.heads, case.d_latent
    out_idx = np.full((len(qs), k), -1, dtype=np.int64)
    out_y = np.zeros((len(qs), H, Dc))
    out_lse = np.full((len(qs), H), -np.inf)
    scores, exact = [], []
    for i, t in enumerate(qs):
        import torch

        b = int(q_seq[t])
        n = sga.visible_count(q_pos[t], seq_capacity(case, b, kv_len))
        q_idx_t = _dec(case.q_idx[t], idx_dt)
        w_t = raw(case.w[t]).astype(np.float64)
        key_rows = torch.as_tensor(cache_rows(case, b, np.arange(n), kv_start, table),
                                   dtype=torch.int64, device=case.k_idx.device)
        keys = _dec(case.k_idx.index_select(0, key_rows), idx_dt)
        s64 = sga.index_scores(q_idx_t, w_t, keys)
        exact.append(sga.fp32_exact_bound(q_idx_t, w_t, keys))
        s32 = sga.to_fp32(s64)
        if keep_scores:
            scores.append(s32)
        sel = sga.select_topk(s32, k)
        out_idx[i] = sel
        chosen = sel[sel >= 0]
        rows_idx = torch.as_tensor(cache_rows(case, b, chosen, kv_start, table), dtype=torch.int64,
                                   device=case.kv.device)
        kv_rows = case.kv.index_select(0, rows_idx)
        if case.kv_dtype == "mxfp8":
            rows = _dec(kv_rows, "mxfp8", case.kv_scale.index_select(0, rows_idx))
        else:
            rows = _dec(kv_rows, case.kv_dtype)
        q_t = _dec(case.q[t], case.q_dtype)
        o, lse, _ = sga.attend(q_t, rows, case.softmax_scale, Dc)
        g = None if case.gate is None else _dec(case.gate[t], case.gate_dtype)
        out_y[i] = sga.output_gate(o, g)
        out_lse[i] = lse
    return {"scores": scores, "scores_exact": exact, "topk_idx": out_idx, "y": out_y,
            "lse": out_lse, "queries": np.array(qs, dtype=np.int64)}


def decode_all(case) -> Dict[str, np.ndarray]:
    """Every input of a (small) case decoded to float64, plus int64 metadata."""
    idx_dt = "fp8" if case.idx_dtype == "fp8" else "f32"
    kv = (_dec(case.kv, "mxfp8", case.kv_scale) if case.kv_dtype == "mxfp8"
          else _dec(case.kv, case.kv_dtype))
    return {
        "q": _dec(case.q, case.q_dtype),
        "kv": kv,
        "q_idx": _dec(case.q_idx, idx_dt),
        "k_idx": _dec(case.k_idx, idx_dt),
        "w": raw(case.w).astype(np.float64),
        "gate": None if case.gate is None else _dec(case.gate, case.gate_dtype),
        "q_seq": raw(case.q_seq).astype(np.int64),
        "q_pos": raw(case.q_pos).astype(np.int64),
        "kv_start": raw(case.kv_start).astype(np.int64),
        "kv_len": raw(case.kv_len).astype(np.int64),
    }


def kl_queries(case, queries: Optional[Iterable[int]] = None) -> Dict[str, object]:
    """The indexer KL loss and its gradients (oracle.kl) for the listed queries.

    Every query's selection, attention probabilities and scores come from the
    oracle itself (run as in run_queries). Returns loss [Q], dw [Q, HI],
    dq_idx [Q, HI, DI] and d_k_idx as {cache row: [DI]} summed over the
    listed queries.
    """
    import torch

    from . import kl

    T = case.num_q
    qs = list(range(T)) if queries is None else [int(t) for t in queries]
    q_seq = raw(case.q_seq).astype(np.int64)
    q_pos = raw(case.q_pos).astype(np.int64)
    kv_start = raw(case.kv_start).astype(np.int64)
    kv_len = raw(case.kv_len).astype(np.int64)
    table = raw(case.block_table).astype(np.int64) if case.page_size else None
    idx_dt = "fp8" if case.idx_dtype == "fp8" else "f32"
    HI, DI, Dc = case.idx_heads, case.idx_dim, case.d_latent
    loss = np.zeros(len(qs))
    dw = np.zeros((len(qs), HI))
    dq = np.zeros((len(qs), HI, DI))
    dk: Dict[int, np.ndarray] = {}
    for i, t in enumerate(qs):
        b = int(q_seq[t])
        n = sga.visible_count(q_pos[t], seq_capacity(case, b, kv_len))
        q_idx_t = _dec(case.q_idx[t], idx_dt)
        w_t = raw(case.w[t]).astype(np.float64)
        key_rows = cache_rows(case, b, np.arange(n), kv_start, table)
        keys = _dec(case.k_idx.index_select(0, torch.as_tensor(key_rows, device=case.k_idx.device)),
                    idx_dt)
        s64 = sga.index_scores(q_idx_t, w_t, keys)
        sel = sga.select_topk(sga.to_fp32(s64), case.topk)
        chosen = sel[sel >= 0]
        rows_idx = torch.as_tensor(key_rows[chosen], dtype=torch.int64, device=case.kv.device)
        kv_rows = case.kv.index_select(0, rows_idx)
        rows = (_dec(kv_rows, "mxfp8", case.kv_scale.index_select(0, rows_idx))
                if case.kv_dtype == "mxfp8" else _dec(kv_rows, case.kv_dtype))
        _, _, p = sga.attend(_dec(case.q[t], case.q_dtype), rows, case.softmax_scale, Dc)
        target = kl.attention_target(p)
        loss[i], g = kl.indexer_kl(s64[chosen], target)
        dw[i], dq[i], dk_rows = kl.indexer_backward(q_idx_t, w_t, keys[chosen], g)
        for r, v in zip(key_rows[chosen].tolist(), dk_rows):
            dk[r] = dk.get(r, 0.0) + v
    return {"loss": loss, "dw": dw, "dq_idx": dq, "dk_idx": dk, "queries": np.array(qs, dtype=np.int64)}
