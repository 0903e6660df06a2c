"""Plain CPU oracle of the Sparse Gated Attention (SGA) forward hot path.

Test infrastructure only: see the package docstring.

Everything is float64 NumPy on decoded inputs, computed the slow, obvious way:
full score rows, a full sort for the selection, a two-pass softmax, then the
sigmoid gate. It shares nothing with the HIP library.

Sources (page title, then section):

* [AK2-ART] "A.X-K2: a sparse-attention upgrade that costs nothing, trained
  natively in FP8", section "Sparse Gated Attention".
* [AK2-NEWS] "SK Telecom Opens A.X K2: 688B Parameters and One Telling
  Benchmark", section "Sparse Gated Attention" and its block-diagram caption.
* [AK2-CARD] "A.X-K2" model card, sections "Sparse Gated Attention (SGA)" and
  "Model Details".
* [AK2-TR] "A.X K2 Technical Report": section 2 (architecture: MLA with a
  per-head output gate), section 3.4 (Stage 3C: an indexer whose selection
  holds 2,048 positions per query; YaRN with mscale 1.0) and the MXFP8 training
  paragraph.

Readings where the pages are silent (each is also listed in the design notes):

R1  indexer form: I[t, s] = sum_h w[t, h] * ReLU(qI[t, h] . kI[s]); one index
    key per cached token shared by all index heads; w per (query, head).
R2  scores are exact: inputs are integers and w is dyadic, so the exact real
    value is representable in fp32 (checked by `fp32_exact_bound`).
R3  -0.0 and +0.0 are the same score (the selection compares values).
R4  ties in score go to the lowest position.
R5  candidates are positions 0..p_t of the query's own sequence (its own key
    included), clipped to the cached length; no forced sink or window.
R6  if a query has n_t <= k candidates it keeps all of them; the index list is
    padded with -1.
R7  softmax runs over the selected set only.
R8  the softmax scale tau is an explicit input (no extra YaRN rescale).
R9  the gate is elementwise over [head, latent channel], applied to the
    latent-space output before any up/output projection.
R10 index lists are ascending positions (the output does not depend on order).
R11 a query with no candidates outputs y = 0 and lse = -inf.
R15 in the selection a NaN score ranks above every number (+inf included);
    NaNs tie with each other, so the lower position wins among them.
"""

from __future__ import annotations

from typing import Dict, Iterable, Optional

import numpy as np


# --------------------------------------------------------------------------
# step 1: indexer scores  ([AK2-ART], [AK2-NEWS], [AK2-CARD]: a cheap indexer
# rates each cached key for each query; readings R1, R2, R5)
# --------------------------------------------------------------------------
def visible_count(q_pos: int, kv_len: int) -> int:
    """Number of candidate positions of a query: positions 0..q_pos that are cached (R5)."""
    return max(0, min(int(q_pos) + 1, int(kv_len)))


def index_scores(q_idx_t: np.ndarray, w_t: np.ndarray, k_idx_rows: np.ndarray) -> np.ndarray:
    """Exact indexer scores of one query against n cached index keys.

    q_idx_t [HI, DI], w_t [HI], k_idx_rows [n, DI] (float64, decoded).
    Returns I [n] with I[s] = sum_h w[h] * max(0, q_idx_t[h] . k_idx_rows[s]).
    With integer q/k and dyadic w every product and partial sum is exact in
    float64, so this is the real value of the definition.
    """
    d = k_idx_rows @ q_idx_t.T            # [n, HI] head dot products
    r = np.maximum(d, 0.0)                # ReLU per head
    scores = r @ w_t                      # weighted sum over index heads
    return scores + 0.0                   # R3: -0.0 becomes +0.0


def fp32_exact_bound(q_idx_t: np.ndarray, w_t: np.ndarray, k_idx_rows: np.ndarray) -> bool:
    """True when every fp32 evaluation order of the score gives the exact value (R2).

    Sufficient condition: all of q, k are integers, w has at most g fractional
    bits, and for every key sum_h |w_h| r_h <= 2^(24 - g) and every head dot
    product |d| <= 2^24. Then each product, each partial sum (any order, any
    subset, with or without fused multiply-add) is a multiple of 2^-g below
    2^(24 - g) in magnitude and therefore representable in fp32.
    """
    if not (np.all(q_idx_t == np.round(q_idx_t)) and np.all(k_idx_rows == np.round(k_idx_rows))):
        return False
    g = 0
    while g <= 60 and not np.all(w_t * 2.0 ** g == np.round(w_t * 2.0 ** g)):
        g += 1
    if g > 60:
        return False
    absdot = np.abs(k_idx_rows) @ np.abs(q_idx_t).T
    if absdot.size and absdot.max() > 2.0 ** 24:
        return False
    r = np.maximum(k_idx_rows @ q_idx_t.T, 0.0)
    bound = r @ np.abs(w_t)
    return bool(bound.size == 0 or bound.max() <= 2.0 ** (24 - g))


def to_fp32(scores: np.ndarray) -> np.ndarray:
    """Round scores to fp32 (nearest-even) as the score buffer stores them; -0 -> +0."""
    return (scores.astype(np.float32) + np.float32(0.0)).astype(np.float32)


# --------------------------------------------------------------------------
# step 2: top-k selection  ([AK2-ART]: 2,048 single positions survive per
# query, chosen one by one rather than in blocks; [AK2-TR] section 3.4; readings R4, R6, R10)
# --------------------------------------------------------------------------
def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Positions of the k best scores, ordered by (score desc, position asc).

    A NaN score ranks above every number, +inf included, and NaNs tie with
    each other whatever their sign or payload (reading R15); -0 equals +0.
    Returns an int64 array of length k holding the chosen positions in
    ascending order, padded with -1 when fewer than k candidates exist.
    """
    n = scores.shape[0]
    out = np.full(k, -1, dtype=np.int64)
    if n <= k:
        out[:n] = np.arange(n)
        return out
    pos = np.arange(n)
    s64 = scores.astype(np.float64)
    nan = np.isnan(s64)
    value = np.where(nan, 0.0, s64)
    order = np.lexsort((pos, -value, ~nan))  # last key is primary: NaN class first
    out[:] = np.sort(order[:k])
    return out


# --------------------------------------------------------------------------
# step 3: MLA over the selected latent rows  ([AK2-ART]: MLA runs exactly
# over KV[I_topk]; [AK2-TR] section 2: MLA backbone; readings R7, R8, R11)
# --------------------------------------------------------------------------
def attend(q_t: np.ndarray, rows: np.ndarray, tau: float, d_latent: int):
    """Absorbed-form MLA for one query over gathered latent rows.

    q_t [H, Dc + Dr]; rows [m, Dc + Dr] = [c_s | kR_s] for the selected s.
    logit[h, s] = tau * (q_t[h, :Dc] . c_s + q_t[h, Dc:] . kR_s);
    p = softmax over the m selected rows (two passes: max, then exp/sum);
    o[h] = sum_s p[h, s] c_s (the 512-wide latent value);
    lse[h] = max + log(sum exp).
    Returns (o [H, Dc], lse [H], p [H, m]).
    """
    H = q_t.shape[0]
    m = rows.shape[0]
    if m == 0:
        return np.zeros((H, d_latent)), np.full(H, -np.inf), np.zeros((H, 0))
    logits = tau * (q_t[:, :d_latent] @ rows[:, :d_latent].T
                    + q_t[:, d_latent:] @ rows[:, d_latent:].T)
    mx = logits.max(axis=1)
    e = np.exp(logits - mx[:, None])
    z = e.sum(axis=1)
    p = e / z[:, None]
    o = p @ rows[:, :d_latent]
    lse = mx + np.log(z)
    return o, lse, p


# --------------------------------------------------------------------------
# step 4: per-head sigmoid gate on the output  ([AK2-ART]: learned,
# input-dependent gate on the attention output before Wo; [AK2-NEWS] caption:
# sigmoid output gate; [AK2-CARD]: head-specific; reading R9)
# --------------------------------------------------------------------------
def output_gate(o: np.ndarray, g: Optional[np.ndarray]) -> np.ndarray:
    """y = sigmoid(g) * o elementwise; g = None means ungated (y = o)."""
    if g is None:
        return o.copy()
    with np.errstate(over="ignore"):
        return o / (1.0 + np.exp(-g))


# --------------------------------------------------------------------------
# the whole path
# --------------------------------------------------------------------------
def sga_forward(
    *,
    q: np.ndarray,
    kv: np.ndarray,
    q_idx: np.ndarray,
    k_idx: np.ndarray,
    w: np.ndarray,
    gate: Optional[np.ndarray],
    q_seq: np.ndarray,
    q_pos: np.ndarray,
    kv_start: np.ndarray,
    kv_len: np.ndarray,
    topk: int,
    tau: float,
    d_latent: int,
    queries: Optional[Iterable[int]] = None,
    keep_scores: bool = True,
) -> Dict[str, object]:
    """SGA forward for the listed queries (all by default), from decoded float64 inputs.

    q [T, H, Dc+Dr], kv [rows, Dc+Dr], q_idx [T, HI, DI], k_idx [rows, DI],
    w [T, HI], gate [T, H, Dc] or None; metadata per query (q_seq, q_pos) and
    per sequence (kv_start, kv_len).

    Returns a dict with, per listed query in order: "scores" (list of fp32
    arrays over the candidates), "scores_exact" (list of bools, R2),
    "topk_idx" [T', k], "y" [T', H, Dc], "lse" [T', H], "queries" [T'].
    """
    T = q.shape[0]
    qs = list(range(T)) if queries is None else [int(t) for t in queries]
    H = q.shape[1]
    out_idx = np.full((len(qs), topk), -1, dtype=np.int64)
    out_y = np.zeros((len(qs), H, d_latent))
    out_lse = np.full((len(qs), H), -np.inf)
    scores_list, exact_list = [], []
    for i, t in enumerate(qs):
        b = int(q_seq[t])
        start = int(kv_start[b])
        n = visible_count(q_pos[t], kv_len[b])
        keys = k_idx[start:start + n]
        s64 = index_scores(q_idx[t], w[t], keys)
        exact_list.append(fp32_exact_bound(q_idx[t], w[t], keys))
        s32 = to_fp32(s64)
        if keep_scores:
            scores_list.append(s32)
        sel = select_topk(s32, topk)
        out_idx[i] = sel
        chosen = sel[sel >= 0]
        o, lse, _ = attend(q[t], kv[start + chosen], tau, d_latent)
        out_y[i] = output_gate(o, None if gate is None else gate[t])
        out_lse[i] = lse
    return {"scores": scores_list, "scores_exact": exact_list, "topk_idx": out_idx,
            "y": out_y, "lse": out_lse, "queries": np.array(qs, dtype=np.int64)}


def dense_causal_mla(q: np.ndarray, kv_seq: np.ndarray, q_pos: np.ndarray, tau: float,
                     d_latent: int):
    """Dense causal absorbed MLA of queries of one sequence, with no indexer.

    Builds the full [T, H, n] logit tensor, masks positions after each query
    (and beyond the cache) with -inf, and normalises over every remaining
    position. SGA with k >= n must reproduce this: before the sparse stage
    the model attends densely ([AK2-ART]; [AK2-TR] section 3.4).
    Returns (o [T, H, Dc], lse [T, H]).
    """
    n = kv_seq.shape[0]
    logits = tau * np.einsum("thd,sd->ths", q, kv_seq)
    pos = np.arange(n)
    mask = pos[None, :] > np.asarray(q_pos)[:, None]        # [T, n]
    logits = np.where(mask[:, None, :], -np.inf, logits)
    mx = logits.max(axis=2, keepdims=True)
    e = np.exp(logits - mx)
    z = e.sum(axis=2, keepdims=True)
    o = np.einsum("ths,sc->thc", e / z, kv_seq[:, :d_latent])
    return o, (mx + np.log(z))[..., 0]
