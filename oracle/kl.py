"""Indexer KL loss restricted to the sparse selection, and its gradients (oracle side).

Test infrastructure only: see the package docstring.

Sources: "A.X K2 Technical Report", section 3.4 (Stage 3C: the indexer
learns from a KL objective that pulls its scores toward the attention
weights, evaluated only on the sparse selection right from the beginning of
that stage); "A.X-K2: a sparse-attention upgrade that
costs nothing, trained natively in FP8", section "Sparse Gated Attention"
(the indexer learns to follow where the gated attention puts its weight). The pages
give no formula. Readings, following the published form of the indexer
design the report contrasts itself with:
  * for query t with selected set S_t, the target is the attention
    distribution over S_t summed over the heads and normalised to sum 1;
  * the indexer's distribution is the softmax of its scores over S_t;
  * the loss is KL(target || indexer) = sum_s target_s (log target_s -
    log softmax(I)_s), a term with target_s = 0 counting 0;
  * the target is a constant for this loss (only the indexer learns from it),
    so dL/dI_s = softmax(I)_s - target_s on S_t and 0 elsewhere;
  * through I_s = sum_h w_h ReLU(qI_h . kI_s) the gradients reach w, qI and
    kI, with ReLU'(0) taken as 0.
"""

from __future__ import annotations

import numpy as np


def attention_target(p_heads: np.ndarray) -> np.ndarray:
    """[H, m] per-head attention probabilities over S_t -> [m] target (sums to 1)."""
    t = p_heads.sum(axis=0)
    s = t.sum()
    return t / s if s > 0 else t


def indexer_kl(scores_sel: np.ndarray, target: np.ndarray):
    """KL(target || softmax(scores_sel)) and its gradient with respect to scores_sel."""
    if scores_sel.size == 0:
        return 0.0, np.zeros(0)
    mx = scores_sel.max()
    log_q = scores_sel - (mx + np.log(np.exp(scores_sel - mx).sum()))
    pos = target > 0
    loss = float(np.sum(target[pos] * (np.log(target[pos]) - log_q[pos])))
    return loss, np.exp(log_q) - target


def indexer_backward(q_idx_t: np.ndarray, w_t: np.ndarray, k_rows: np.ndarray, g: np.ndarray):
    """Gradients of sum_s g_s I_s with I_s = sum_h w_h ReLU(qI_h . kI_s).

    q_idx_t [HI, DI], w_t [HI], k_rows [m, DI], g [m] -> (dw [HI], dq_idx [HI, DI], dk_rows [m, DI]).
    """
    z = q_idx_t @ k_rows.T                       # [HI, m]
    dw = np.maximum(z, 0.0) @ g                  # [HI]
    gz = (z > 0) * w_t[:, None] * g[None, :]     # dL/dz [HI, m]
    return dw, gz @ k_rows, gz.T @ q_idx_t
