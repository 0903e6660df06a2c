"""Pins for the oracle's indexer scores and top-k selection (CPU only).

Scores are pinned against an exact brute force in Python integers and
Fractions, and against closed forms; the selection against an independent
heap-based selection and the invariants any correct top-k must satisfy.
"""

import heapq
import random
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import sga


def _brute_scores(q, w, keys):
    """Python-integer / Fraction evaluation of sum_h w_h * max(0, q_h . k_s)."""
    out = []
    for ks in keys:
        tot = Fraction(0)
        for h in range(len(q)):
            d = sum(int(a) * int(b) for a, b in zip(q[h], ks))
            if d > 0:
                tot += Fraction(float(w[h])) * d
        out.append(tot)
    return out


@pytest.mark.parametrize("seed", range(6))
def test_scores_match_exact_brute_force(seed):
    rng = random.Random(seed)
    HI, DI, n = rng.randint(1, 4), rng.randint(1, 9), rng.randint(1, 40)
    q = np.array([[rng.randint(-8, 8) for _ in range(DI)] for _ in range(HI)], dtype=np.float64)
    keys = np.array([[rng.randint(-8, 8) for _ in range(DI)] for _ in range(n)], dtype=np.float64)
    w = np.array([rng.randint(-1024, 1024) / 256.0 for _ in range(HI)])
    got = sga.index_scores(q, w, keys)
    ref = _brute_scores(q, w, keys)
    assert [Fraction(float(x)) for x in got] == ref


def test_scores_closed_form_and_relu():
    # q_h = all ones; key s = c_s * ones  ->  d_h = DI * c_s for every head
    DI, HI = 5, 3
    c = np.array([-3.0, -1.0, 0.0, 2.0, 7.0])
    keys = c[:, None] * np.ones((1, DI))
    q = np.ones((HI, DI))
    w = np.array([0.5, 0.25, 1.0])
    got = sga.index_scores(q, w, keys)
    assert np.array_equal(got, np.maximum(DI * c, 0) * w.sum())
    # a head with a negative dot product contributes nothing (the ReLU), even with w < 0
    q2 = np.stack([np.ones(DI), -np.ones(DI)])
    w2 = np.array([1.0, -2.0])
    got2 = sga.index_scores(q2, w2, keys)
    assert np.array_equal(got2, np.where(c > 0, DI * c, 0.0) - 2.0 * np.where(c < 0, -DI * c, 0.0))


def test_negative_zero_score_is_positive_zero():
    # w < 0 times a zero ReLU output produces -0.0 in IEEE arithmetic
    q = np.array([[1.0, 0.0]])
    keys = np.array([[-1.0, 0.0], [0.0, 0.0]])
    got = sga.index_scores(q, np.array([-0.5]), keys)
    assert not np.any(np.signbit(got))
    assert not np.any(np.signbit(sga.to_fp32(np.array([-0.0]))))


def test_visible_count_includes_own_position_and_clips_to_cache():
    assert sga.visible_count(0, 10) == 1
    assert sga.visible_count(9, 10) == 10
    assert sga.visible_count(12, 10) == 10
    assert sga.visible_count(-1, 10) == 0
    assert sga.visible_count(5, 0) == 0


def test_fp32_exact_bound():
    q = np.full((64, 128), 8.0)
    keys = np.full((3, 128), 8.0)
    w_ok = np.full(64, 0.5)            # bound: 64 * 0.5 * 8192 * 2^1 = 2^19 * 2 <= 2^24
    assert sga.fp32_exact_bound(q, w_ok, keys)
    w_fine = np.full(64, 1.0 + 2.0 ** -20)  # 20 fractional bits -> bound fails
    assert not sga.fp32_exact_bound(q, w_fine, keys)
    assert not sga.fp32_exact_bound(q + 0.5, w_ok, keys)


def _heap_topk(scores, k):
    n = len(scores)
    if n <= k:
        return list(range(n)) + [-1] * (k - n)
    best = heapq.nsmallest(k, ((-float(s), i) for i, s in enumerate(scores)))
    return sorted(i for _, i in best)


@pytest.mark.parametrize("seed", range(20))
def test_topk_matches_heap_selection_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 300))
    k = int(rng.integers(1, 64))
    scores = rng.integers(-3, 4, n).astype(np.float32) * np.float32(0.25)
    got = sga.select_topk(scores, k)
    assert list(got) == _heap_topk(scores, k)


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(-4, 4), min_size=0, max_size=80), st.integers(1, 40))
def test_topk_invariants(vals, k):
    scores = np.array(vals, dtype=np.float32)
    n = len(vals)
    sel = sga.select_topk(scores, k)
    assert len(sel) == k
    chosen = [int(i) for i in sel if i >= 0]
    assert chosen == sorted(chosen) and len(set(chosen)) == len(chosen)
    assert len(chosen) == min(n, k)
    assert all(int(i) == -1 for i in sel[len(chosen):])
    rest = sorted(set(range(n)) - set(chosen))
    if chosen and rest:
        lo = min(scores[i] for i in chosen)
        assert all(scores[j] <= lo for j in rest)
        # at the threshold value every chosen position precedes every dropped one
        tie_sel = [i for i in chosen if scores[i] == lo]
        tie_rest = [j for j in rest if scores[j] == lo]
        if tie_rest:
            assert max(tie_sel) < min(tie_rest)


def test_topk_special_cases():
    assert list(sga.select_topk(np.zeros(10, np.float32), 4)) == [0, 1, 2, 3]
    assert list(sga.select_topk(np.arange(3, dtype=np.float32), 5)) == [0, 1, 2, -1, -1]
    s = np.array([1, 5, 2, 5, 0], np.float32)
    assert list(sga.select_topk(s, 1)) == [1]
    assert list(sga.select_topk(s, 2)) == [1, 3]
    assert list(sga.select_topk(np.zeros(0, np.float32), 3)) == [-1, -1, -1]
    # -0.0 and +0.0 are the same score: the lower position wins the tie
    s2 = np.array([0.0, -0.0, 0.0], np.float32)[[1, 0, 2]]
    assert list(sga.select_topk(s2, 1)) == [0]


def test_topk_nan_ranks_first_and_ties_by_position():
    # R15: every NaN (either sign, any payload) ranks above +inf; NaNs tie with
    # each other, so the lower position wins among them. Worked by hand.
    neg_nan = np.array([0xFFC00001], dtype=np.uint32).view(np.float32)[0]
    pos_nan = np.array([0x7FC00000], dtype=np.uint32).view(np.float32)[0]
    s = np.array([1.0, neg_nan, np.inf, 3.0, pos_nan, -np.inf, neg_nan], np.float32)
    assert list(sga.select_topk(s, 1)) == [1]
    assert list(sga.select_topk(s, 2)) == [1, 4]
    assert list(sga.select_topk(s, 3)) == [1, 4, 6]
    assert list(sga.select_topk(s, 4)) == [1, 2, 4, 6]
    assert list(sga.select_topk(s, 5)) == [1, 2, 3, 4, 6]
    assert list(sga.select_topk(s, 6)) == [0, 1, 2, 3, 4, 6]
