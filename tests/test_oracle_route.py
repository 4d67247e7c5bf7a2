"""Pins for the oracle's router step (top-k selection and softmax weights).

The oracle picks experts by repeated selection of the largest remaining
logit and computes weights from a double-precision softmax.  These tests
check it against independent formulations: brute force over ordered k-tuples,
numpy's lexsort, scipy's softmax, and closed forms (pplx blog, Introduction:
top-K experts of the router's probability distribution; "How GPUs Talk",
section 7: the router's score weights each expert's output).
"""
import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import workloads as W


def _brute_topk(row, k):
    """The ordered k-tuple of distinct experts whose key sequence
    (logit, -index) is lexicographically largest."""
    E = len(row)
    best, best_key = None, None
    for tup in itertools.permutations(range(E), k):
        key = tuple((float(row[e]), -e) for e in tup)
        if best_key is None or key > best_key:
            best, best_key = tup, key
    return list(best)


def _tiny_rows(rng, n, E):
    """Random rows with planted ties, signed zeros and repeated values."""
    rows = rng.standard_normal((n, E)).astype(np.float32)
    for i in range(n):
        kind = i % 5
        if kind == 1:      # coarse values -> many ties
            rows[i] = rng.integers(-2, 3, E).astype(np.float32)
        elif kind == 2:    # signed zeros mixed with ties
            rows[i] = rng.choice(np.array([0.0, -0.0, 1.0, -1.0], np.float32), E)
        elif kind == 3:    # all equal
            rows[i] = np.float32(0.37)
    return rows


@pytest.mark.parametrize("E,k", [(1, 1), (2, 1), (2, 2), (5, 3), (8, 2), (9, 4), (10, 3)])
def test_topk_matches_brute_force(E, k):
    rng = np.random.default_rng(100 + 10 * E + k)
    rows = _tiny_rows(rng, 40, E)
    idx, _ = oracle.route_topk(rows, k)
    for t in range(rows.shape[0]):
        assert list(idx[t]) == _brute_topk(rows[t], k), (t, rows[t])


def test_topk_tiny_workload_brute_force():
    w = W.WORKLOADS["tiny"]
    logits = W.make_logits(w).numpy()
    idx, _ = oracle.route_topk(logits, w.k)
    for t in range(w.T):
        assert list(idx[t]) == _brute_topk(logits[t], w.k)


@pytest.mark.parametrize("name", W.ORDER)
def test_topk_matches_lexsort(name):
    w = W.WORKLOADS[name]
    logits = W.make_logits(w).numpy()
    idx, _ = oracle.route_topk(logits, w.k)
    ex = np.broadcast_to(np.arange(w.E), logits.shape)
    order = np.lexsort((ex, -logits), axis=-1)[:, : w.k]
    np.testing.assert_array_equal(idx, order)


@pytest.mark.parametrize("name", W.ORDER)
def test_weights_match_scipy_softmax(name):
    w = W.WORKLOADS[name]
    logits = W.make_logits(w).numpy()
    idx, wt = oracle.route_topk(logits, w.k)
    p = softmax(logits.astype(np.float64), axis=-1)
    ref = np.take_along_axis(p, idx.astype(np.int64), axis=-1)
    # both are double computations rounded once: within one float ulp
    np.testing.assert_allclose(wt, ref, rtol=2.0 ** -23, atol=0)


def test_all_equal_row():
    for E, k in [(8, 2), (256, 8), (128, 8), (3, 3)]:
        row = np.full((2, E), -1.25, np.float32)
        idx, wt = oracle.route_topk(row, k)
        assert (idx == np.arange(k)).all()
        np.testing.assert_allclose(wt, 1.0 / E, rtol=2.0 ** -23)


def test_two_expert_logistic_closed_form():
    rng = np.random.default_rng(7)
    ab = rng.standard_normal((200, 2)).astype(np.float32) * 4
    idx, wt = oracle.route_topk(ab, 2)
    for t in range(200):
        a, b = float(ab[t, 0]), float(ab[t, 1])
        p0 = 1.0 / (1.0 + math.exp(b - a))
        want = {0: p0, 1: 1.0 - p0}
        for j in range(2):
            assert abs(wt[t, j] - want[idx[t, j]]) <= 2.0 ** -23 * want[idx[t, j]] + 2.0 ** -60


def test_single_expert_weight_is_one():
    logits = np.random.default_rng(3).standard_normal((50, 1)).astype(np.float32)
    idx, wt = oracle.route_topk(logits, 1)
    assert (idx == 0).all() and (wt == 1.0).all()


def test_full_k_weights_sum_to_one():
    rng = np.random.default_rng(11)
    for E in (4, 16, 64):
        logits = rng.standard_normal((30, E)).astype(np.float32) * 3
        idx, wt = oracle.route_topk(logits, E)
        # full selection is a sort
        np.testing.assert_array_equal(np.sort(idx, axis=1), np.broadcast_to(np.arange(E), idx.shape))
        s = wt.astype(np.float64).sum(axis=1)
        assert np.all(np.abs(s - 1.0) <= E * 2.0 ** -24)
        # weights follow the selection order
        assert np.all(np.diff(wt, axis=1) <= 0)


def test_shift_invariance():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((64, 32)).astype(np.float32)
    shifted = (logits.astype(np.float64) + 0.5).astype(np.float32)
    i0, w0 = oracle.route_topk(logits, 4)
    i1, w1 = oracle.route_topk(shifted, 4)
    # a shift can create or break float ties only through rounding of the shift
    same = (np.sort(np.unique(logits, axis=1), axis=1).shape == logits.shape)
    if same:
        np.testing.assert_array_equal(i0, i1)
        np.testing.assert_allclose(w0, w1, rtol=2.0 ** -18)


def test_rejects_bad_arguments():
    logits = np.zeros((4, 3), np.float32)
    with pytest.raises(ValueError):
        oracle.route_topk(logits, 4)
    with pytest.raises(ValueError):
        oracle.route_topk(logits, 0)


def test_zero_tokens():
    idx, wt = oracle.route_topk(np.zeros((0, 8), np.float32), 2)
    assert idx.shape == (0, 2) and wt.shape == (0, 2)
