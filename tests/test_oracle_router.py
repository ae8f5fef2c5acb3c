"""Pins of the oracle's router (top-K of the logits, renormalised softmax) and
of its backward, against an independent top-K, closed forms and finite
differences."""
import numpy as np
import pytest

import oracle


def brute_topk(row, K):
    """K rounds of 'largest remaining logit, lowest id on ties'."""
    left = list(range(len(row)))
    out = []
    for _ in range(K):
        best = left[0]
        for e in left[1:]:
            if row[e] > row[best]:
                best = e
        out.append(best)
        left.remove(best)
    return out


@pytest.mark.parametrize("T,E,K,seed,quant", [(20, 8, 2, 0, 0), (15, 64, 8, 1, 0), (10, 130, 5, 2, 0.5),
                                             (12, 16, 16, 3, 0), (30, 7, 3, 4, 1.0)])
def test_ids_match_repeated_argmax(T, E, K, seed, quant):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if quant:   # many exact ties
        lg = (np.round(lg / quant) * quant).astype(np.float32)
    ids, w = oracle.router(lg, K)
    for t in range(T):
        assert list(ids[t]) == brute_topk(lg[t].astype(np.float64), K)


def test_ties_go_to_the_lower_id():
    lg = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]], dtype=np.float32)
    ids, w = oracle.router(lg, 4)
    assert list(ids[0]) == [1, 2, 4, 3]
    np.testing.assert_allclose(w[0, :3], w[0, 0])


def test_weights_are_the_softmax_of_the_chosen_logits():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((40, 32)) * 3
    ids, w = oracle.router(lg, 6)
    sel = np.take_along_axis(lg, ids, axis=1)
    ref = np.exp(sel) / np.exp(sel).sum(axis=1, keepdims=True)
    np.testing.assert_allclose(w, ref, rtol=1e-13)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_all_experts_chosen_gives_the_full_softmax():
    lg = np.array([[0.5, -1.0, 2.0, 0.0]])
    ids, w = oracle.router(lg, 4)
    p = np.exp(lg[0]) / np.exp(lg[0]).sum()
    assert list(ids[0]) == [2, 0, 3, 1]
    np.testing.assert_allclose(w[0], p[[2, 0, 3, 1]], rtol=1e-14)


def test_large_logit_range_keeps_the_logit_order():
    """Softmax probabilities underflow to 0 far below the max; the choice still
    follows the logits."""
    lg = np.array([[0.0, -2000.0, -1000.0, 5.0]])
    ids, w = oracle.router(lg, 3)
    assert list(ids[0]) == [3, 0, 2]
    assert w[0, 2] == 0.0 and abs(w[0, 0] + w[0, 1] - 1) < 1e-15


def test_backward_matches_finite_differences():
    rng = np.random.default_rng(7)
    T, E, K = 6, 12, 4
    lg = rng.standard_normal((T, E))
    g = rng.standard_normal((T, K))
    ids, w = oracle.router(lg, K)
    d = oracle.router_backward(ids, w, g, E)
    h = 1e-6
    fd = np.zeros_like(lg)
    for t in range(T):
        for e in range(E):
            lp, lm = lg.copy(), lg.copy()
            lp[t, e] += h
            lm[t, e] -= h
            ip, wp = oracle.router(lp, K)
            im, wm = oracle.router(lm, K)
            assert np.array_equal(ip, ids) and np.array_equal(im, ids)   # no choice flips at this step
            fd[t, e] = (np.sum(g * wp) - np.sum(g * wm)) / (2 * h)
    np.testing.assert_allclose(d, fd, atol=1e-8)


def test_backward_rows_sum_to_zero_and_unchosen_are_zero():
    rng = np.random.default_rng(8)
    lg = rng.standard_normal((9, 20))
    ids, w = oracle.router(lg, 5)
    d = oracle.router_backward(ids, w, rng.standard_normal((9, 5)), 20)
    np.testing.assert_allclose(d.sum(axis=1), 0, atol=1e-14)
    mask = np.zeros_like(d, dtype=bool)
    np.put_along_axis(mask, ids, True, axis=1)
    assert np.all(d[~mask] == 0)
