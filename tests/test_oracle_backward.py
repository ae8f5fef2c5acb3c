"""Pins of the oracle's backward ("MoE expert parallel execution backward").

* central finite differences of L = <dY, forward(...)> along random
  directions in every input (hidden, routing weights, gate_up, down);
* torch fp64 autograd of the dense formulation (a third implementation);
* Euler identities: the output is linear in the routing weights and in the
  down weights, so sum(w * dTopkW) = sum(Wd * dWd) = <dY, out>;
* dTopkW[s] = <dY_t, y_s> with y from the dense formulation;
* experts with no slots get exactly zero weight gradients;
* the clamped GLU in its clamped regions (inputs scaled up) has the
  derivative of the clamp.
"""
import numpy as np
import pytest
import torch

import oracle
from tests._dense import dense_forward, ffn, t64


def problem(seed, T=9, H=10, I=8, E=4, K=2, xscale=1.0, wscale=0.3):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, H)) * xscale
    ids = rng.integers(0, E, size=(T, K))
    w = rng.random((T, K))
    Wgu = rng.standard_normal((E, 2 * I, H)) * wscale
    Wd = rng.standard_normal((E, H, I)) * wscale
    dY = rng.standard_normal((T, H))
    return rng, X, ids, w, Wgu, Wd, dY


def run_fwd(X, ids, w, Wgu, Wd, act, layout):
    return oracle.forward(X, ids, w, oracle.expert_accessor(Wgu, Wd), Wgu.shape[0], act, layout)


def run_bwd(X, ids, w, Wgu, Wd, dY, act, layout):
    return oracle.backward(X, ids, w, dY, oracle.expert_accessor(Wgu, Wd), Wgu.shape[0], act, layout)


def pre_activations(X, ids, Wgu):
    """gate_up outputs of every slot (to keep FD points away from the clamp kinks)."""
    T, K = ids.shape
    return np.stack([X[s // K] @ Wgu[ids.reshape(-1)[s]].T for s in range(T * K)])


CASES = [("swiglu", "concat", 1.0), ("swiglu", "interleaved", 1.0),
         ("clamped", "interleaved", 1.0), ("clamped", "concat", 6.0), ("clamped", "interleaved", 6.0)]


@pytest.mark.parametrize("act,layout,xscale", CASES)
def test_finite_differences(act, layout, xscale):
    for seed in range(20):
        rng, X, ids, w, Wgu, Wd, dY = problem(seed, xscale=xscale)
        Z = pre_activations(X, ids, Wgu)
        if np.min(np.abs(np.abs(Z) - 7.0)) > 0.05:
            break
    if act == "clamped" and xscale > 1:
        assert np.mean(np.abs(Z) > 7.0) > 0.1      # the clamps are really exercised
    dX, dW, dWgu, dWd = run_bwd(X, ids, w, Wgu, Wd, dY, act, layout)

    def L(X_, w_, Wgu_, Wd_):
        return float(np.sum(dY * run_fwd(X_, ids, w_, Wgu_, Wd_, act, layout)))

    h = 1e-6
    for trial in range(3):
        vX, vw = rng.standard_normal(X.shape), rng.standard_normal(w.shape)
        vgu, vd = rng.standard_normal(Wgu.shape), rng.standard_normal(Wd.shape)
        fd = (L(X + h * vX, w + h * vw, Wgu + h * vgu, Wd + h * vd)
              - L(X - h * vX, w - h * vw, Wgu - h * vgu, Wd - h * vd)) / (2 * h)
        an = np.sum(dX * vX) + np.sum(dW * vw) + np.sum(dWgu * vgu) + np.sum(dWd * vd)
        assert an == pytest.approx(fd, rel=1e-6, abs=1e-7 * max(1.0, abs(fd)))
        # each input separately, so that a wrong grad cannot hide behind another
        for part in range(4):
            v = [vX * (part == 0), vw * (part == 1), vgu * (part == 2), vd * (part == 3)]
            fd = (L(X + h * v[0], w + h * v[1], Wgu + h * v[2], Wd + h * v[3])
                  - L(X - h * v[0], w - h * v[1], Wgu - h * v[2], Wd - h * v[3])) / (2 * h)
            an = [np.sum(dX * v[0]), np.sum(dW * v[1]), np.sum(dWgu * v[2]), np.sum(dWd * v[3])][part]
            assert an == pytest.approx(fd, rel=1e-6, abs=1e-7 * max(1.0, abs(fd)))


@pytest.mark.parametrize("act,layout,xscale", CASES)
def test_matches_dense_autograd(act, layout, xscale):
    rng, X, ids, w, Wgu, Wd, dY = problem(3, T=12, E=5, K=3, xscale=xscale)
    tX, tw, tgu, td = t64(X, True), t64(w, True), t64(Wgu, True), t64(Wd, True)
    out = dense_forward(tX, ids, tw, tgu, td, act, layout)
    (out * t64(dY)).sum().backward()
    dX, dW, dWgu, dWd = run_bwd(X, ids, w, Wgu, Wd, dY, act, layout)
    for mine, ref in [(dX, tX.grad), (dW, tw.grad), (dWgu, tgu.grad), (dWd, td.grad)]:
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("act", ["swiglu", "clamped"])
def test_euler_identities(act):
    _, X, ids, w, Wgu, Wd, dY = problem(8, T=15, E=6, K=3)
    out = run_fwd(X, ids, w, Wgu, Wd, act, "concat")
    dX, dW, dWgu, dWd = run_bwd(X, ids, w, Wgu, Wd, dY, act, "concat")
    ip = np.sum(dY * out)
    assert np.sum(w * dW) == pytest.approx(ip, rel=1e-12)
    assert np.sum(Wd * dWd) == pytest.approx(ip, rel=1e-12)


def test_dtopkw_closed_form():
    _, X, ids, w, Wgu, Wd, dY = problem(12, T=10, E=3, K=3)
    _, dW, _, _ = run_bwd(X, ids, w, Wgu, Wd, dY, "swiglu", "interleaved")
    for t in range(10):
        for k in range(3):
            e = ids[t, k]
            y = ffn(t64(X[t:t + 1]), t64(Wgu[e]), t64(Wd[e]), "swiglu", "interleaved").numpy()[0]
            assert dW[t, k] == pytest.approx(float(dY[t] @ y), rel=1e-12, abs=1e-14)


def test_zero_weight_slot_still_gets_dtopkw():
    _, X, ids, w, Wgu, Wd, dY = problem(13)
    w[0, 0] = 0.0
    dX, dW, dWgu, dWd = run_bwd(X, ids, w, Wgu, Wd, dY, "swiglu", "concat")
    e = ids[0, 0]
    y = ffn(t64(X[:1]), t64(Wgu[e]), t64(Wd[e]), "swiglu", "concat").numpy()[0]
    assert dW[0, 0] == pytest.approx(float(dY[0] @ y), rel=1e-12)


def test_empty_experts_have_zero_weight_grads():
    _, X, ids, w, Wgu, Wd, dY = problem(14, E=6)
    ids[ids >= 3] = 0                   # experts 3, 4, 5 receive nothing
    dX, dW, dWgu, dWd = run_bwd(X, ids, w, Wgu, Wd, dY, "clamped", "interleaved")
    assert np.all(dWgu[3:] == 0) and np.all(dWd[3:] == 0)
    assert np.any(dWgu[:3] != 0) and np.any(dWd[:3] != 0)


def test_streamed_weight_grads_equal_stacked():
    _, X, ids, w, Wgu, Wd, dY = problem(15, E=5)
    ids[ids == 2] = 1                   # one empty expert
    full = run_bwd(X, ids, w, Wgu, Wd, dY, "swiglu", "concat")
    got = {}
    dX, dW, none1, none2 = oracle.backward(X, ids, w, dY, oracle.expert_accessor(Wgu, Wd), 5, "swiglu",
                                           "concat", dw_sink=lambda e, a, b: got.__setitem__(e, (a, b)))
    assert none1 is None and none2 is None and sorted(got) == list(range(5))
    np.testing.assert_array_equal(dX, full[0])
    assert got[2] == (None, None) and np.all(full[2][2] == 0) and np.all(full[3][2] == 0)
    for e in [0, 1, 3, 4]:
        np.testing.assert_array_equal(got[e][0], full[2][e])
        np.testing.assert_array_equal(got[e][1], full[3][e])


def test_clamp_region_derivatives():
    g = np.array([8.0, 6.0, -9.0, 3.0, 3.0, 3.0])
    u = np.array([1.0, 1.0, 1.0, 8.0, -8.0, 6.5])
    dg, du = oracle.glu_backward(g, u, np.ones(6), "clamped")
    assert dg[0] == 0.0                 # gate above the limit: flat
    assert dg[2] != 0.0                 # no lower clamp on the gate
    assert du[3] == 0.0 and du[4] == 0.0   # up outside [-7, 7]: flat
    assert du[5] != 0.0 and dg[1] != 0.0
