"""Pins of the oracle's forward against things other than itself.

* dense brute force: every expert on every token, gated by a dense [T,E]
  matrix, in torch fp64 (torch.nn.functional.silu / linear);
* all experts sharing weights reduces to one dense FFN times the sum of the
  token's routing weights;
* E=1, K=1, w=1 reduces to a textbook two-layer gated FFN;
* linearity in the routing weights, token/expert permutation equivariance,
  duplicate ids, layout equivalence;
* special values of the gated activations.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synth import WORKLOADS, make_host_inputs
from tests._dense import dense_forward, ffn, t64


def rand_problem(rng, T=11, H=12, I=10, E=4, K=3, scale=1.0):
    X = rng.standard_normal((T, H)) * scale
    ids = rng.integers(0, E, size=(T, K))
    w = rng.random((T, K))
    Wgu = rng.standard_normal((E, 2 * I, H)) * 0.3
    Wd = rng.standard_normal((E, H, I)) * 0.3
    return X, ids, w, Wgu, Wd


def ofwd(X, ids, w, Wgu, Wd, act, layout):
    return oracle.forward(X, ids, w, oracle.expert_accessor(Wgu, Wd), Wgu.shape[0], act, layout)


ACTS = ["swiglu", "clamped"]
LAYOUTS = ["concat", "interleaved"]


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dense_brute_force(act, layout, seed):
    rng = np.random.default_rng(seed)
    X, ids, w, Wgu, Wd = rand_problem(rng, scale=3.0 if act == "clamped" else 1.0)
    ref = dense_forward(t64(X), ids, t64(w), t64(Wgu), t64(Wd), act, layout).numpy()
    np.testing.assert_allclose(ofwd(X, ids, w, Wgu, Wd, act, layout), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act", ACTS)
def test_shared_weights_is_dense_ffn(act):
    rng = np.random.default_rng(7)
    X, ids, w, Wgu, Wd = rand_problem(rng, E=5)
    Wgu[:] = Wgu[0]
    Wd[:] = Wd[0]
    dense = ffn(t64(X), t64(Wgu[0]), t64(Wd[0]), act, "concat").numpy()
    expect = dense * w.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(ofwd(X, ids, w, Wgu, Wd, act, "concat"), expect, rtol=1e-12, atol=1e-12)


def test_single_expert_is_textbook_swiglu_ffn():
    rng = np.random.default_rng(3)
    X, ids, w, Wgu, Wd = rand_problem(rng, E=1, K=1)
    ids[:] = 0
    w[:] = 1.0
    x = torch.tensor(X)
    gate = F.linear(x, torch.tensor(Wgu[0, :10]))
    up = F.linear(x, torch.tensor(Wgu[0, 10:]))
    ref = F.linear(F.silu(gate) * up, torch.tensor(Wd[0])).numpy()
    np.testing.assert_allclose(ofwd(X, ids, w, Wgu, Wd, "swiglu", "concat"), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act", ACTS)
def test_linear_in_routing_weights(act):
    rng = np.random.default_rng(11)
    X, ids, w, Wgu, Wd = rand_problem(rng)
    w2 = rng.random(w.shape)
    a, b = 0.7, -1.3
    lhs = ofwd(X, ids, a * w + b * w2, Wgu, Wd, act, "concat")
    rhs = a * ofwd(X, ids, w, Wgu, Wd, act, "concat") + b * ofwd(X, ids, w2, Wgu, Wd, act, "concat")
    np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-12)
    assert np.all(ofwd(X, ids, 0 * w, Wgu, Wd, act, "concat") == 0)


def test_token_and_expert_permutation():
    rng = np.random.default_rng(5)
    X, ids, w, Wgu, Wd = rand_problem(rng, T=13, E=5)
    base = ofwd(X, ids, w, Wgu, Wd, "clamped", "interleaved")
    pt = rng.permutation(13)
    np.testing.assert_allclose(ofwd(X[pt], ids[pt], w[pt], Wgu, Wd, "clamped", "interleaved"),
                               base[pt], rtol=1e-12, atol=1e-13)
    pe = rng.permutation(5)            # new id j holds old expert pe[j]
    new_of_old = np.argsort(pe)
    np.testing.assert_allclose(ofwd(X, new_of_old[ids], w, Wgu[pe], Wd[pe], "clamped", "interleaved"),
                               base, rtol=1e-12, atol=1e-13)


def test_duplicate_ids_add_their_weights():
    rng = np.random.default_rng(9)
    X, ids, w, Wgu, Wd = rand_problem(rng, K=2)
    ids[:, 1] = ids[:, 0]
    one = ofwd(X, ids[:, :1], w.sum(axis=1, keepdims=True), Wgu, Wd, "swiglu", "concat")
    np.testing.assert_allclose(ofwd(X, ids, w, Wgu, Wd, "swiglu", "concat"), one, rtol=1e-12, atol=1e-13)


def test_layouts_agree_after_row_permutation():
    rng = np.random.default_rng(4)
    X, ids, w, Wgu, Wd = rand_problem(rng)
    I = Wd.shape[2]
    inter = np.empty_like(Wgu)
    inter[:, 0::2] = Wgu[:, :I]
    inter[:, 1::2] = Wgu[:, I:]
    for act in ACTS:
        np.testing.assert_allclose(ofwd(X, ids, w, inter, Wd, act, "interleaved"),
                                   ofwd(X, ids, w, Wgu, Wd, act, "concat"), rtol=1e-12, atol=1e-13)


def test_glu_special_values():
    g = np.array([0.0, 0.0, 1e3, -1e3])
    u = np.array([5.0, -2.0, 2.0, 2.0])
    # silu(0) = 0; silu(g) -> g for large g, -> 0 for very negative g
    np.testing.assert_allclose(oracle.glu(g, u, "swiglu"), [0.0, 0.0, 2e3, 0.0], atol=1e-12)
    # sigmoid(1.702*g) = 3/4 exactly when 1.702*g = ln 3
    g0 = math.log(3.0) / 1.702
    for uu in [-3.0, 0.0, 2.5, 6.9]:
        assert oracle.glu(np.array([g0]), np.array([uu]), "clamped")[0] == pytest.approx((uu + 1) * g0 * 0.75, rel=1e-14)
    # up clamps at +-7 and carries the +1 offset: up = -1 gives zero output
    assert oracle.glu(np.array([g0]), np.array([10.0]), "clamped")[0] == pytest.approx(8 * g0 * 0.75, rel=1e-14)
    assert oracle.glu(np.array([g0]), np.array([-10.0]), "clamped")[0] == pytest.approx(-6 * g0 * 0.75, rel=1e-14)
    assert oracle.glu(np.array([2.0]), np.array([-1.0]), "clamped")[0] == 0.0
    # gate clamps above at 7 only: constant for g >= 7, saturating sigmoid
    hi = oracle.glu(np.array([7.0, 9.0, 100.0]), np.array([1.0, 1.0, 1.0]), "clamped")
    assert hi[0] == hi[1] == hi[2]
    assert 2 * 7 * (1 - 1e-5) < hi[0] < 2 * 7
    # no lower clamp on the gate: x*sigmoid(1.702x) -> 0 as x -> -inf
    assert abs(oracle.glu(np.array([-50.0]), np.array([1.0]), "clamped")[0]) < 1e-30
    # quick-GELU shape: x*sigmoid(1.702x) stays within 0.03 of exact GELU
    x = np.linspace(-6, 6, 101)
    qg = oracle.glu(x, np.zeros_like(x), "clamped")
    gelu = F.gelu(torch.tensor(x)).numpy()
    assert np.max(np.abs(qg - gelu)) < 0.03


def test_tiny_workload_runs_and_matches_dense():
    inp = make_host_inputs(WORKLOADS["tiny"], seed=0)
    wl = inp.wl
    out = oracle.forward(inp.hidden, inp.topk_ids, inp.topk_weights,
                         oracle.expert_accessor(inp.w_gate_up, inp.w_down), wl.E, wl.act, wl.layout)
    ref = dense_forward(t64(inp.hidden), inp.topk_ids, t64(inp.topk_weights),
                        t64(inp.w_gate_up), t64(inp.w_down), wl.act, wl.layout).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("act,layout", [("swiglu", "concat"), ("clamped", "interleaved")])
def test_slot_outputs_weight_into_the_forward_and_the_topk_weight_gradient(act, layout):
    """slot_outputs y[s] (unweighted expert output of slot s) ties out two
    ways: out[t] = sum_k w[t,k] y[t*K+k], and, since out is linear in the
    routing weights, dL/dw[t,k] = <dY[t], y[t*K+k]> from the backward."""
    rng = np.random.default_rng(41)
    X, ids, w, Wgu, Wd = rand_problem(rng)
    T, K = ids.shape
    E = Wgu.shape[0]
    ex = oracle.expert_accessor(Wgu, Wd)
    Y = oracle.slot_outputs(X, ids, ex, E, act, layout)
    out = oracle.forward(X, ids, w, ex, E, act, layout)
    np.testing.assert_allclose(out, np.einsum("tk,tkh->th", w, Y.reshape(T, K, -1)), rtol=1e-12, atol=1e-12)
    dY = rng.standard_normal(out.shape)
    _, dW, _, _ = oracle.backward(X, ids, w, dY, ex, E, act, layout)
    np.testing.assert_allclose(dW, np.einsum("th,tkh->tk", dY, Y.reshape(T, K, -1)), rtol=1e-12, atol=1e-12)
