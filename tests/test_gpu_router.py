"""GPU parity of the router (moe_router, moe_fwd_logits, moe_router_bwd)
with the fp64 oracle.

Ids, counts, offsets and the slot permutation are decided by comparisons of
the fp32 logits only and must be bit-exact.  The weights are an fp32 softmax
of the chosen logits: the difference l_k - l_0 is rounded once (relative
2^-24, times |l_k - l_0| <= 16 here, in the exponent), expf adds about an ulp,
the k-order sum and the division a few more, so each weight is checked to
4e-6 of its own value (about 30 fp32 ulp).  The router backward is fp32 with
one K-term dot per token: rel-Frobenius 1e-6 and max-abs 1e-5 of its largest
element.
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_histogram_amd as moe
import oracle
from mixture_experts_expert_histogram_amd import _lib
from synth import WORKLOADS, make_routing, router_logits
from tests._gpu import assert_parity, host, small_inputs

pytestmark = pytest.mark.gpu

W_REL = 4e-6


def logits_case(T, E, seed, kind="normal"):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if kind == "ties":          # many exactly equal logits
        lg = (np.round(lg * 2) / 2).astype(np.float32)
    elif kind == "neg_inf":     # masked experts (-inf logits); expert 0 never masked
        mask = rng.random((T, E)) < 0.3
        mask[:, 0] = False
        lg[mask] = -np.inf
    return lg


def check_router(lg, K):
    T, E = lg.shape
    ids, w, counts, offsets, ss, ip, ws = moe.router(torch.from_numpy(lg).cuda(), K)
    torch.cuda.synchronize()
    assert moe.check_device_status(ws) == 0
    r_ids, r_w = oracle.router(lg, K)
    np.testing.assert_array_equal(ids.cpu().numpy(), r_ids)
    wg = w.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(r_w)) and np.all(np.isfinite(wg))
    bad = np.abs(wg - r_w) > W_REL * r_w
    assert not bad.any(), f"{bad.sum()} weights off, worst {np.max(np.abs(wg - r_w) / np.maximum(r_w, 1e-300)):.2e}"
    c, o, s, i = oracle.route(r_ids, E)
    np.testing.assert_array_equal(counts.cpu().numpy(), c)
    np.testing.assert_array_equal(offsets.cpu().numpy(), o)
    np.testing.assert_array_equal(ss.cpu().numpy(), s)
    np.testing.assert_array_equal(ip.cpu().numpy(), i)
    return ids, w


@pytest.mark.parametrize("T,E,K", [(1, 1, 1), (5, 8, 8), (300, 128, 4), (4097, 256, 8), (1000, 1024, 64),
                                   (777, 60, 3), (2500, 128, 1), (4096, 128, 4)])
@pytest.mark.parametrize("kind", ["normal", "ties", "neg_inf"])
def test_router_matches_oracle(T, E, K, kind):
    check_router(logits_case(T, E, T + E + K, kind), K)


def test_router_no_tokens():
    ids, w, counts, offsets, ss, ip, ws = moe.router(torch.empty((0, 16), dtype=torch.float32, device="cuda"), 2)
    torch.cuda.synchronize()
    assert moe.check_device_status(ws) == 0
    assert ids.shape == (0, 2) and int(counts.abs().sum()) == 0 and int(offsets.abs().sum()) == 0


def test_router_nan_token_reports_bad_ids():
    lg = logits_case(10, 8, 3)
    lg[3, :] = np.nan
    ids, w, counts, offsets, ss, ip, ws = moe.router(torch.from_numpy(lg).cuda(), 2)
    torch.cuda.synchronize()
    assert moe.check_device_status(ws) == _lib.MOE_ERR_BAD_EXPERT_ID
    got = ids.cpu().numpy()
    assert np.all(got[3] == -1)
    keep = np.r_[0:3, 4:10]
    r_ids, _ = oracle.router(lg[keep], 2)
    np.testing.assert_array_equal(got[keep], r_ids)


@pytest.mark.parametrize("act,layout", [("swiglu", "concat"), ("clamped", "interleaved")])
def test_fwd_from_logits_equals_fwd_on_router_output(act, layout):
    T, H, I, E, K = 300, 256, 136, 16, 4
    inp = small_inputs(T, H, I, E, K, "bf16", act, layout, seed=9)
    lg = logits_case(T, E, 11)
    dev = "cuda"
    hidden = torch.from_numpy(inp.hidden).to(dev).to(torch.bfloat16)
    wgu = torch.from_numpy(inp.w_gate_up).to(dev).to(torch.bfloat16)
    wd = torch.from_numpy(inp.w_down).to(dev).to(torch.bfloat16)
    lgt = torch.from_numpy(lg).to(dev)
    kw = dict(act=act, layout=layout)
    out1, ids1, w1, _, ws1 = moe.fwd_logits(hidden, lgt, K, wgu, wd, **kw)
    ids2, w2, *_ = moe.router(lgt, K)
    out2, _, ws2 = moe.fwd(hidden, ids2, w2, wgu, wd, **kw)
    torch.cuda.synchronize()
    assert moe.check_device_status(ws1) == 0 and moe.check_device_status(ws2) == 0
    assert torch.equal(ids1, ids2) and torch.equal(w1, w2)
    assert torch.equal(out1, out2)
    r_ids, r_w = oracle.router(lg, K)
    ref = oracle.forward(inp.hidden, r_ids, r_w, oracle.expert_accessor(inp.w_gate_up, inp.w_down), E, act, layout)
    assert_parity(host(out1), ref, "out from logits", kind="out")


@pytest.mark.parametrize("T,E,K", [(500, 128, 4), (64, 1024, 64), (3, 8, 8)])
def test_router_bwd_matches_oracle(T, E, K):
    lg = logits_case(T, E, 21)
    ids, w = check_router(lg, K)
    g = np.random.default_rng(22).standard_normal((T, K)).astype(np.float32)
    d = moe.router_bwd(ids, w, torch.from_numpy(g).cuda(), E)
    torch.cuda.synchronize()
    ref = oracle.router_backward(ids.cpu().numpy(), w.cpu().numpy(), g, E)
    got = d.cpu().numpy().astype(np.float64)
    assert np.linalg.norm(got - ref) <= 1e-6 * np.linalg.norm(ref)
    assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))
    mask = np.zeros_like(ref, dtype=bool)
    np.put_along_axis(mask, ids.cpu().numpy().astype(np.int64), True, axis=1)
    assert np.all(got[~mask] == 0)


@pytest.mark.parametrize("name", ["gptoss", "large", "backward"])
def test_router_reproduces_the_workload_routing(name):
    """The synthetic workloads' ids and weights are the top-K and renormalised
    softmax of their N(0,1) router logits; the router on those logits gives
    the same ids and the same weights to fp32 rounding."""
    wl = WORKLOADS[name]
    ids_ref, w_ref = make_routing(wl, seed=0)
    ids, w, counts, *_ = moe.router(torch.from_numpy(router_logits(wl.T, wl.E, 0)).cuda(), wl.K)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(w.cpu().numpy(), w_ref, rtol=W_REL)
    np.testing.assert_array_equal(counts.cpu().numpy(), np.bincount(ids_ref.ravel(), minlength=wl.E))


def test_router_full_size_batch():
    """The Zipf batch size (32768 tokens) with the large shapes' 256 experts and
    top-8: every id, count and position bit-exact, every weight to W_REL, and
    the router backward's rows summing to zero."""
    T, E, K = 32768, 256, 8
    lg = logits_case(T, E, 33)
    ids, w = check_router(lg, K)
    g = torch.randn((T, K), device="cuda", generator=torch.Generator(device="cuda").manual_seed(3))
    d = moe.router_bwd(ids, w, g, E)
    torch.cuda.synchronize()
    rows = d.double().sum(dim=1).abs()
    scale = (w.double() * g.double()).abs().sum(dim=1) + 1e-30
    assert float((rows / scale).max()) < 1e-5
