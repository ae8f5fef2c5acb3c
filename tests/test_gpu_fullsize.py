"""Parity at the full workload sizes, in the launch configuration the
benchmark times (moe_fwd with saved Z, then moe_bwd; weight gradients
accumulated in fp32 and stored as bf16, the parameter dtype; fp32 storage is
checked on the gpt-oss workload too).

The fp64 oracle cannot evaluate a whole layer at these sizes in test time, so
it checks samples it can compute one by one:
  * out, d_hidden and d_topk_weights of sampled tokens (a token depends only
    on its own K slots);
  * all weight gradients of sampled experts (an expert's gradients depend
    only on its own slots);
and, for the hottest expert of the Zipf workload (tens of thousands of
tokens), the identity sum(Wd[e] * dWd[e]) = sum over its slots of
w_s * dTopkW_s, which holds at any size because the output is linear in the
down weights and in the routing weights.
Expert weights are drawn in device memory; the oracle reads the experts it
needs back from there.
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_histogram_amd as moe
import oracle
from synth import WORKLOADS, device_weights, make_dout, make_hidden, make_routing, to_device
from tests._gpu import assert_parity, assert_parity_slots, host, slot_factors

pytestmark = pytest.mark.gpu

_cache = {}
_weights = {}


def shape_weights(name):
    """Device expert weights of a workload's layer shape, kept while tests of
    that shape run (at several token counts)."""
    if name not in _weights:
        _weights.clear()
        _cache.clear()
        torch.cuda.empty_cache()
        _weights[name] = device_weights(WORKLOADS[name], "cuda", seed=0)
    return _weights[name]


def run_workload(name, grad_dtype="bf16", T=None):
    key = (name, grad_dtype, T)
    if key in _cache:
        return _cache[key]
    _cache.clear()
    torch.cuda.empty_cache()
    wl = WORKLOADS[name] if T is None else WORKLOADS[name].with_(T=T)
    dev = "cuda"
    ids, w = make_routing(wl, seed=0)
    X, dY = make_hidden(wl, 0), make_dout(wl, 0)
    d = dict(hidden=to_device(X, wl, dev), topk_ids=torch.from_numpy(ids).to(dev),
             topk_weights=torch.from_numpy(w).to(dev), d_out=to_device(dY, wl, dev))
    Wgu, Wd = shape_weights(name)
    kw = dict(act=wl.act, layout=wl.layout, limit=wl.limit, alpha=wl.alpha)
    out, saved, ws = moe.fwd(d["hidden"], d["topk_ids"], d["topk_weights"], Wgu, Wd, save=True, **kw)
    dh, dw, dgu, dd, ws2 = moe.bwd(d["hidden"], d["topk_ids"], d["topk_weights"], Wgu, Wd, d["d_out"],
                                   saved=saved, grad_dtype=grad_dtype, **kw)
    torch.cuda.synchronize()
    assert moe.check_device_status(ws) == 0 and moe.check_device_status(ws2) == 0
    del saved, ws, ws2
    res = dict(wl=wl, ids=ids, w=w, X=X, dY=dY, Wgu=Wgu, Wd=Wd, out=out, dh=dh, dw=dw, dgu=dgu, dd=dd)
    _cache[key] = res
    return res


def expert_fetch(r):
    def fetch(e):
        return r["Wgu"][e].float().cpu().numpy(), r["Wd"][e].float().cpu().numpy()
    return fetch


def sample_tokens(r, n, seed=1):
    return np.sort(np.random.default_rng(seed).choice(r["wl"].T, size=n, replace=False))


@pytest.mark.parametrize("name,ntok", [("gptoss", 8), ("large", 8), ("zipf", 8)])
def test_forward_sampled_tokens(name, ntok):
    r = run_workload(name)
    wl = r["wl"]
    toks = sample_tokens(r, ntok)
    ex = oracle.expert_accessor(expert_fetch(r))
    ref = oracle.forward(r["X"][toks], r["ids"][toks], r["w"][toks], ex, wl.E, wl.act, wl.layout, wl.limit, wl.alpha)
    assert_parity(host(r["out"][toks]), ref, f"{name} out[{list(toks)}]", kind="out")


@pytest.mark.parametrize("name,ntok", [("gptoss", 8), ("backward", 8), ("zipf", 8)])
def test_backward_sampled_tokens(name, ntok):
    r = run_workload(name)
    wl = r["wl"]
    toks = sample_tokens(r, ntok, seed=2)
    ex = oracle.expert_accessor(expert_fetch(r))
    dX, dW, _, _ = oracle.backward(r["X"][toks], r["ids"][toks], r["w"][toks], r["dY"][toks], ex, wl.E, wl.act,
                                   wl.layout, wl.limit, wl.alpha, dw_sink=lambda *a: None)
    assert_parity(host(r["dh"][toks]), dX, f"{name} d_hidden sample", kind="d_hidden")
    assert_parity(host(r["dw"][toks]), dW, f"{name} d_topk_weights sample", kind="d_topk_weights")


def expert_subproblem(r, e):
    """The slots routed to expert e as a one-expert, one-slot-per-token problem."""
    wl = r["wl"]
    flat = r["ids"].ravel()
    slots = np.nonzero(flat == e)[0]
    tok = slots // wl.K
    return slots, r["X"][tok], np.zeros((len(slots), 1), np.int32), r["w"].ravel()[slots].reshape(-1, 1), r["dY"][tok]


def halves(x, layout):
    I = x.shape[0] // 2
    return (x[0::2], x[1::2]) if layout == "interleaved" else (x[:I], x[I:])


@pytest.mark.parametrize("name,which", [("gptoss", "coldest"), ("gptoss", "median"), ("backward", "coldest"),
                                        ("backward", "median"), ("backward", "resident_max"),
                                        ("backward", "tiled_min"), ("zipf", "coldest"), ("zipf", "median"),
                                        ("zipf", "long_min")])
def test_backward_sampled_experts(name, which):
    check_sampled_expert(run_workload(name), which)


@pytest.mark.parametrize("which", ["coldest", "median"])
def test_fp32_weight_grads_sampled_experts(which):
    check_sampled_expert(run_workload("gptoss", "fp32"), which)


def check_sampled_expert(r, which):
    name = r["wl"].name
    wl = r["wl"]
    counts = np.bincount(r["ids"].ravel(), minlength=wl.E)
    nonempty = [e for e in np.argsort(counts, kind="stable") if counts[e] > 0]
    # resident_max / tiled_min: the experts on either side of the resident
    # weight-gradient kernel's limit of 240 positions; long_min: the smallest
    # expert above the long-K kernel's threshold of 512 positions
    below = [x for x in nonempty if counts[x] <= 240]
    above = [x for x in nonempty if counts[x] > 240]
    long_ = [x for x in nonempty if counts[x] > 512]
    pick = {"coldest": lambda: nonempty[0], "median": lambda: nonempty[len(nonempty) // 2],
            "hottest": lambda: nonempty[-1], "resident_max": lambda: below[-1], "tiled_min": lambda: above[0],
            "long_min": lambda: long_[0]}
    e = pick[which]()
    slots, Xe, ids1, w1, dYe = expert_subproblem(r, e)
    gu, dn = expert_fetch(r)(e)
    got = {}
    dX, dW, _, _ = oracle.backward(Xe, ids1, w1, dYe, oracle.expert_accessor(lambda _e: (gu, dn)), 1, wl.act,
                                   wl.layout, wl.limit, wl.alpha, dw_sink=lambda i, a, b: got.__setitem__(i, (a, b)))
    ref_gu, ref_dn = got[0]
    g_gu, g_dn = host(r["dgu"][e]), host(r["dd"][e])
    dz, xs, dys, wa = slot_factors(Xe, w1, dYe, gu, dn, wl.act, wl.layout, wl.limit, wl.alpha)
    for half, g, ref, P in zip(["gate", "up"], halves(g_gu, wl.layout), halves(ref_gu, wl.layout),
                               oracle.split_gate_up(dz, wl.layout)):
        assert_parity_slots(g, ref, P, xs, f"{name} dW_{half}[{e}] ({counts[e]} slots)")
    assert_parity_slots(g_dn, ref_dn, dys, wa, f"{name} dW_down[{e}] ({counts[e]} slots)")
    assert_parity(host(r["dw"]).ravel()[slots], dW.ravel(), f"{name} d_topk_weights of expert {e}",
                  kind="d_topk_weights")


@pytest.mark.parametrize("which", ["hottest", "second"])
def test_zipf_hot_expert_sampled_columns(which):
    """Element-wise weight gradients of the Zipf workload's hottest experts
    (tens of thousands of slots, the long-K weight gradient at its longest
    K) on 64 sampled intermediate columns j.  The activation acts column by
    column, so the oracle run on the expert restricted to those columns (gate
    and up rows j of w_gate_up, columns j of w_down) gives exactly rows j of
    dW_gate and dW_up and columns j of dW_down."""
    r = run_workload("zipf")
    wl = r["wl"]
    counts = np.bincount(r["ids"].ravel(), minlength=wl.E)
    order = np.argsort(-counts, kind="stable")
    e = int(order[0] if which == "hottest" else order[1])
    assert counts[e] > 10000
    cols = np.sort(np.random.default_rng(7).choice(wl.I, size=64, replace=False))
    slots, Xe, ids1, w1, dYe = expert_subproblem(r, e)
    gu, dn = expert_fetch(r)(e)
    g_rows, u_rows = halves(gu, wl.layout)
    sub_g, sub_u = g_rows[cols], u_rows[cols]
    if wl.layout == "interleaved":
        gu_sub = np.empty((2 * len(cols), wl.H), dtype=gu.dtype)
        gu_sub[0::2], gu_sub[1::2] = sub_g, sub_u
    else:
        gu_sub = np.concatenate([sub_g, sub_u], axis=0)
    dn_sub = np.ascontiguousarray(dn[:, cols])
    got = {}
    oracle.backward(Xe, ids1, w1, dYe, oracle.expert_accessor(lambda _e: (gu_sub, dn_sub)), 1, wl.act, wl.layout,
                    wl.limit, wl.alpha, dw_sink=lambda i, a, b: got.__setitem__(i, (a, b)))
    ref_gu, ref_dn = got[0]
    g_gu, g_dn = host(r["dgu"][e]), host(r["dd"][e])
    gpu_g, gpu_u = halves(g_gu, wl.layout)
    dz, xs, dys, wa = slot_factors(Xe, w1, dYe, gu_sub, dn_sub, wl.act, wl.layout, wl.limit, wl.alpha)
    for half, g, ref, P in zip(["gate", "up"], [gpu_g[cols], gpu_u[cols]], halves(ref_gu, wl.layout),
                               oracle.split_gate_up(dz, wl.layout)):
        assert_parity_slots(g, ref, P, xs, f"zipf dW_{half}[{e}] rows of 64 columns ({counts[e]} slots)")
    assert_parity_slots(g_dn[:, cols], ref_dn, dys, wa, f"zipf dW_down[{e}] 64 columns ({counts[e]} slots)")


def test_zipf_hot_expert_identity():
    r = run_workload("zipf")
    wl = r["wl"]
    counts = np.bincount(r["ids"].ravel(), minlength=wl.E)
    e = int(np.argmax(counts))
    assert counts[e] > 10000
    lhs = float(torch.sum(r["Wd"][e].double() * r["dd"][e].double()))
    slots = np.nonzero(r["ids"].ravel() == e)[0]
    rhs = float(np.sum(r["w"].ravel()[slots].astype(np.float64) * host(r["dw"]).ravel()[slots]))
    assert abs(lhs - rhs) <= 1e-2 * max(abs(lhs), abs(rhs)), (lhs, rhs)


def test_zipf_empty_or_cold_experts_and_shapes():
    r = run_workload("zipf")
    wl = r["wl"]
    counts = np.bincount(r["ids"].ravel(), minlength=wl.E)
    assert counts.max() > 20 * np.median(counts)
    for e in np.nonzero(counts == 0)[0]:
        assert torch.count_nonzero(r["dgu"][e]) == 0 and torch.count_nonzero(r["dd"][e]) == 0
    assert torch.isfinite(r["out"]).all() and torch.isfinite(r["dh"]).all()


@pytest.mark.parametrize("name,T", [("gptoss", 1), ("gptoss", 37), ("large", 1), ("large", 16), ("large", 2048),
                                    ("backward", 5), ("backward", 300)])
def test_small_token_counts_at_full_shapes(name, T):
    """The layer shapes at token counts from 1 up: most experts empty, a few
    with one or two slots, every M-tile a ragged tail."""
    r = run_workload(name, T=T)
    wl = r["wl"]
    toks = np.arange(T) if T <= 4 else sample_tokens(r, 4, seed=3)
    ex = oracle.expert_accessor(expert_fetch(r))
    ref = oracle.forward(r["X"][toks], r["ids"][toks], r["w"][toks], ex, wl.E, wl.act, wl.layout, wl.limit, wl.alpha)
    assert_parity(host(r["out"][toks]), ref, f"{name} T={T} out", kind="out")
    dX, dW, _, _ = oracle.backward(r["X"][toks], r["ids"][toks], r["w"][toks], r["dY"][toks], ex, wl.E, wl.act,
                                   wl.layout, wl.limit, wl.alpha, dw_sink=lambda *a: None)
    assert_parity(host(r["dh"][toks]), dX, f"{name} T={T} d_hidden", kind="d_hidden")
    assert_parity(host(r["dw"][toks]), dW, f"{name} T={T} d_topk_weights", kind="d_topk_weights")
    for which in ("coldest", "median", "hottest"):
        check_sampled_expert(r, which)
    counts = np.bincount(r["ids"].ravel(), minlength=wl.E)
    empty = torch.from_numpy(np.nonzero(counts == 0)[0]).cuda()
    assert int(torch.count_nonzero(r["dgu"].index_select(0, empty))) == 0
    assert int(torch.count_nonzero(r["dd"].index_select(0, empty))) == 0
