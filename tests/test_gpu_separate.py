"""Separate gate and up weight tensors (moe_fwd_sep / moe_bwd_sep) on the GPU.

The fixtures draw a fused [E,2I,H] tensor and split it into w_gate and w_up
[E,I,H] by the fused layout, so the oracle's fused definition is the
reference.  I = 200 makes the weight-gradient tiles (128 rows of 2I = 400)
straddle the boundary between the gate and the up tensor.  With the
concatenated fused layout the separate path does the same arithmetic in the
same order, so its results must be bit-identical to the fused path's.
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_histogram_amd as moe
from tests._gpu import assert_parity, device_inputs, host, oracle_fwd_bwd, small_inputs
from tests.test_gpu_parity import check_weight_grads, gate_up_halves, skewed_ids

pytestmark = pytest.mark.gpu


def split_weights(wgu, layout):
    """w_gate, w_up [E,I,H] of a fused [E,2I,H] device tensor in `layout`."""
    I = wgu.shape[1] // 2
    g, u = (wgu[:, 0::2], wgu[:, 1::2]) if layout == "interleaved" else (wgu[:, :I], wgu[:, I:])
    return g.contiguous(), u.contiguous()


@pytest.mark.parametrize("act,layout", [("swiglu", "concat"), ("clamped", "interleaved")])
@pytest.mark.parametrize("dtype,grad_dtype", [("bf16", "bf16"), ("bf16", "fp32"), ("fp32", "fp32")])
@pytest.mark.parametrize("save", [True, False])
def test_separate_weights_match_oracle(act, layout, dtype, grad_dtype, save):
    T, H, I, E, K = 300, 328, 200, 6, 3
    inp = small_inputs(T, H, I, E, K, dtype, act, layout, seed=13, ids=skewed_ids(T, K, E, 13))
    check_separate(inp, act, layout, dtype, grad_dtype, save)


@pytest.mark.parametrize("layout", ["concat", "interleaved"])
@pytest.mark.parametrize("grad_dtype", ["bf16", "fp32"])
def test_separate_weights_all_weight_gradient_kernels(layout, grad_dtype):
    """Experts of 0, 16, 240, 241, 300, 513 and 1601 slots: the resident,
    tiled and long-K weight gradients each write rows of the separate gate
    and up tensors (tiles straddling their boundary at I = 200)."""
    counts = [1601, 513, 300, 241, 240, 16, 0]
    E, K = len(counts), 1
    T, H, I = sum(counts), 264, 200
    rng = np.random.default_rng(41)
    ids = rng.permutation(np.repeat(np.arange(E), counts)).reshape(T, K).astype(np.int32)
    inp = small_inputs(T, H, I, E, K, "bf16", "swiglu", layout, seed=41, ids=ids)
    check_separate(inp, "swiglu", layout, "bf16", grad_dtype, True)


def check_separate(inp, act, layout, dtype, grad_dtype, save):
    E = inp.wl.E
    d = device_inputs(inp)
    wg, wu = split_weights(d["w_gate_up"], layout)
    kw = dict(act=act, limit=inp.wl.limit, alpha=inp.wl.alpha)
    out, saved, ws = moe.fwd_sep(d["hidden"], d["topk_ids"], d["topk_weights"], wg, wu, d["w_down"], save=save, **kw)
    dh, dw, dg, du, dd, ws2 = moe.bwd_sep(d["hidden"], d["topk_ids"], d["topk_weights"], wg, wu, d["w_down"],
                                          d["d_out"], saved=saved, grad_dtype=grad_dtype, **kw)
    torch.cuda.synchronize()
    assert moe.check_device_status(ws) == 0 and moe.check_device_status(ws2) == 0
    ref_out, (r_dx, r_dw, r_dgu, r_dd) = oracle_fwd_bwd(inp)
    bf = dtype == "bf16"
    assert_parity(host(out), ref_out, "out (separate weights)", kind="out")
    assert_parity(host(dh), r_dx, "d_hidden (separate weights)", kind="d_hidden")
    assert_parity(host(dw), r_dw, "d_topk_weights (separate weights)", kind="d_topk_weights")
    # gate / up gradients as one concatenated block per expert, checked per expert and half
    r_cat = np.stack([np.concatenate(gate_up_halves(r_dgu[e], layout), axis=0) for e in range(E)])
    got_cat = torch.cat([dg, du], dim=1)
    counts = np.bincount(inp.topk_ids.ravel(), minlength=E)
    check_weight_grads(got_cat, dd, r_cat, r_dd, counts, "concat", bf16_workload=bf)


def test_separate_weights_equal_the_fused_concatenated_path():
    T, H, I, E, K = 257, 264, 200, 5, 2
    inp = small_inputs(T, H, I, E, K, "bf16", "swiglu", "concat", seed=17)
    d = device_inputs(inp)
    wg, wu = split_weights(d["w_gate_up"], "concat")
    out1, s1, _ = moe.fwd(d["hidden"], d["topk_ids"], d["topk_weights"], d["w_gate_up"], d["w_down"], save=True)
    out2, s2, _ = moe.fwd_sep(d["hidden"], d["topk_ids"], d["topk_weights"], wg, wu, d["w_down"], save=True)
    r1 = moe.bwd(d["hidden"], d["topk_ids"], d["topk_weights"], d["w_gate_up"], d["w_down"], d["d_out"], saved=s1,
                 grad_dtype="bf16")
    r2 = moe.bwd_sep(d["hidden"], d["topk_ids"], d["topk_weights"], wg, wu, d["w_down"], d["d_out"], saved=s2,
                     grad_dtype="bf16")
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])
    assert torch.equal(r1[2][:, :I], r2[2]) and torch.equal(r1[2][:, I:], r2[3])
    assert torch.equal(r1[3], r2[4])


def test_separate_weights_no_tokens():
    H, I, E, K = 264, 136, 4, 2
    dev = "cuda"
    wg = torch.randn(E, I, H, device=dev).to(torch.bfloat16)
    wu = torch.randn(E, I, H, device=dev).to(torch.bfloat16)
    wd = torch.randn(E, H, I, device=dev).to(torch.bfloat16)
    hidden = torch.empty((0, H), dtype=torch.bfloat16, device=dev)
    ids = torch.empty((0, K), dtype=torch.int32, device=dev)
    w = torch.empty((0, K), dtype=torch.float32, device=dev)
    grads = (torch.empty((0, H), dtype=torch.bfloat16, device=dev), torch.empty((0, K), dtype=torch.float32, device=dev),
             torch.full((E, I, H), float("nan"), dtype=torch.bfloat16, device=dev),
             torch.full((E, I, H), float("nan"), dtype=torch.bfloat16, device=dev),
             torch.full((E, H, I), float("nan"), dtype=torch.bfloat16, device=dev))
    _, _, dg, du, dd, ws = moe.bwd_sep(hidden, ids, w, wg, wu, wd, hidden, grads=grads, grad_dtype="bf16")
    torch.cuda.synchronize()
    assert moe.check_device_status(ws) == 0
    assert bool((dg == 0).all()) and bool((du == 0).all()) and bool((dd == 0).all())
