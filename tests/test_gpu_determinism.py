"""Run-to-run bitwise reproducibility of the forward + backward.

The pages accumulate the expert outputs with index_add_ ("Sparse expert
dispatch and combine", description), whose floating-point result depends on
the order of the adds.  Here every output element has one writer and every
sum runs in a fixed order (per-token combine in k order, routing-weight
partials in tile order, weight gradients over an expert's positions in
position order), so two runs on the same inputs must agree bit for bit.
Each run starts from workspaces, saved buffer and outputs filled with 0xFF
bytes (NaN), so a result that leaned on stale memory would differ.
"""
import pytest
import torch

import mixture_experts_expert_histogram_amd as moe
from synth import WORKLOADS, device_weights, make_dout, make_hidden, make_routing, to_device
from tests.test_gpu_parity import poisoned_buffers

pytestmark = pytest.mark.gpu


def one_run(wl, X, ids, w, Wgu, Wd, dY):
    kw = dict(act=wl.act, layout=wl.layout, limit=wl.limit, alpha=wl.alpha)
    b = poisoned_buffers(wl, "bf16")
    out, saved, ws = moe.fwd(X, ids, w, Wgu, Wd, save=True, ws=b["ws_f"], out=b["out"], saved=b["saved"], **kw)
    dh, dw, dgu, dd, ws2 = moe.bwd(X, ids, w, Wgu, Wd, dY, saved=saved, ws=b["ws_b"], grads=b["grads"],
                                   grad_dtype="bf16", **kw)
    torch.cuda.synchronize()
    assert moe.check_device_status(ws) == 0 and moe.check_device_status(ws2) == 0
    del b, saved, ws, ws2
    return out, dh, dw, dgu, dd


@pytest.mark.parametrize("name", ["gptoss", "zipf"])
def test_fwd_bwd_bitwise_reproducible(name):
    wl = WORKLOADS[name]
    torch.cuda.empty_cache()
    ids_np, w_np = make_routing(wl, seed=0)
    X, dY = to_device(make_hidden(wl, 0), wl, "cuda"), to_device(make_dout(wl, 0), wl, "cuda")
    ids, w = torch.from_numpy(ids_np).cuda(), torch.from_numpy(w_np).cuda()
    Wgu, Wd = device_weights(wl, "cuda", seed=0)
    first = one_run(wl, X, ids, w, Wgu, Wd, dY)
    second = one_run(wl, X, ids, w, Wgu, Wd, dY)
    for nm, a, b in zip(["out", "d_hidden", "d_topk_weights", "d_w_gate_up", "d_w_down"], first, second):
        assert bool(torch.isfinite(a).all()), f"{name} {nm}: non-finite values"
        assert torch.equal(a, b), f"{name} {nm}: two runs differ"
    del first, second, Wgu, Wd
    torch.cuda.empty_cache()
