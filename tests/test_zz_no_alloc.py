"""moe_fwd_noalloc: the forward with the library's own per-GPU scratch array
as its workspace, for callers that cannot allocate device memory.

On the GPU its outputs must equal moe_fwd's bit for bit (same kernels, same
order), on two calls in a row with the second smaller, so the array's
leftover contents from the first call must not leak into the second.  On the
host, shapes whose workspace exceeds the array are rejected before any
device call.
"""
import ctypes

import numpy as np
import pytest
import torch

import mixture_experts_expert_histogram_amd as moe
from mixture_experts_expert_histogram_amd import _lib


def test_noalloc_rejects_shapes_beyond_the_scratch_array():
    d = moe.make_desc(32768, 2880, 2880, 128, 4, "bf16", "clamped", "interleaved")
    fws, _, _ = moe.workspace_size(d)
    assert fws > moe.NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(16)
    lib = moe.library()
    assert lib.moe_fwd_noalloc(ctypes.byref(d), p, p, p, p, p, p, None, 0, None, None) == _lib.MOE_ERR_WORKSPACE
    small = moe.make_desc(512, 2880, 2880, 128, 4, "bf16", "clamped", "interleaved")
    assert moe.workspace_size(small)[0] <= moe.NOALLOC_SCRATCH_BYTES
    assert lib.moe_fwd_noalloc(ctypes.byref(small), p, None, p, p, p, p, None, 0, None,
                               None) == _lib.MOE_ERR_INVALID_ARG


def _inputs(T, H, I, E, K, seed, dev="cuda", hot=0.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    X = torch.randn(T, H, generator=g).to(torch.bfloat16).to(dev)
    logits = torch.randn(T, E, generator=g)
    logits[:, 0] += hot   # hot > 0: expert 0 takes (nearly) every token
    top = torch.topk(logits, K, dim=1)
    ids = top.indices.to(torch.int32).to(dev)
    w = torch.softmax(top.values, dim=1).to(torch.float32).to(dev)
    Wgu = (0.02 * torch.randn(E, 2 * I, H, generator=g)).to(torch.bfloat16).to(dev)
    Wd = (0.02 * torch.randn(E, H, I, generator=g)).to(torch.bfloat16).to(dev)
    return X, ids, w, Wgu, Wd


@pytest.mark.gpu
@pytest.mark.parametrize("act,layout", [("clamped", "interleaved"), ("swiglu", "concat")])
def test_noalloc_forward_equals_moe_fwd(act, layout):
    H, I, E, K = 1024, 512, 16, 4
    # calls in a row, each smaller than the one before; the first gives expert
    # 0 every token (900 slots: the 256 x 256-tile kernels), the others
    # spread the slots (the 128-row tiles only)
    for T, seed, hot in [(900, 3, 50.0), (700, 1, 0.0), (96, 2, 0.0)]:
        X, ids, w, Wgu, Wd = _inputs(T, H, I, E, K, seed, hot=hot)
        if hot:
            assert int((ids == 0).sum()) >= 512
        kw = dict(act=act, layout=layout)
        ref, ref_saved, ws = moe.fwd(X, ids, w, Wgu, Wd, save=True, **kw)
        sbytes = moe.workspace_size(moe.make_desc(T, H, I, E, K, "bf16", act, layout))[2]
        saved = torch.full((sbytes,), 0xFF, dtype=torch.uint8, device="cuda")
        out = torch.full_like(X, float("nan"))
        bad = torch.full((4,), -7, dtype=torch.int32, device="cuda")
        moe.fwd_noalloc(X, ids, w, Wgu, Wd, out=out, saved=saved, bad_ids=bad, **kw)
        torch.cuda.synchronize()
        assert moe.check_device_status(ws) == 0
        assert int(bad[0]) == 0
        assert torch.equal(out, ref), f"T={T}: outputs differ"
        assert torch.equal(saved, ref_saved), f"T={T}: saved Z differs"
