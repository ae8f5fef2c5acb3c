"""GPU parity of the HIP path (through the C ABI) with the fp64 oracle.

Small cases span several 128-row and 128-column tiles with ragged tails in
every dimension (H and I not multiples of 64, experts with more than two
M-tiles, empty experts); bf16 and fp32; SwiGLU and the clamped GLU;
concatenated and interleaved gate/up rows; saved and recomputed Z.
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_histogram_amd as moe
import oracle
from synth import WORKLOADS, HostInputs, Workload, make_all_weights, make_dout, make_hidden, make_host_inputs, make_routing
from tests._gpu import assert_parity, device_inputs, host, oracle_fwd_bwd, small_inputs

pytestmark = pytest.mark.gpu


def skewed_ids(T, K, E, seed):
    """Expert 0 gets ~40% of slots (several M-tiles), expert E-1 none."""
    rng = np.random.default_rng(seed)
    ids = np.where(rng.random((T, K)) < 0.4, 0, rng.integers(1, E - 1, size=(T, K)))
    return ids.astype(np.int32)


def gate_up_halves(x, layout):
    """(gate rows, up rows) of one expert's [2I, H] block."""
    I = x.shape[0] // 2
    return (x[0::2], x[1::2]) if layout == "interleaved" else (x[:I], x[I:])


def check_weight_grads(dgu, dd, r_dgu, r_dd, counts, layout, experts=None, bf16_workload=True):
    """Each expert's dW_gate, dW_up and dW_down is a parameter tensor of its own
    and meets the bar on its own scale; an expert with no slots gets zeros."""
    experts = range(len(counts)) if experts is None else experts
    bf = bf16_workload
    for e in experts:
        g_gu, g_d = host(dgu[e]), host(dd[e])
        if counts[e] == 0:
            assert np.all(g_gu == 0) and np.all(g_d == 0), f"expert {e} has no slots but nonzero dW"
            continue
        for half, (g, r) in zip(["gate", "up"], zip(gate_up_halves(g_gu, layout), gate_up_halves(r_dgu[e], layout))):
            assert_parity(g, r, f"dW_{half}[{e}]", stored_bf16=bf, kind="dW expert block")
        assert_parity(g_d, r_dd[e], f"dW_down[{e}]", stored_bf16=bf, kind="dW expert block")


def poisoned_buffers(wl, grad_dtype, dev="cuda"):
    """Workspaces, saved buffer and outputs of a fwd + bwd call, every byte
    0xFF (NaN for floats, -1 for integers), so an element a kernel fails to
    write, or a table it reads before writing, shows in the results."""
    desc = moe.make_desc(wl.T, wl.H, wl.I, wl.E, wl.K, wl.dtype, wl.act, wl.layout, wl.limit, wl.alpha,
                         grad_dtype or wl.dtype)
    fws, bws, sbytes = moe.workspace_size(desc)
    ff = lambda n: torch.full((max(n, 256),), 0xFF, dtype=torch.uint8, device=dev)
    adt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    gdt = torch.float32 if (grad_dtype or wl.dtype) == "fp32" else torch.bfloat16
    nan = lambda shape, dt: torch.full(shape, float("nan"), dtype=dt, device=dev)
    grads = (nan((wl.T, wl.H), adt), nan((wl.T, wl.K), torch.float32), nan((wl.E, 2 * wl.I, wl.H), gdt),
             nan((wl.E, wl.H, wl.I), gdt))
    return dict(ws_f=ff(fws), ws_b=ff(bws), saved=ff(sbytes), out=nan((wl.T, wl.H), adt), grads=grads)


def run_gpu(inp, save=True, grad_dtype=None, poison=False, ids=None, expect_status=0):
    """moe_fwd then moe_bwd on device copies of the inputs (ids: override the
    device topk_ids); returns (out, d_hidden, d_topk_weights, dW_gate_up, dW_down)."""
    wl = inp.wl
    d = device_inputs(inp)
    if ids is not None:
        d["topk_ids"] = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    kw = dict(act=wl.act, layout=wl.layout, limit=wl.limit, alpha=wl.alpha)
    bufs = poisoned_buffers(wl, grad_dtype) if poison else {}
    out, saved, ws = moe.fwd(d["hidden"], d["topk_ids"], d["topk_weights"], d["w_gate_up"], d["w_down"],
                             save=save, ws=bufs.get("ws_f"), out=bufs.get("out"),
                             saved=bufs.get("saved") if save else None, **kw)
    dh, dw, dgu, dd, ws2 = moe.bwd(d["hidden"], d["topk_ids"], d["topk_weights"], d["w_gate_up"], d["w_down"],
                                   d["d_out"], saved=saved, grad_dtype=grad_dtype, ws=bufs.get("ws_b"),
                                   grads=bufs.get("grads"), **kw)
    torch.cuda.synchronize()
    assert moe.check_device_status(ws) == expect_status and moe.check_device_status(ws2) == expect_status
    return out, dh, dw, dgu, dd


def run_and_compare(inp, save=True, grad_dtype=None, poison=False):
    wl = inp.wl
    out, dh, dw, dgu, dd = run_gpu(inp, save, grad_dtype, poison)
    ref_out, (r_dx, r_dw, r_dgu, r_dd) = oracle_fwd_bwd(inp)
    bf = wl.dtype == "bf16"
    assert_parity(host(out), ref_out, "out", kind="out")
    assert_parity(host(dh), r_dx, "d_hidden", kind="d_hidden")
    assert_parity(host(dw), r_dw, "d_topk_weights", kind="d_topk_weights")
    # stacked weight gradients (all experts as one tensor): the plain bar, with
    # only the bf16 store's half-ulp allowed when they are stored in bf16
    g16 = dgu.dtype == torch.bfloat16
    assert_parity(host(dgu), r_dgu, "d_w_gate_up", kind="dW stacked", stored_bf16=g16)
    assert_parity(host(dd), r_dd, "d_w_down", kind="dW stacked", stored_bf16=g16)
    check_weight_grads(dgu, dd, r_dgu, r_dd, np.bincount(inp.topk_ids.ravel(), minlength=wl.E), wl.layout,
                       bf16_workload=bf)
    return out, dh, dw, dgu, dd


# ------------------------------------------------------------------ routing
def check_route(ids, E):
    t = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    counts, offsets, ss, ip, ws = moe.route(t, E)
    torch.cuda.synchronize()
    c, o, s, i = oracle.route(ids, E)
    np.testing.assert_array_equal(counts.cpu().numpy(), c)
    np.testing.assert_array_equal(offsets.cpu().numpy(), o)
    np.testing.assert_array_equal(ss.cpu().numpy(), s)
    np.testing.assert_array_equal(ip.cpu().numpy(), i)
    assert moe.check_device_status(ws) == 0


@pytest.mark.parametrize("T,K,E,seed", [(1, 1, 1, 0), (7, 3, 5, 1), (1000, 4, 128, 2), (3000, 8, 256, 3),
                                        (513, 2, 1024, 4), (4096, 4, 3, 5), (257, 64, 17, 6)])
def test_route_random(T, K, E, seed):
    check_route(np.random.default_rng(seed).integers(0, E, size=(T, K)), E)


def test_route_edge_cases():
    check_route(np.zeros((5000, 4)), 8)                       # every slot to one expert
    check_route(np.full((300, 2), 6), 7)                      # only the last expert
    check_route(skewed_ids(2049, 3, 9, 0), 9)                 # chunk boundary + empty expert
    ids = np.random.default_rng(1).integers(0, 4, size=(777, 5))
    ids[:, 1] = ids[:, 0]                                     # duplicates inside each token
    check_route(ids, 4)


@pytest.mark.parametrize("name", ["gptoss", "large", "zipf"])
def test_route_workloads(name):
    wl = WORKLOADS[name]
    ids, _ = make_routing(wl)
    check_route(ids, wl.E)


def test_route_bad_id_sets_flag():
    ids = np.random.default_rng(2).integers(0, 8, size=(100, 2)).astype(np.int32)
    ids[10, 1] = 8
    ids[50, 0] = -3
    t = torch.from_numpy(ids).cuda()
    counts, offsets, ss, ip, ws = moe.route(t, 8)
    assert moe.check_device_status(ws) == 5
    good = np.ones(200, bool)
    good[[21, 100]] = False
    f = ids.ravel()
    np.testing.assert_array_equal(counts.cpu().numpy(), np.bincount(f[good], minlength=8))
    ipn = ip.cpu().numpy()
    assert ipn[21] == -1 and ipn[100] == -1
    # the good slots keep their stable order; the bad ones follow, in slot order
    order = np.argsort(np.where(good, f, 99), kind="stable")[:198]
    np.testing.assert_array_equal(ss.cpu().numpy()[:198], order)
    np.testing.assert_array_equal(ss.cpu().numpy()[198:], [21, 100])
    assert offsets.cpu().numpy()[-1] == 198


# ------------------------------------------------------------------ fwd + bwd
def test_tiny_fp32_workload():
    run_and_compare(make_host_inputs(WORKLOADS["tiny"], seed=0))


@pytest.mark.parametrize("act,layout", [("swiglu", "concat"), ("swiglu", "interleaved"),
                                        ("clamped", "interleaved"), ("clamped", "concat")])
@pytest.mark.parametrize("dtype,grad_dtype", [("bf16", "fp32"), ("bf16", "bf16"), ("fp32", "fp32")])
def test_small_ragged(act, layout, dtype, grad_dtype):
    T, H, I, E, K = 300, 328, 200, 6, 3
    inp = small_inputs(T, H, I, E, K, dtype, act, layout, seed=3, ids=skewed_ids(T, K, E, 3))
    run_and_compare(inp, grad_dtype=grad_dtype)


@pytest.mark.parametrize("save", [True, False])
def test_saved_and_recomputed_z_agree(save):
    T, H, I, E, K = 200, 256, 192, 5, 2
    inp = small_inputs(T, H, I, E, K, "bf16", "swiglu", "concat", seed=4)
    run_and_compare(inp, save=save, grad_dtype="fp32")


def test_clamps_exercised():
    T, H, I, E, K = 256, 136, 72, 4, 2
    inp = small_inputs(T, H, I, E, K, "bf16", "clamped", "interleaved", seed=5, xscale=30.0)
    z = np.stack([inp.hidden[s // K] @ inp.w_gate_up[inp.topk_ids.ravel()[s]].T.astype(np.float64)
                  for s in range(T * K)])
    assert np.mean(np.abs(z) > 7) > 0.05
    run_and_compare(inp, grad_dtype="fp32")


@pytest.mark.parametrize("grad_dtype", ["fp32", "bf16"])
def test_no_tokens_gives_zero_weight_grads(grad_dtype):
    """T = 0: every expert is empty, so every weight gradient is exactly zero
    (the outputs start as NaN, so a tile the kernels skip would show)."""
    H, I, E, K = 264, 136, 5, 2
    dev = "cuda"
    g = torch.Generator(device="cpu").manual_seed(7)
    wgu = torch.randn(E, 2 * I, H, generator=g).to(torch.bfloat16).to(dev)
    wd = torch.randn(E, H, I, generator=g).to(torch.bfloat16).to(dev)
    hidden = torch.empty((0, H), dtype=torch.bfloat16, device=dev)
    ids = torch.empty((0, K), dtype=torch.int32, device=dev)
    w = torch.empty((0, K), dtype=torch.float32, device=dev)
    d_out = torch.empty((0, H), dtype=torch.bfloat16, device=dev)
    gdt = torch.float32 if grad_dtype == "fp32" else torch.bfloat16
    grads = (torch.empty((0, H), dtype=torch.bfloat16, device=dev), torch.empty((0, K), dtype=torch.float32, device=dev),
             torch.full((E, 2 * I, H), float("nan"), dtype=gdt, device=dev),
             torch.full((E, H, I), float("nan"), dtype=gdt, device=dev))
    # a workspace whose status word holds a stale flag: the T = 0 calls clear it
    _, bws, _ = moe.workspace_size(moe.make_desc(0, H, I, E, K, grad_dtype=grad_dtype))
    ws = torch.full((bws,), 7, dtype=torch.uint8, device=dev)
    out, _, ws = moe.fwd(hidden, ids, w, wgu, wd, ws=ws)
    assert moe.check_device_status(ws) == 0 and out.shape == (0, H)
    ws.fill_(7)
    _, _, dgu, dd, ws = moe.bwd(hidden, ids, w, wgu, wd, d_out, grads=grads, grad_dtype=grad_dtype, ws=ws)
    torch.cuda.synchronize()
    assert moe.check_device_status(ws) == 0
    assert bool((dgu == 0).all()) and bool((dd == 0).all())


@pytest.mark.parametrize("E,K", [(1, 1), (1, 3), (2, 4)])
def test_degenerate_expert_counts(E, K):
    """One expert (every slot lands on it, repeatedly when K > 1) and more
    slots per token than experts: repeated ids are independent slots."""
    T, H, I = 150, 136, 72
    rng = np.random.default_rng(E * 10 + K)
    wl = Workload("degenerate", T, H, I, E, K, "bf16", "swiglu", "concat")
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    gu, dn = make_all_weights(wl, seed=E + K)
    inp = HostInputs(wl, make_hidden(wl, E + K), ids, w, make_dout(wl, E + K), gu, dn)
    run_and_compare(inp, grad_dtype="bf16")


@pytest.mark.parametrize("act,layout", [("swiglu", "concat"), ("clamped", "interleaved")])
def test_large_experts_ragged(act, layout):
    """Experts averaging several hundred slots (the 256-row tile shape) with
    ragged H and I and one expert holding ~40 % of all slots."""
    T, H, I, E, K = 900, 328, 200, 4, 2
    inp = small_inputs(T, H, I, E, K, "bf16", act, layout, seed=21, ids=skewed_ids(T, K, E, 21))
    assert T * K // E >= 320
    run_and_compare(inp, grad_dtype="bf16")


@pytest.mark.parametrize("grad_dtype", ["bf16", "fp32"])
def test_weight_grad_expert_sizes(grad_dtype):
    """Experts of 0, 1, 16, 17, 208, 209, 240, 241, 256, 257, 512, 513 and
    1601 slots: the resident-operand weight gradient takes experts of up to
    240 slots (k-slices of 16, zeros for an empty expert), the long-K one
    those above 512 (ragged last k-step) and the tiled one the rest, all in
    one call, for bf16 and for fp32 gradient storage."""
    counts = [1601, 513, 512, 256, 257, 240, 241, 208, 209, 1, 16, 17, 0]
    E, K = len(counts), 1
    T, H, I = sum(counts), 264, 200
    rng = np.random.default_rng(31)
    ids = rng.permutation(np.repeat(np.arange(E), counts)).reshape(T, K).astype(np.int32)
    inp = small_inputs(T, H, I, E, K, "bf16", "clamped", "interleaved", seed=31, ids=ids)
    run_and_compare(inp, grad_dtype=grad_dtype)


@pytest.mark.parametrize("save", [True, False])
def test_poisoned_buffers_ragged(save):
    """Workspaces, saved buffer and every output start as 0xFF bytes (NaN);
    a ragged multi-tile case must still match the oracle everywhere."""
    T, H, I, E, K = 300, 328, 200, 6, 3
    inp = small_inputs(T, H, I, E, K, "bf16", "clamped", "interleaved", seed=9, ids=skewed_ids(T, K, E, 9))
    run_and_compare(inp, save=save, grad_dtype="bf16", poison=True)


@pytest.mark.parametrize("save", [True, False])
def test_bad_expert_ids_are_dropped(save):
    """Ids outside [0, E) (E, E + 100 and -1): the device flags them, nothing
    outside the caller's buffers is touched (the backward gathers rows for
    every position, including the bad slots placed last), and every output
    equals the oracle's for the same inputs with those slots' routing weight
    set to zero, except d_topk_weights of a bad slot, which is 0.  Buffers
    start as NaN so a skipped element shows."""
    T, H, I, E, K = 300, 328, 200, 6, 3
    inp = small_inputs(T, H, I, E, K, "bf16", "swiglu", "concat", seed=11, ids=skewed_ids(T, K, E, 11))
    bad_ids = inp.topk_ids.copy()
    bad = [(5, 1, E), (77, 0, -1), (150, 2, E + 100), (299, 2, E)]
    for t, k, v in bad:
        bad_ids[t, k] = v
    out, dh, dw, dgu, dd = run_gpu(inp, save=save, grad_dtype="bf16", poison=True, ids=bad_ids,
                                   expect_status=moe.MOE_ERR_BAD_EXPERT_ID)
    # the oracle's inputs: bad slots on expert 0 with weight 0
    for t, k, _ in bad:
        inp.topk_ids[t, k] = 0
        inp.topk_weights[t, k] = 0.0
    ref_out, (r_dx, r_dw, r_dgu, r_dd) = oracle_fwd_bwd(inp)
    assert_parity(host(out), ref_out, "out (bad ids dropped)", kind="out")
    assert_parity(host(dh), r_dx, "d_hidden (bad ids dropped)", kind="d_hidden")
    g_dw = host(dw)
    keep = np.ones((T, K), bool)
    for t, k, _ in bad:
        keep[t, k] = False
        assert g_dw[t, k] == 0.0
    assert_parity(g_dw[keep], r_dw[keep], "d_topk_weights (bad ids dropped)", kind="d_topk_weights")
    assert_parity(host(dgu), r_dgu, "d_w_gate_up (bad ids dropped)", kind="dW stacked", stored_bf16=True)
    assert_parity(host(dd), r_dd, "d_w_down (bad ids dropped)", kind="dW stacked", stored_bf16=True)
    counts = np.bincount(bad_ids.ravel()[(bad_ids.ravel() >= 0) & (bad_ids.ravel() < E)], minlength=E)
    check_weight_grads(dgu, dd, r_dgu, r_dd, counts, "concat")
