"""Benchmark of the routed MoE expert computation on one MI355X.

A step is one forward (moe_fwd, keeping Z for the backward) plus one backward
(moe_bwd) of a routed MoE layer over one batch of synthetic tokens: routing
permutation, gate_up projection with the gated activation, down projection
with the routing weight, per-token combine, then the backward's input
gradients, routing-weight gradients and weight gradients.

The default workload is the largest one that fits one GPU: the gpt-oss layer
shape (H = I = 2880, E = 128, top-4, clamped GLU) at T = 32768 tokens with
Zipf(1.2) expert popularity, forward plus backward.

Prints one JSON line.  `value` is useful routed TFLOP/s over the whole step:
forward 6*S*H*I plus backward 12*S*H*I floating-point operations (S = T*K),
with inputs and weights resident in HBM before the timed region starts.  The
timed region records no per-kernel events; a second, instrumented pass over
the same steps gives each kernel's average launch time for `roofline`.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
METRIC = "ms/layer and routed TFLOP/s (fwd, bwd) at 1 MI355X; % of bf16 MFMA peak"


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="zipf", help="synthetic workload name (synth.WORKLOADS)")
    p.add_argument("--grad-dtype", default="bf16", choices=["fp32", "bf16"],
                   help="weight-gradient storage (accumulation is fp32 either way); bf16 is the parameter dtype")
    p.add_argument("--no-alt-grad-dtype", action="store_true",
                   help="skip the extra timing of the same steps with fp32 weight-gradient storage")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle's CPU sample")
    p.add_argument("--no-kernel-timing", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (for scaling HBM counters) and exit")
    p.add_argument("--protocol", action="store_true",
                   help="time every workload's passes (forward with Z saved or not, backward with saved Z or "
                        "recomputing it) with a cache flush between iterations; one JSON line per case")
    p.add_argument("--sweep", action="store_true",
                   help="token-count sweep: 16 values of T per layer shape, forward and backward; "
                        "one JSON line per case and a mean-latency line per shape")
    p.add_argument("--shapes", default="gptoss,large,backward", help="layer shapes of --sweep")
    p.add_argument("--iters", type=int, default=20, help="timed iterations per case of --protocol / --sweep")
    p.add_argument("--oracle-seconds", type=float, default=6.0,
                   help="CPU budget of each workload's oracle sample in --protocol")
    return p.parse_args()


COPY_BYTES = 1 << 30


def copy_calibration():
    """A plain device-to-device copy of COPY_BYTES, repeated 5 times (the
    reference for scaling FETCH_SIZE / WRITE_SIZE counters to bytes)."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 5}), flush=True)


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_expert_histogram_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload, grad_dtype):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None if there is none, it was taken on another workload or weight-gradient
    dtype, or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if (rec.get("source_hash") != kernel_source_hash() or rec.get("workload") != workload
            or rec.get("grad_dtype") != grad_dtype):
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


# ------------------------------------------------------------------ per-kernel model
RES_KMAX = 240   # the resident-operand weight gradient's limit (positions per expert)
LONG_MIN = 512  # experts with more positions take the long-K weight gradient (without the large-tile engine)
LARGE_MIN = 512  # experts with at least this many slots take the 256-row token-row tiles


def large_tile_experts(wl, counts):
    """Experts the library runs on the 256-row tiles: from LARGE_MIN slots on,
    and below that those whose 256-row tiles hold no more rows than the other
    tiles (192 rows when the batch averages 101-176 slots per expert and H or
    I is not a multiple of 64, else 128) would."""
    import numpy as np
    counts = np.asarray(counts)
    if not large_tiles(wl):
        return np.zeros(len(counts), dtype=bool)
    mean = wl.S // wl.E if wl.E else 0
    dma_small = large_tiles(wl) and wl.H % 64 == 0 and wl.I % 64 == 0   # the small experts' 128-row DMA tiles
    bms = 192 if 100 < mean <= 176 and not dma_small else 128
    rows_big = (counts + 255) // 256 * 256
    rows_small = (counts + bms - 1) // bms * bms
    return (counts >= LARGE_MIN) | ((counts > 0) & (rows_big <= rows_small))


def large_wgrad(wl):
    """Whether the weight gradients of experts above RES_KMAX positions run on
    the large-tile engine (its token-row conditions, and every position row of
    dZ and the hidden states below 2^31 bytes)."""
    lim = 1 << 31
    return large_tiles(wl) and wl.S * 4 * wl.I < lim and wl.S * 2 * wl.H < lim


def large_tiles(wl):
    """Whether the library runs the 256 x 256-tile engine for this workload's
    big experts (bf16 operands, H and I multiples of 32, offsets in range)."""
    lim = 1 << 31
    return (wl.dtype == "bf16" and wl.H % 32 == 0 and wl.I % 32 == 0 and wl.T * wl.H * 2 < lim
            and 4 * wl.I * wl.H < lim and 256 * 4 * wl.I < lim and 256 * 2 * wl.H < lim)


def kernel_model(wl, counts, grad_bytes):
    """Algorithmic bytes and routed flops of one launch of each kernel.

    Bytes are the layer's own inputs and outputs that the kernel must move,
    each element once: the weights of the experts that receive slots (read by
    the projections and their input gradients), the hidden states and output
    gradient rows (read), and the weight gradients (written).  The per-slot
    intermediates (the activation, Z, dZ, the permuted rows, the per-slot
    expert outputs) are implementation traffic and are not counted, except
    for the data-movement kernels (combine, row gather, routing-weight
    reduce), whose whole work is moving them.  Flops count the routed work
    only (2*M*N*K per product over the slots).
    """
    S, T, H, I = wl.S, wl.T, wl.H, wl.I
    eb = 2 if wl.dtype == "bf16" else 4
    m = {
        "combine": (S * H * 4 + T * H * eb + S * 4, 0.0),
        "gather_rows": (2 * S * H * eb + S * 4, 0.0),
        "topkw_reduce": (S * 4 * 2, 0.0),
    }

    # Token-row products.  Experts with at least LARGE_MIN slots run on the
    # 256-row tiles (*_big) when the workload allows them, the rest on the
    # 128/192-row tiles; each part is charged its experts' weights and the
    # hidden / output-gradient rows prorated by its slots.
    def rows(sel, suffix):
        touched = int(((counts > 0) & sel).sum())
        s_part = int(counts[sel].sum())
        tok = s_part / S if S else 0.0
        Wgu, Wd = touched * 2 * I * H * eb, touched * H * I * eb
        m["gate_up_glu" + suffix] = (Wgu + tok * T * H * eb, 4.0 * s_part * H * I)
        m["down_weighted" + suffix] = (Wd, 2.0 * s_part * H * I)
        m["down_dgrad_glu_bwd" + suffix] = (Wd + tok * T * H * eb, 2.0 * s_part * H * I)
        m["gate_up_dgrad" + suffix] = (Wgu, 4.0 * s_part * H * I)
    import numpy as np
    counts = np.asarray(counts)
    big = large_tile_experts(wl, counts)
    rows(~big, "")
    if big.any():
        rows(big, "_big")
    # Weight gradients.  With bf16 operands, experts with at most RES_KMAX
    # positions (and those without any) take the resident-operand kernel,
    # named wgrad_down / wgrad_gate_up; the rest take the large-tile kernel
    # (*_long) where that engine applies, else those with more than LONG_MIN
    # the long-K kernel (*_long) and the others the tiled one (*_hot); with fp32
    # operands the tiled kernel takes every expert under the plain names.
    # Each writes its experts' gradients; the hidden / output-gradient rows it
    # reads are prorated by the positions it covers.
    def wgrad(sel):
        s_part = int(counts[sel].sum())
        e_part = int(sel.sum())
        tok = s_part / S if S else 0.0
        down = (tok * T * H * eb + e_part * H * I * grad_bytes, 2.0 * s_part * H * I)
        gu = (tok * T * H * eb + e_part * 2 * I * H * grad_bytes, 4.0 * s_part * H * I)
        return down, gu
    if wl.dtype == "bf16":
        small = counts <= RES_KMAX
        long_ = counts > (RES_KMAX if large_wgrad(wl) else LONG_MIN)
        mid = ~small & ~long_
        m["wgrad_down"], m["wgrad_gate_up"] = wgrad(small)
        if mid.any():
            m["wgrad_down_hot"], m["wgrad_gate_up_hot"] = wgrad(mid)
        if long_.any():
            m["wgrad_down_long"], m["wgrad_gate_up_long"] = wgrad(long_)
    else:
        m["wgrad_down"], m["wgrad_gate_up"] = wgrad(counts >= 0)
    return m


def roofline_for(name, avg_ms, model):
    """Achieved rate of one kernel against the roof that bounds it: MFMA when
    its routed flops take longer at the bf16 dense peak than its algorithmic
    bytes at the HBM peak, else HBM."""
    nbytes, flops = model[name]
    t_hbm = nbytes / (PEAK_HBM_GBPS * 1e9)
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    if t_mfma > t_hbm:
        ach = flops / (avg_ms * 1e-3) / 1e12
        return {"kernel": name, "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "avg_ms": round(avg_ms, 4), "algorithmic_bytes": nbytes, "flops": flops}
    ach = nbytes / (avg_ms * 1e-3) / 1e9
    return {"kernel": name, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": None, "avg_ms": round(avg_ms, 4),
            "algorithmic_bytes": nbytes, "flops": flops}


# ------------------------------------------------------------------ per-pass roofline
def pass_model(wl, counts, pass_, grad_bytes):
    """Useful flops, algorithmic HBM bytes and weight-stream bytes of one pass.

    Useful flops count the routed work only: 6*S*H*I forward, 12*S*H*I
    backward (a Z recompute is not useful work).  Algorithmic bytes are the
    weights of the experts that receive slots (read), the hidden states in
    and the output out (forward); the backward adds the output gradient in,
    the input gradient out and every expert's weight gradient out (the
    outputs are fully written, zeros for experts without slots).
    Intermediates (the activation, Z, the permuted rows) are not counted.
    """
    S, T, H, I, E = wl.S, wl.T, wl.H, wl.I, wl.E
    eb = 2 if wl.dtype == "bf16" else 4
    touched = int((counts > 0).sum())
    w_read = touched * 3 * H * I * eb
    route = T * wl.K * 8
    if pass_ == "fwd":
        flops = 6.0 * S * H * I
        nbytes = w_read + 2 * T * H * eb + route
        stream = w_read
    else:
        flops = 12.0 * S * H * I
        dw = E * 3 * H * I * grad_bytes
        nbytes = w_read + dw + 3 * T * H * eb + route + T * wl.K * 4
        stream = w_read + dw
    return flops, nbytes, stream


def pass_record(wl, counts, pass_, grad_bytes, times_ms):
    import numpy as np
    flops, nbytes, stream = pass_model(wl, counts, pass_, grad_bytes)
    t = np.asarray(times_ms, dtype=np.float64)
    med, mn, mean = float(np.median(t)), float(t.min()), float(t.mean())
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12) * 1e3
    t_hbm = nbytes / (PEAK_HBM_GBPS * 1e9) * 1e3
    t_roof = max(t_mfma, t_hbm)
    return {"median_ms": round(med, 4), "min_ms": round(mn, 4), "mean_ms": round(mean, 4),
            "tflops": round(flops / (med * 1e-3) / 1e12, 2),
            "pct_of_bf16_peak": round(100 * flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "bound": "mfma" if t_mfma >= t_hbm else "hbm", "t_roof_ms": round(t_roof, 4),
            "pct_of_roofline": round(100 * t_roof / med, 2),
            "weight_stream_gbps": round(stream / (med * 1e-3) / 1e9, 1),
            "useful_gflop": round(flops / 1e9, 1), "algorithmic_gb": round(nbytes / 1e9, 3),
            "experts_with_slots": int((counts > 0).sum())}


def oracle_record(wl, runner, budget_s):
    """The fp64 oracle (forward + backward) on whole experts of the workload,
    one after another until `budget_s` seconds of CPU time are spent; the tiny
    workload instead runs whole, ten times (median)."""
    import numpy as np
    import oracle
    from synth import make_dout, make_hidden, make_host_inputs
    if wl.name == "tiny":
        inp = make_host_inputs(wl, 0)
        ex = oracle.expert_accessor(inp.w_gate_up, inp.w_down)
        times = []
        for _ in range(10):
            t0 = time.perf_counter()
            oracle.forward(inp.hidden, inp.topk_ids, inp.topk_weights, ex, wl.E, wl.act, wl.layout, wl.limit, wl.alpha)
            oracle.backward(inp.hidden, inp.topk_ids, inp.topk_weights, inp.dout, ex, wl.E, wl.act, wl.layout,
                            wl.limit, wl.alpha)
            times.append(time.perf_counter() - t0)
        sec = float(np.median(times))
        return {"workload": wl.name, "pass": "oracle fwd+bwd", "seconds": round(sec, 4),
                "gflops": round(18.0 * wl.S * wl.H * wl.I / sec / 1e9, 3), "sample": "whole workload, median of 10"}
    rec = cpu_baseline(wl, runner.ids_np, runner.w_np, make_hidden(wl, 0), make_dout(wl, 0), runner.Wgu, runner.Wd,
                       budget_s)
    return {"workload": wl.name, "pass": "oracle fwd+bwd", "seconds": rec["seconds"],
            "gflops": round(rec["value"] * 1e3, 3), "cores": rec["cores"], "sample": rec["sample"]}


class PassRunner:
    """Resident inputs, weights, outputs and workspaces of one workload, and
    the timing of its passes with a 512 MiB write between iterations (larger
    than the 256 MiB last-level cache, so activations start cold as the
    weights do)."""

    FLUSH_BYTES = 512 << 20

    def __init__(self, wl, dev, weights=None, grad_dtype="bf16", seed=0):
        import numpy as np
        import torch
        import mixture_experts_expert_histogram_amd as moe
        from synth import device_weights, make_dout, make_hidden, make_routing, to_device
        self.moe, self.torch, self.wl, self.grad_dtype = moe, torch, wl, grad_dtype
        ids_np, w_np = make_routing(wl, seed=seed)
        self.ids_np, self.w_np = ids_np, w_np
        self.counts = np.bincount(ids_np.ravel(), minlength=wl.E)
        self.X = to_device(make_hidden(wl, seed), wl, dev)
        self.dY = to_device(make_dout(wl, seed), wl, dev)
        self.ids = torch.from_numpy(ids_np).to(dev)
        self.w = torch.from_numpy(w_np).to(dev)
        self.Wgu, self.Wd = weights if weights is not None else device_weights(wl, dev, seed=seed)
        self.kw = dict(act=wl.act, layout=wl.layout, limit=wl.limit, alpha=wl.alpha)
        desc = moe.make_desc(wl.T, wl.H, wl.I, wl.E, wl.K, wl.dtype, wl.act, wl.layout, wl.limit, wl.alpha,
                             grad_dtype)
        fws, bws, sbytes = moe.workspace_size(desc)
        self.ws_f, self.ws_b = moe.empty_workspace(fws, dev), moe.empty_workspace(bws, dev)
        self.saved = moe.empty_workspace(sbytes, dev)
        self.out = torch.empty_like(self.X)
        gdt = torch.float32 if grad_dtype == "fp32" else torch.bfloat16
        self.grads = (torch.empty_like(self.X), torch.empty((wl.T, wl.K), dtype=torch.float32, device=dev),
                      torch.empty(self.Wgu.shape, dtype=gdt, device=dev),
                      torch.empty(self.Wd.shape, dtype=gdt, device=dev))
        self.flush = torch.empty(self.FLUSH_BYTES, dtype=torch.uint8, device=dev)
        self.grad_bytes = 4 if grad_dtype == "fp32" else 2

    def fwd(self, save):
        self.moe.fwd(self.X, self.ids, self.w, self.Wgu, self.Wd, save=save, ws=self.ws_f, out=self.out,
                     saved=self.saved if save else None, **self.kw)

    def bwd(self, saved):
        self.moe.bwd(self.X, self.ids, self.w, self.Wgu, self.Wd, self.dY, saved=self.saved if saved else None,
                     ws=self.ws_b, grads=self.grads, grad_dtype=self.grad_dtype, **self.kw)

    def time(self, fn, warmup, iters):
        torch = self.torch
        for _ in range(warmup):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        for a, b in ev:
            self.flush.fill_(1)
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        if self.moe.check_device_status(self.ws_f) != 0:
            raise RuntimeError("bad expert id reported by the device")
        return [a.elapsed_time(b) for a, b in ev]

    def run_pass(self, pass_, saved, warmup, iters):
        if pass_ == "fwd":
            times = self.time(lambda: self.fwd(saved), warmup, iters)
        else:
            self.fwd(True)          # untimed: routing and Z for the backward
            times = self.time(lambda: self.bwd(saved), warmup, iters)
        return pass_record(self.wl, self.counts, pass_, self.grad_bytes, times)


# The passes timed per workload: the gpt-oss and large shapes' forward without
# Z kept; the backward workload's backward with saved Z and recomputing it;
# the Zipf workload's forward with and without Z kept and its backward both ways.
PROTOCOL = [("gptoss", "fwd", False), ("gptoss", "fwd", True), ("gptoss", "bwd", True), ("gptoss", "bwd", False),
            ("large", "fwd", False),
            ("backward", "bwd", True), ("backward", "bwd", False),
            ("zipf", "fwd", True), ("zipf", "fwd", False), ("zipf", "bwd", True), ("zipf", "bwd", False)]


def router_record(wl, dev, warmup, iters, seed=0):
    """Time moe_router on the workload's router logits (fp32 [T,E]) and, for
    comparison, moe_route on the ids it produces, each iteration after a
    512 MiB cache flush.  Algorithmic bytes: logits in, ids and weights out,
    the slot permutation and its inverse out."""
    import numpy as np
    import torch
    import mixture_experts_expert_histogram_amd as moe
    from synth import router_logits
    lg = torch.from_numpy(router_logits(wl.T, wl.E, seed)).to(dev)
    flush = torch.empty(PassRunner.FLUSH_BYTES, dtype=torch.uint8, device=dev)
    d = moe.make_desc(wl.T, 8, 8, wl.E, wl.K)
    ws = moe.empty_workspace(moe.route_workspace_size(d), dev)
    ids = torch.empty((wl.T, wl.K), dtype=torch.int32, device=dev)
    w = torch.empty((wl.T, wl.K), dtype=torch.float32, device=dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        for a, b in ev:
            flush.fill_(1)
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3

    t_router = timed(lambda: moe.router(lg, wl.K, ws=ws, out=(ids, w)))
    t_route = timed(lambda: moe.route(ids, wl.E, ws=ws))
    if moe.check_device_status(ws) != 0:
        raise RuntimeError("bad expert id reported by the device")
    nbytes = wl.T * wl.E * 4 + wl.S * 8 + wl.S * 8
    return {"workload": wl.name, "pass": "router", "T": wl.T, "E": wl.E, "K": wl.K,
            "router_median_us": round(t_router, 2), "route_from_ids_median_us": round(t_route, 2),
            "algorithmic_mb": round(nbytes / 1e6, 3), "router_gbps": round(nbytes / (t_router * 1e-6) / 1e9, 1)}


def separate_record(runner, warmup, iters):
    """The fwd (Z saved) + bwd step with the gate and up weights as two
    [E,I,H] tensors (moe_fwd_sep / moe_bwd_sep), beside the same step with
    the fused [E,2I,H] tensor, each iteration after the cache flush."""
    import numpy as np
    import torch
    import mixture_experts_expert_histogram_amd as moe
    wl = runner.wl
    I = wl.I
    W = runner.Wgu
    wg, wu = ((W[:, 0::2], W[:, 1::2]) if wl.layout == "interleaved" else (W[:, :I], W[:, I:]))
    wg, wu = wg.contiguous(), wu.contiguous()
    gdt = runner.grads[2].dtype
    sep_grads = (runner.grads[0], runner.grads[1], torch.empty_like(wg, dtype=gdt), torch.empty_like(wu, dtype=gdt),
                 runner.grads[3])
    kw = dict(act=wl.act, limit=wl.limit, alpha=wl.alpha)

    def step_sep():
        moe.fwd_sep(runner.X, runner.ids, runner.w, wg, wu, runner.Wd, save=True, ws=runner.ws_f, out=runner.out,
                    saved=runner.saved, **kw)
        moe.bwd_sep(runner.X, runner.ids, runner.w, wg, wu, runner.Wd, runner.dY, saved=runner.saved,
                    ws=runner.ws_b, grads=sep_grads, grad_dtype=runner.grad_dtype, **kw)

    def step_fused():
        runner.fwd(True)
        runner.bwd(True)

    t_sep = float(np.median(runner.time(step_sep, warmup, iters)))
    t_fused = float(np.median(runner.time(step_fused, warmup, iters)))
    flops = 18.0 * wl.S * wl.H * wl.I
    return {"workload": wl.name, "pass": "fwd+bwd", "mode": "separate gate/up weights", "median_ms": round(t_sep, 4),
            "tflops": round(flops / (t_sep * 1e-3) / 1e12, 2), "fused_median_ms": round(t_fused, 4)}


def run_protocol(args):
    import torch
    from synth import WORKLOADS
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    for name in ("gptoss", "large", "backward", "zipf"):
        print(json.dumps(router_record(WORKLOADS[name], dev, args.warmup, args.iters)), flush=True)
    runner = PassRunner(WORKLOADS["gptoss"], dev, grad_dtype=args.grad_dtype)
    print(json.dumps(separate_record(runner, args.warmup, args.iters)), flush=True)
    print(json.dumps(oracle_record(WORKLOADS["tiny"], None, 0)), flush=True)
    current, runner = None, None
    for name, pass_, saved in PROTOCOL:
        if name != current:
            runner = None
            torch.cuda.empty_cache()
            print(f"[protocol] {name}: drawing inputs", file=sys.stderr, flush=True)
            runner = PassRunner(WORKLOADS[name], dev, grad_dtype=args.grad_dtype)
            current = name
            if not args.no_cpu_baseline:
                print(json.dumps(oracle_record(runner.wl, runner, args.oracle_seconds)), flush=True)
        rec = runner.run_pass(pass_, saved, args.warmup, args.iters)
        wl = runner.wl
        mode = ("Z saved" if saved else "Z not kept") if pass_ == "fwd" else ("saved Z" if saved else "recompute Z")
        line = {"workload": name, "pass": pass_, "mode": mode, "T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E,
                "K": wl.K, "grad_dtype": args.grad_dtype if pass_ == "bwd" else None,
                "iters": args.iters, "warmup": args.warmup}
        line.update(rec)
        print(json.dumps(line), flush=True)


SWEEP_T = [1 << k for k in range(16)]     # 16 token counts per shape, 1 .. 32768


def run_sweep(args):
    import numpy as np
    import torch
    from synth import WORKLOADS, device_weights
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    for name in args.shapes.split(","):
        base = WORKLOADS[name]
        torch.cuda.empty_cache()
        weights = device_weights(base, dev, seed=0)
        lat = {"fwd": [], "bwd": []}
        for T in SWEEP_T:
            wl = base.with_(T=T)
            runner = PassRunner(wl, dev, weights=weights, grad_dtype=args.grad_dtype)
            for pass_ in ("fwd", "bwd"):
                rec = runner.run_pass(pass_, pass_ == "bwd", args.warmup, args.iters)
                lat[pass_].append(rec["mean_ms"])
                line = {"shape": name, "pass": pass_, "T": T, "S": wl.S}
                line.update(rec)
                print(json.dumps(line), flush=True)
            del runner
        for pass_ in ("fwd", "bwd"):
            print(json.dumps({"shape": name, "pass": pass_, "cases": len(SWEEP_T),
                              "mean_latency_ms": round(float(np.mean(lat[pass_])), 4)}), flush=True)
        del weights


# ------------------------------------------------------------------ CPU baseline
def cpu_baseline(wl, ids, w, X, dY, Wgu_dev, Wd_dev, budget_s):
    """The fp64 oracle on a bounded sample: whole experts of this workload,
    forward + backward, one expert after another until the budget is spent."""
    import numpy as np
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    counts = np.bincount(ids.ravel(), minlength=wl.E)
    order = [e for e in np.argsort(-counts, kind="stable") if counts[e] > 0]
    rng = np.random.default_rng(0)
    order = list(rng.permutation(order))
    flat_ids, flat_w = ids.ravel(), w.ravel()
    done_slots, elapsed, experts = 0, 0.0, 0
    for e in order:
        slots = np.nonzero(flat_ids == e)[0]
        tok = slots // wl.K
        gu = Wgu_dev[e].float().cpu().numpy()
        dn = Wd_dev[e].float().cpu().numpy()
        sub_ids = np.zeros((len(slots), 1), dtype=np.int32)
        sub_w = flat_w[slots].reshape(-1, 1)
        acc = oracle.expert_accessor(lambda _e: (gu, dn))
        t0 = time.perf_counter()
        oracle.forward(X[tok], sub_ids, sub_w, acc, 1, wl.act, wl.layout, wl.limit, wl.alpha)
        oracle.backward(X[tok], sub_ids, sub_w, dY[tok], acc, 1, wl.act, wl.layout, wl.limit, wl.alpha)
        elapsed += time.perf_counter() - t0
        done_slots += len(slots)
        experts += 1
        if elapsed >= budget_s:
            break
    flops = 18.0 * done_slots * wl.H * wl.I
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{experts} whole experts ({done_slots} slots) of the workload, fp64 forward+backward, "
                      f"{elapsed:.1f} s", "seconds": round(elapsed, 2)}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested); "
              "the expert-parallel multi-GPU path is not part of this library", file=sys.stderr)
        sys.exit(2)
    if args.protocol:
        run_protocol(args)
        return
    if args.sweep:
        run_sweep(args)
        return
    import numpy as np
    import torch

    import mixture_experts_expert_histogram_amd as moe
    from synth import WORKLOADS, device_weights, make_dout, make_hidden, make_routing, to_device

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] workload {wl}", file=sys.stderr, flush=True)
    ids_np, w_np = make_routing(wl, seed=0)
    X_np, dY_np = make_hidden(wl, 0), make_dout(wl, 0)
    X, dY = to_device(X_np, wl, dev), to_device(dY_np, wl, dev)
    ids = torch.from_numpy(ids_np).to(dev)
    w = torch.from_numpy(w_np).to(dev)
    Wgu, Wd = device_weights(wl, dev, seed=0)
    kw = dict(act=wl.act, layout=wl.layout, limit=wl.limit, alpha=wl.alpha)
    gdt = torch.float32 if args.grad_dtype == "fp32" else torch.bfloat16
    desc = moe.make_desc(wl.T, wl.H, wl.I, wl.E, wl.K, wl.dtype, wl.act, wl.layout, wl.limit, wl.alpha,
                         args.grad_dtype)
    fws, bws, sbytes = moe.workspace_size(desc)
    ws_f = moe.empty_workspace(fws, dev)
    ws_b = moe.empty_workspace(bws, dev)
    saved = moe.empty_workspace(sbytes, dev)
    out = torch.empty_like(X)
    grads = (torch.empty_like(X), torch.empty((wl.T, wl.K), dtype=torch.float32, device=dev),
             torch.empty(Wgu.shape, dtype=gdt, device=dev), torch.empty(Wd.shape, dtype=gdt, device=dev))
    torch.cuda.synchronize()
    print("[bench] inputs resident", file=sys.stderr, flush=True)

    def fwd():
        moe.fwd(X, ids, w, Wgu, Wd, save=True, ws=ws_f, out=out, saved=saved, **kw)

    def bwd():
        moe.bwd(X, ids, w, Wgu, Wd, dY, saved=saved, ws=ws_b, grads=grads, grad_dtype=args.grad_dtype, **kw)

    def step():
        fwd()
        bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if moe.check_device_status(ws_f) != 0:
        raise RuntimeError("bad expert id reported by the device")

    # separate fwd / bwd timings (context)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    fwd_ms, bwd_ms = [], []
    for _ in range(max(3, min(args.steps, 10))):
        ev[0].record(); fwd(); ev[1].record(); bwd(); ev[2].record()
        torch.cuda.synchronize()
        fwd_ms.append(ev[0].elapsed_time(ev[1]))
        bwd_ms.append(ev[1].elapsed_time(ev[2]))

    # timed region: exactly `steps` steps, nothing recorded between the launches
    t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_stop.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_stop) / args.steps
    print(f"[bench] {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)

    # instrumented pass over the same number of steps: HIP events recorded on
    # the launch stream around every kernel give each kernel's average launch
    # time (for `roofline` and `kernels_avg_ms`)
    kernels = {}
    if not args.no_kernel_timing:
        moe.timing_enable(64 * args.steps)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        kernels = {k: (n, ms) for k, (n, ms) in moe.timing_read().items()}
        moe.timing_disable()

    S, H, I = wl.S, wl.H, wl.I
    flops_fwd, flops_bwd = 6.0 * S * H * I, 12.0 * S * H * I
    value = (flops_fwd + flops_bwd) / (ms_per_step * 1e-3) / 1e12
    counts = np.bincount(ids_np.ravel(), minlength=wl.E)
    model = kernel_model(wl, counts, 4 if args.grad_dtype == "fp32" else 2)
    roof = None
    kern_avg = {}
    if kernels:
        kern_avg = {k: round(ms / n, 4) for k, (n, ms) in kernels.items()}
        dominant = max((k for k in kernels if k in model), key=lambda k: kernels[k][1])
        roof = roofline_for(dominant, kernels[dominant][1] / kernels[dominant][0], model)
        roof["traffic"] = measured_traffic(dominant, wl.name, args.grad_dtype)

    # The same steps with fp32 weight-gradient storage (context for the dtype reading).
    alt = None
    if args.grad_dtype == "bf16" and not args.no_alt_grad_dtype:
        d32 = moe.make_desc(wl.T, wl.H, wl.I, wl.E, wl.K, wl.dtype, wl.act, wl.layout, wl.limit, wl.alpha, "fp32")
        ws_b32 = moe.empty_workspace(moe.workspace_size(d32)[1], dev)
        grads32 = (grads[0], grads[1], torch.empty(Wgu.shape, dtype=torch.float32, device=dev),
                   torch.empty(Wd.shape, dtype=torch.float32, device=dev))

        def step32():
            fwd()
            moe.bwd(X, ids, w, Wgu, Wd, dY, saved=saved, ws=ws_b32, grads=grads32, grad_dtype="fp32", **kw)

        for _ in range(args.warmup):
            step32()
        torch.cuda.synchronize()
        t_start.record()
        for _ in range(args.steps):
            step32()
        t_stop.record()
        torch.cuda.synchronize()
        ms32 = t_start.elapsed_time(t_stop) / args.steps
        alt = {"grad_dtype": "fp32", "ms_per_step": round(ms32, 4),
               "value": round((flops_fwd + flops_bwd) / (ms32 * 1e-3) / 1e12, 2), "unit": "TFLOP/s"}
        del grads32, ws_b32
        print(f"[bench] fp32 weight grads: {ms32:.3f} ms/step", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, ids_np, w_np, X_np, dY_np, Wgu, Wd, args.cpu_seconds)

    fm, bm = float(np.median(fwd_ms)), float(np.median(bwd_ms))
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "fp32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: routed MoE layer forward+backward, T={wl.T} H={wl.H} I={wl.I} "
                               f"E={wl.E} top-{wl.K}, {wl.act} GLU, gate/up {wl.layout}, "
                               f"{wl.routing} routing"
                               + (f" (s={wl.zipf_s})" if wl.routing == "zipf" else "")
                               + f", {args.grad_dtype} weight grads (fp32 accumulation), saved Z",
                   "T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E, "K": wl.K, "parallelism": "single GPU"},
        "fwd_ms": round(fm, 4),
        "bwd_ms": round(bm, 4),
        "fwd_tflops": round(flops_fwd / (fm * 1e-3) / 1e12, 2),
        "bwd_tflops": round(flops_bwd / (bm * 1e-3) / 1e12, 2),
        "pct_of_bf16_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roof,
        "kernels_avg_ms": kern_avg,
        "fp32_weight_grads": alt,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
