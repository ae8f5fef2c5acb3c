"""The benchmark's roofline model of one launch per kernel (host logic, CPU).

With bf16 operands the weight gradients run as three kernels: the
resident-operand one for experts of at most RES_KMAX positions (and empty
experts), the long-K one for experts of more than LONG_MIN and the tiled one
for the rest, whether the gradients are stored in bf16 or fp32.  The model
entries must split the useful flops and the gradient bytes by expert
exactly; with fp32 operands a single entry covers every expert.
"""
import numpy as np
import pytest

import bench
from synth import WORKLOADS, Workload


@pytest.mark.parametrize("grad_bytes", [2, 4])
def test_weight_gradient_split_covers_every_expert(grad_bytes):
    E = 128
    counts = np.zeros(E, dtype=np.int64)
    rng = np.random.default_rng(0)
    counts[:100] = rng.integers(1, bench.RES_KMAX + 1, size=100)
    counts[100:120] = rng.integers(bench.RES_KMAX + 1, 4000, size=20)
    counts[120] = bench.RES_KMAX            # at the limit: resident
    counts[121] = bench.RES_KMAX + 1        # just above: tiled
    counts[122] = bench.LONG_MIN            # at the limit: tiled
    counts[123] = bench.LONG_MIN + 1        # just above: long-K
    # experts 124.. are empty; one slot per token so that S = T = counts.sum()
    wl = Workload("model", int(counts.sum()), 2880, 2880, E, 1, "bf16", "clamped", "interleaved")
    m = bench.kernel_model(wl, counts, grad_bytes)
    H, I, S = wl.H, wl.I, wl.S
    for name, per_flop in [("wgrad_down", 2.0), ("wgrad_gate_up", 4.0)]:
        parts = [m[name]] + [m[name + suf] for suf in ("_hot", "_long") if name + suf in m]
        assert len(parts) == 3
        assert sum(p[1] for p in parts) == pytest.approx(per_flop * S * H * I)
        small, long_ = counts <= bench.RES_KMAX, counts > bench.LONG_MIN
        assert m[name][1] == pytest.approx(per_flop * counts[small].sum() * H * I)
        assert m[name + "_hot"][1] == pytest.approx(per_flop * counts[~small & ~long_].sum() * H * I)
        assert m[name + "_long"][1] == pytest.approx(per_flop * counts[long_].sum() * H * I)
        # every expert's gradient is written once, by exactly one of the kernels,
        # and the operand rows are read once in total
        dw = (2 if name == "wgrad_gate_up" else 1) * E * H * I * grad_bytes
        act = S * (2 * I if name == "wgrad_gate_up" else I) * 2
        assert sum(p[0] for p in parts) - dw == pytest.approx(wl.T * H * 2 + act)


def test_no_hot_entry_without_hot_experts():
    wl = WORKLOADS["gptoss"]
    counts = np.full(wl.E, wl.S // wl.E, dtype=np.int64)
    m = bench.kernel_model(wl, counts, 2)
    assert "wgrad_gate_up_hot" not in m and "wgrad_down_hot" not in m
    assert "wgrad_gate_up_long" not in m and "wgrad_down_long" not in m


def test_fp32_operands_use_one_entry():
    wl = Workload("model32", 600, 64, 32, 4, 1, "fp32", "swiglu", "concat")
    counts = np.array([300, 250, 50, 0])
    m = bench.kernel_model(wl, counts, 4)
    assert "wgrad_gate_up_hot" not in m and m["wgrad_gate_up"][1] == pytest.approx(4.0 * 600 * 64 * 32)
