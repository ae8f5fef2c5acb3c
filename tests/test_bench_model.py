"""The benchmark's roofline model of one launch per kernel (host logic, CPU).

With bf16 operands the weight gradients run as the resident-operand kernel
for experts of at most RES_KMAX positions (and empty experts) and the
large-tile kernel for the rest where that engine applies (H and I multiples
of 32), else as three kernels: the resident one, the long-K one for experts
of more than LONG_MIN and the tiled one for the rest, whether the gradients
are stored in bf16 or fp32.  The model entries must split the useful flops
and the gradient bytes by expert exactly; with fp32 operands a single entry
covers every expert.
"""
import numpy as np
import pytest

import bench
from synth import WORKLOADS, Workload


@pytest.mark.parametrize("grad_bytes", [2, 4])
@pytest.mark.parametrize("I,large", [(2880, True), (2872, False)])
def test_weight_gradient_split_covers_every_expert(grad_bytes, I, large):
    E = 128
    counts = np.zeros(E, dtype=np.int64)
    rng = np.random.default_rng(0)
    counts[:100] = rng.integers(1, bench.RES_KMAX + 1, size=100)
    counts[100:120] = rng.integers(bench.RES_KMAX + 1, 4000, size=20)
    counts[120] = bench.RES_KMAX            # at the limit: resident
    counts[121] = bench.RES_KMAX + 1        # just above: tiled (large-tile where it applies)
    counts[122] = bench.LONG_MIN            # at the limit: tiled (large-tile)
    counts[123] = bench.LONG_MIN + 1        # just above: long-K (large-tile)
    # experts 124.. are empty; one slot per token so that S = T = counts.sum()
    wl = Workload("model", int(counts.sum()), 2880, I, E, 1, "bf16", "clamped", "interleaved")
    assert bench.large_wgrad(wl) == large
    m = bench.kernel_model(wl, counts, grad_bytes)
    H, S = wl.H, wl.S
    for name, per_flop in [("wgrad_down", 2.0), ("wgrad_gate_up", 4.0)]:
        parts = [m[name]] + [m[name + suf] for suf in ("_hot", "_long") if name + suf in m]
        assert len(parts) == (2 if large else 3)
        assert sum(p[1] for p in parts) == pytest.approx(per_flop * S * H * I)
        small = counts <= bench.RES_KMAX
        long_ = counts > (bench.RES_KMAX if large else bench.LONG_MIN)
        assert m[name][1] == pytest.approx(per_flop * counts[small].sum() * H * I)
        if not large:
            assert m[name + "_hot"][1] == pytest.approx(per_flop * counts[~small & ~long_].sum() * H * I)
        assert m[name + "_long"][1] == pytest.approx(per_flop * counts[long_].sum() * H * I)
        # every expert's gradient is written once, by exactly one of the kernels,
        # and the hidden / output-gradient rows are read once in total; the
        # per-slot intermediates (dZ, w*a) are not algorithmic bytes
        dw = (2 if name == "wgrad_gate_up" else 1) * E * H * I * grad_bytes
        assert sum(p[0] for p in parts) - dw == pytest.approx(wl.T * H * 2)


def test_projection_bytes_are_weights_and_layer_inputs():
    """The projections and their input gradients are charged the weights of
    the experts with slots plus the layer's own input rows, nothing else."""
    wl = WORKLOADS["gptoss"]
    counts = np.zeros(wl.E, dtype=np.int64)
    counts[:3] = [wl.S - 2, 1, 1]
    m = bench.kernel_model(wl, counts, 2)
    H, I, T = wl.H, wl.I, wl.T

    def both(name):   # the hot expert runs on the 256-row tiles, the other two on the small ones
        return m[name][0] + m[name + "_big"][0]
    assert both("gate_up_glu") == pytest.approx(3 * 2 * I * H * 2 + T * H * 2)
    assert both("down_weighted") == 3 * H * I * 2
    assert both("down_dgrad_glu_bwd") == pytest.approx(3 * H * I * 2 + T * H * 2)
    assert both("gate_up_dgrad") == 3 * 2 * I * H * 2
    assert bench.roofline_for("gate_up_glu_big", 1.0, m)["bound"] == "mfma"   # 1 expert's weights, 16382 slots
    spread = bench.kernel_model(wl, np.full(wl.E, wl.S // wl.E, dtype=np.int64), 2)
    rf = bench.roofline_for("gate_up_glu", 1.0, spread)
    assert rf["bound"] == "hbm"            # every expert's weights for ~128 slots each: weight-stream bound
    assert rf["achieved"] == pytest.approx((wl.E * 2 * I * H * 2 + T * H * 2) / 1e-3 / 1e9, rel=1e-3)
    zipf = WORKLOADS["zipf"]
    zc = np.full(zipf.E, zipf.S // zipf.E, dtype=np.int64)
    mz = bench.kernel_model(zipf, zc, 2)
    rz = bench.roofline_for("gate_up_glu_big", 2.0, mz)   # 1024 slots per expert: the 256-row tiles
    assert rz["bound"] == "mfma" and rz["achieved"] == pytest.approx(4.0 * zipf.S * H * I / 2e-3 / 1e12, rel=1e-3)


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


def test_token_row_split_by_tile_engine():
    """With bf16 operands and H, I multiples of 32, the large-tile experts
    (LARGE_MIN slots and more, and smaller ones whose 256-row tiles hold no
    more rows than 128-row tiles would) are charged to the 256-row kernels
    (*_big), the rest to the small-tile ones; flops and weights split by
    expert exactly and the layer's input rows are charged once in total."""
    wl = WORKLOADS["zipf"]
    rng = np.random.default_rng(3)
    counts = rng.integers(0, 2 * bench.LARGE_MIN, size=wl.E).astype(np.int64)
    counts[0] = bench.LARGE_MIN          # at the limit: large tiles
    counts[1] = 300                      # 512 rows of 256-row tiles against 384 of 128-row ones: small tiles
    counts[2] = 0
    counts[3] = 200                      # one 256-row tile against two 128-row ones: large tiles
    counts[-1] += wl.S - counts.sum()    # make the slots add up to S
    assert counts[-1] >= 0
    m = bench.kernel_model(wl, counts, 2)
    H, I, T, S = wl.H, wl.I, wl.T, wl.S
    big = bench.large_tile_experts(wl, counts)
    assert big[0] and not big[1] and not big[2] and big[3]
    for name, per_flop, w_rows, x_rows in [("gate_up_glu", 4.0, 2 * I * H, True), ("down_weighted", 2.0, H * I, False),
                                           ("down_dgrad_glu_bwd", 2.0, H * I, True), ("gate_up_dgrad", 4.0, 2 * I * H, False)]:
        assert m[name + "_big"][1] == pytest.approx(per_flop * counts[big].sum() * H * I)
        assert m[name][1] + m[name + "_big"][1] == pytest.approx(per_flop * S * H * I)
        touched = int((counts > 0).sum())
        total = m[name][0] + m[name + "_big"][0]
        assert total == pytest.approx(touched * w_rows * 2 + (T * H * 2 if x_rows else 0))
    # H not a multiple of 32: one entry per product
    odd = Workload("odd", 4096, 264, 200, 8, 1, "bf16", "swiglu", "concat")
    m2 = bench.kernel_model(odd, np.array([4000, 96, 0, 0, 0, 0, 0, 0]), 2)
    assert "gate_up_glu_big" not in m2 and m2["gate_up_glu"][1] == pytest.approx(4.0 * 4096 * 264 * 200)


@pytest.mark.parametrize("bms", [128, 192])
def test_large_tile_rule_rows(bms):
    """The rule takes an expert to the 256-row tiles exactly when its rows
    padded to 256 do not exceed its rows padded to the small tile (brute
    force over 1..600 slots)."""
    mean = 150 if bms == 192 else 400
    # 192-row tiles only where the 128-row DMA tiles do not apply (I % 64 != 0)
    wl = Workload("rule", mean * 8, 2880, 2880 if bms == 128 else 2848, 8, 1, "bf16", "swiglu", "concat")
    c = np.arange(0, 601)
    got = bench.large_tile_experts(wl, c)
    for n in range(0, 601):
        want = n >= bench.LARGE_MIN or (n > 0 and -(-n // 256) * 256 <= -(-n // bms) * bms)
        assert got[n] == want, n
    if bms == 128:
        assert got[129] and got[256] and not got[257] and not got[384] and got[385] and not got[128]
    else:
        assert not got[192] and got[193] and got[256] and not got[257] and got[385]
