"""GPU parity of the large-tile engine (experts with at least 512 slots, bf16,
H and I multiples of 32) against the fp64 oracle.

Experts of 1300, 600, 513 and 512 slots take the 256 x 256-tile kernels
(ragged last M-tiles), those of 511, 100 and 0 slots the 128-row kernels, in
the same call.  H = 288 and I = 160 leave ragged N-tiles in every product
(gate_up: 160 of 256 activation columns in the second tile; down: 32 of 256
hidden columns; the input gradients: 160 and 32 of 256).  Z is saved or
recomputed (the Z-only gate_up kernel); gate and up weights are fused in
either layout or separate tensors.

The weight gradients of experts above 512 slots take the large-tile kernel
too: k (the expert's slots) is ragged, so its last 32-slot step reads the
expert's last slot again and zeroes those rows of the dZ / dY tile.
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_histogram_amd as moe
from tests._gpu import assert_parity, device_inputs, host, oracle_fwd_bwd, small_inputs
from tests.test_gpu_parity import check_weight_grads, gate_up_halves, run_and_compare
from tests.test_gpu_separate import check_separate

pytestmark = pytest.mark.gpu

COUNTS = [1300, 600, 513, 512, 511, 100, 0]
H, I = 288, 160


def large_tile_inputs(act, layout, seed):
    E, K = len(COUNTS), 1
    T = sum(COUNTS)
    rng = np.random.default_rng(seed)
    ids = rng.permutation(np.repeat(np.arange(E), COUNTS)).reshape(T, K).astype(np.int32)
    return small_inputs(T, H, I, E, K, "bf16", act, layout, seed=seed, ids=ids)


@pytest.mark.parametrize("act,layout", [("clamped", "interleaved"), ("swiglu", "concat")])
@pytest.mark.parametrize("save", [True, False])
def test_large_tile_experts_match_oracle(act, layout, save):
    run_and_compare(large_tile_inputs(act, layout, 51), save=save, grad_dtype="bf16", poison=True)


# The GLU epilogues are compiled per activation kind and gate / up layout:
# every combination runs through both tile sizes of the large-tile engine.
ALL_GLU = [("clamped", "interleaved"), ("swiglu", "concat"), ("clamped", "concat"), ("swiglu", "interleaved")]


@pytest.mark.parametrize("act,layout", ALL_GLU)
def test_large_tile_experts_64k_stages(act, layout):
    """H = 320 and I = 192 (multiples of 64): the token-row kernels take
    stages of 64 k (gate_up 5 stages, an odd count for the two-stage ring;
    down 3).  N stays ragged: gate_up 384 dZ columns (128 of 256 in the
    second tile), down 320 (64), the input gradients 320 and 192."""
    E, K = len(COUNTS), 1
    T = sum(COUNTS)
    rng = np.random.default_rng(59)
    ids = rng.permutation(np.repeat(np.arange(E), COUNTS)).reshape(T, K).astype(np.int32)
    inp = small_inputs(T, 320, 192, E, K, "bf16", act, layout, seed=59, ids=ids)
    run_and_compare(inp, save=act == "clamped", grad_dtype="bf16", poison=True)


@pytest.mark.parametrize("act,layout", ALL_GLU)
@pytest.mark.parametrize("save", [True, False])
def test_small_experts_64k_stages(act, layout, save):
    """H = 320 and I = 192 with the batch averaging 293 slots per expert: the
    experts of 1-300 slots (all but the 1300-slot one) take the same engine's
    128 x 256 tiles (three 64-k stages; 300 slots: two full tiles and one of
    44 rows), N ragged in every product as above."""
    counts = [1300, 300, 260, 257, 128, 100, 1, 0]
    E, K = len(counts), 1
    T = sum(counts)
    assert T // E > 176
    rng = np.random.default_rng(73)
    ids = rng.permutation(np.repeat(np.arange(E), counts)).reshape(T, K).astype(np.int32)
    inp = small_inputs(T, 320, 192, E, K, "bf16", act, layout, seed=73, ids=ids)
    run_and_compare(inp, save=save, grad_dtype="bf16", poison=True)


@pytest.mark.parametrize("layout", ["interleaved", "concat"])
def test_large_tile_separate_weights(layout):
    check_separate(large_tile_inputs("swiglu", layout, 53), "swiglu", layout, "bf16", "fp32", True)


def test_large_tile_two_slots_per_token():
    """K = 2: the same token rows gathered into two experts' large tiles."""
    E, K = 5, 2
    counts = np.array([1100, 700, 120, 60, 20])
    T = int(counts.sum()) // K
    rng = np.random.default_rng(57)
    flat = rng.permutation(np.repeat(np.arange(E), counts))
    ids = flat.reshape(T, K).astype(np.int32)
    inp = small_inputs(T, H, I, E, K, "bf16", "clamped", "interleaved", seed=57, ids=ids)
    run_and_compare(inp, save=True, grad_dtype="bf16")


# remainders of the 32-slot step: 2080 -> 0, 1055 -> 31, 777 -> 9, 544 -> 0,
# 513 -> 1, 600 -> 24; 40 and 0 stay on the other kernels
WG_COUNTS = [2080, 1055, 777, 544, 513, 600, 40, 0]


def weight_grad_inputs(layout, seed, H=544, I=1056):
    E, K = len(WG_COUNTS), 1
    T = sum(WG_COUNTS)
    rng = np.random.default_rng(seed)
    ids = rng.permutation(np.repeat(np.arange(E), WG_COUNTS)).reshape(T, K).astype(np.int32)
    return small_inputs(T, H, I, E, K, "bf16", "swiglu", layout, seed=seed, ids=ids)


@pytest.mark.parametrize("grad_dtype", ["bf16", "fp32"])
def test_large_tile_weight_grads(grad_dtype):
    """dW_gate_up [2I = 2112, H = 544]: 9 M-tiles of 256 (two groups of 8,
    the last 64 rows wide) by 3 N-tiles (the last 32 wide); dW_down
    [H = 544, I = 1056]: 3 by 5 (the last 32 wide)."""
    run_and_compare(weight_grad_inputs("interleaved", 61), save=True, grad_dtype=grad_dtype, poison=True)


@pytest.mark.parametrize("grad_dtype", ["bf16", "fp32"])
def test_large_tile_weight_grads_short_k(grad_dtype):
    """Experts of 241, 300, 464, 465 and 700 positions (the large-tile
    weight gradient: 8 to 22 steps of 32, ragged last steps of 1 to 28) and
    240 (the resident-operand kernel) at H = 544, I = 1056."""
    counts = [700, 465, 464, 300, 241, 240]
    E, K = len(counts), 1
    T = sum(counts)
    rng = np.random.default_rng(67)
    ids = rng.permutation(np.repeat(np.arange(E), counts)).reshape(T, K).astype(np.int32)
    inp = small_inputs(T, 544, 1056, E, K, "bf16", "swiglu", "interleaved", seed=67, ids=ids)
    run_and_compare(inp, save=True, grad_dtype=grad_dtype, poison=True)


@pytest.mark.parametrize("layout", ["interleaved", "concat"])
def test_large_tile_weight_grads_separate(layout):
    """Separate gate and up gradient tensors: a 256-row tile of dZ columns
    maps to rows of both tensors (interleaved) or straddles the boundary
    between them at I = 1056 (concatenated)."""
    check_separate(weight_grad_inputs(layout, 63), "swiglu", layout, "bf16", "bf16", True)


@pytest.mark.parametrize("act,layout", [("clamped", "interleaved"), ("swiglu", "concat")])
@pytest.mark.parametrize("save", [True, False])
def test_small_experts_with_large_tile_shapes(act, layout, save):
    """Experts below 512 slots with H and I multiples of 32 (the large-tile
    engine enabled but finding no expert of its own): 192-row tiles when the
    batch averages 101-176 slots per expert (here 116), 128 x 256 tiles above
    that (the large-tile tests above, mean 505).  N is ragged in every
    product (gate_up 320 dZ columns, down 288, gate_up dgrad 288, down dgrad
    160); experts of 1-290 slots span one or two M-tiles."""
    counts = [290, 193, 192, 150, 60, 1, 10]
    E, K = len(counts), 1
    T = sum(counts)
    assert 101 <= T // E <= 176
    rng = np.random.default_rng(71)
    ids = rng.permutation(np.repeat(np.arange(E), counts)).reshape(T, K).astype(np.int32)
    inp = small_inputs(T, H, I, E, K, "bf16", act, layout, seed=71, ids=ids)
    run_and_compare(inp, save=save, grad_dtype="bf16", poison=True)
