"""GPU parity of the large-tile engine (experts with at least 512 slots, bf16,
H and I multiples of 32) against the fp64 oracle.

Experts of 1300, 600, 513 and 512 slots take the 256 x 256-tile kernels
(ragged last M-tiles), those of 511, 100 and 0 slots the 128-row kernels, in
the same call.  H = 288 and I = 160 leave ragged N-tiles in every product
(gate_up: 160 of 256 activation columns in the second tile; down: 32 of 256
hidden columns; the input gradients: 160 and 32 of 256).  Z is saved or
recomputed (the Z-only gate_up kernel); gate and up weights are fused in
either layout or separate tensors.
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
