"""The synthetic workloads carry the pages' shapes; the generator is sane."""
import os

import numpy as np
import pytest

from synth import (WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, make_routing,
                   routing_softmax_topk, routing_zipf)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_workloads.txt")


def page_params():
    rows = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        title, name, val = [x.strip() for x in line.split("|")]
        rows.setdefault(title, {})[name] = int(val)
    return rows


def test_workload_shapes_follow_the_pages():
    p = page_params()
    p1 = p["Sparse expert dispatch and combine"]
    p2 = p["MoE training token repeat and expert computation"]
    p3 = p["MoE expert parallel execution backward"]
    assert p1["intermediate_size_x2"] == 2 * p1["intermediate_size"]
    for name in ["gptoss", "zipf"]:
        wl = WORKLOADS[name]
        assert (wl.H, wl.I, wl.E, wl.K) == (p1["hidden_size"], p1["intermediate_size"],
                                            p1["num_local_experts"], p1["num_experts_per_tok"])
        assert wl.act == "clamped"
    wl = WORKLOADS["large"]
    assert (wl.H, wl.I, wl.E, wl.K) == (p2["hidden_size"], p2["moe_intermediate_size"],
                                        p2["num_experts"], p2["num_experts_per_tok"])
    wl = WORKLOADS["backward"]
    assert (wl.H, wl.I, wl.E, wl.K) == (p3["hidden_size"], p3["moe_intermediate_size"],
                                        p3["n_routed_experts"], p3["num_experts_per_tok"])


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20, -2.5, 0.0], dtype=np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(x))
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6); above the tie rounds up
    np.testing.assert_array_equal(got, np.array([1.0, 1.0, 1.0 + 2**-6, 1.0 + 2**-7, -2.5, 0.0], dtype=np.float32))
    y = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    r = bf16_bits_to_f32(f32_to_bf16_bits(y))
    assert np.max(np.abs(r - y) / np.abs(y)) <= 2**-8   # unit roundoff of an 8-bit significand


def test_softmax_topk_routing():
    ids, w = routing_softmax_topk(100, 16, 4, seed=0)
    assert ids.shape == (100, 4) and ids.dtype == np.int32
    assert all(len(set(r)) == 4 for r in ids.tolist())
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)        # descending logits -> descending weights
    ids2, w2 = routing_softmax_topk(100, 16, 4, seed=0)
    np.testing.assert_array_equal(ids, ids2)


def test_zipf_routing_is_skewed_and_distinct():
    ids, w = routing_zipf(4096, 128, 4, 1.2, seed=0)
    assert all(len(set(r)) == 4 for r in ids[:500].tolist())
    c = np.bincount(ids.ravel(), minlength=128)
    assert c.max() > 20 * np.median(c)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)


@pytest.mark.parametrize("name", ["tiny", "gptoss"])
def test_make_routing(name):
    wl = WORKLOADS[name]
    ids, w = make_routing(wl.with_(T=min(wl.T, 256)))
    assert ids.max() < wl.E and ids.min() >= 0


def test_softmax_topk_routing_needs_k_experts():
    from synth import routing_softmax_topk
    with pytest.raises(ValueError):
        routing_softmax_topk(4, 2, 3)
