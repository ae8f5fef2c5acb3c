"""Seeded synthetic inputs for the routed MoE expert computation.

This module is shared by the tests, the benchmark and the smoke check.  It
draws the inputs of a routed MoE layer (hidden states, top-k expert ids and
weights, expert weights, output gradient) and converts fp32 draws to bf16
bit patterns.  It holds none of the MoE layer's arithmetic: the gathers,
projections, gated activations, weighting and sums live only in the oracle
(``oracle/``) and in the HIP library, which never import each other.

Workloads (shape names from the three kernelindex operation pages, workload
lines: "Sparse expert dispatch and combine", "MoE training token repeat and
expert computation", "MoE expert parallel execution backward"):

* ``tiny``     T=64,    H=128,  I=128,  E=8,   k=2, fp32, SwiGLU, gate|up concatenated
* ``gptoss``   T=4096,  H=2880, I=2880, E=128, k=4, bf16, clamped GLU, gate/up interleaved
* ``large``    T=4096,  H=8192, I=2048, E=256, k=8, bf16, SwiGLU, concatenated
* ``backward`` T=8192,  H=4096, I=2048, E=256, k=8, bf16, SwiGLU, concatenated
* ``zipf``     T=32768, H=2880, I=2880, E=128, k=4, bf16, clamped GLU, interleaved,
               expert popularity Zipf(s=1.2)

Recipe (every stream derives from ``numpy.random.SeedSequence(seed)``):

* router logits N(0,1) fp32 [T,E]; the k largest per token by a stable
  descending sort (ties go to the lower expert id); weights are the softmax
  of the chosen k logits, computed in fp64 and stored fp32 (this equals a
  full softmax renormalised over the top k).
* Zipf routing: expert popularity p_r ~ r^-s over ranks r=1..E, ranks mapped
  to ids by a seeded permutation; each token draws k distinct experts by
  Gumbel-top-k on log p; weights are the softmax of fresh N(0,1) logits over
  the chosen experts.
* hidden N(0,1), output gradient N(0,1), expert weights N(0,0.02); fp32 draws
  rounded to bf16 with round-to-nearest-even where the workload is bf16.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

ACT_SWIGLU = "swiglu"
ACT_CLAMPED = "clamped"
LAYOUT_CONCAT = "concat"
LAYOUT_INTERLEAVED = "interleaved"

CLAMP_LIMIT = 7.0
GLU_ALPHA = 1.702
WEIGHT_STD = 0.02


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int
    K: int
    dtype: str          # "fp32" or "bf16"
    act: str            # ACT_SWIGLU or ACT_CLAMPED
    layout: str         # LAYOUT_CONCAT or LAYOUT_INTERLEAVED
    routing: str = "softmax_topk"   # or "zipf"
    zipf_s: float = 1.2
    limit: float = CLAMP_LIMIT
    alpha: float = GLU_ALPHA

    @property
    def S(self) -> int:
        return self.T * self.K

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 64, 128, 128, 8, 2, "fp32", ACT_SWIGLU, LAYOUT_CONCAT),
    "gptoss": Workload("gptoss", 4096, 2880, 2880, 128, 4, "bf16", ACT_CLAMPED, LAYOUT_INTERLEAVED),
    "large": Workload("large", 4096, 8192, 2048, 256, 8, "bf16", ACT_SWIGLU, LAYOUT_CONCAT),
    "backward": Workload("backward", 8192, 4096, 2048, 256, 8, "bf16", ACT_SWIGLU, LAYOUT_CONCAT),
    "zipf": Workload("zipf", 32768, 2880, 2880, 128, 4, "bf16", ACT_CLAMPED, LAYOUT_INTERLEAVED,
                     routing="zipf"),
}

# stream ids inside SeedSequence(seed): one child per tensor kind
_S_LOGITS, _S_HIDDEN, _S_DOUT, _S_WGU, _S_WD, _S_ZIPF = range(6)


def _child(seed: int, stream: int, sub: Optional[int] = None) -> np.random.Generator:
    key = [int(seed), int(stream)] if sub is None else [int(seed), int(stream), int(sub)]
    return np.random.default_rng(np.random.SeedSequence(key))


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(x)
    out = r.astype(np.uint16)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32, exact."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values as the workload stores them (returned as fp32 numbers)."""
    x = np.asarray(x, dtype=np.float32)
    return bf16_bits_to_f32(f32_to_bf16_bits(x)) if dtype == "bf16" else x


# ---------------------------------------------------------------- routing
def router_logits(T: int, E: int, seed: int = 0) -> np.ndarray:
    """The N(0,1) router logits [T,E] (fp32) behind routing_softmax_topk."""
    return _child(seed, _S_LOGITS).standard_normal((T, E), dtype=np.float32)


def routing_softmax_topk(T: int, E: int, K: int, seed: int = 0):
    """Top-k ids and renormalised softmax weights from N(0,1) router logits."""
    if K > E:
        raise ValueError(f"top-{K} routing needs at least {K} experts (E = {E})")
    logits = router_logits(T, E, seed)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :K]
    chosen = np.take_along_axis(logits, order, axis=1).astype(np.float64)
    z = np.exp(chosen - chosen.max(axis=1, keepdims=True))
    w = z / z.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def routing_zipf(T: int, E: int, K: int, s: float = 1.2, seed: int = 0):
    """k distinct experts per token drawn from a Zipf(s) popularity."""
    rng = _child(seed, _S_ZIPF)
    ranks = np.arange(1, E + 1, dtype=np.float64)
    logp = -s * np.log(ranks)
    perm = rng.permutation(E)             # rank r -> expert id perm[r]
    logp_by_id = np.empty(E)
    logp_by_id[perm] = logp
    ids = np.empty((T, K), dtype=np.int32)
    chunk = 8192
    for t0 in range(0, T, chunk):
        n = min(chunk, T - t0)
        g = rng.gumbel(size=(n, E)) + logp_by_id[None, :]
        ids[t0:t0 + n] = np.argsort(-g, axis=1, kind="stable")[:, :K]
    logits = _child(seed, _S_LOGITS).standard_normal((T, K), dtype=np.float32).astype(np.float64)
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


def make_routing(wl: Workload, seed: int = 0):
    if wl.routing == "zipf":
        return routing_zipf(wl.T, wl.E, wl.K, wl.zipf_s, seed)
    return routing_softmax_topk(wl.T, wl.E, wl.K, seed)


# ---------------------------------------------------------------- tensors
def make_hidden(wl: Workload, seed: int = 0) -> np.ndarray:
    """hidden [T,H], N(0,1), rounded to the workload dtype (fp32 array)."""
    x = _child(seed, _S_HIDDEN).standard_normal((wl.T, wl.H), dtype=np.float32)
    return round_to_dtype(x, wl.dtype)


def make_dout(wl: Workload, seed: int = 0) -> np.ndarray:
    """output gradient [T,H], N(0,1), rounded to the workload dtype."""
    x = _child(seed, _S_DOUT).standard_normal((wl.T, wl.H), dtype=np.float32)
    return round_to_dtype(x, wl.dtype)


def make_expert_weights(wl: Workload, e: int, seed: int = 0):
    """(w_gate_up[e] [2I,H], w_down[e] [H,I]) of one expert, N(0,0.02), host."""
    gu = _child(seed, _S_WGU, e).standard_normal((2 * wl.I, wl.H), dtype=np.float32) * np.float32(WEIGHT_STD)
    dn = _child(seed, _S_WD, e).standard_normal((wl.H, wl.I), dtype=np.float32) * np.float32(WEIGHT_STD)
    return round_to_dtype(gu, wl.dtype), round_to_dtype(dn, wl.dtype)


def make_all_weights(wl: Workload, seed: int = 0):
    """Every expert's weights on the host: [E,2I,H] and [E,H,I] (small workloads)."""
    gu = np.empty((wl.E, 2 * wl.I, wl.H), dtype=np.float32)
    dn = np.empty((wl.E, wl.H, wl.I), dtype=np.float32)
    for e in range(wl.E):
        gu[e], dn[e] = make_expert_weights(wl, e, seed)
    return gu, dn


@dataclasses.dataclass
class HostInputs:
    wl: Workload
    hidden: np.ndarray        # fp32 [T,H] (values representable in wl.dtype)
    topk_ids: np.ndarray      # int32 [T,K]
    topk_weights: np.ndarray  # fp32 [T,K]
    dout: np.ndarray          # fp32 [T,H]
    w_gate_up: np.ndarray     # fp32 [E,2I,H]
    w_down: np.ndarray        # fp32 [E,H,I]


def make_host_inputs(wl: Workload, seed: int = 0) -> HostInputs:
    """All inputs on the host (for workloads whose weights fit comfortably)."""
    ids, w = make_routing(wl, seed)
    gu, dn = make_all_weights(wl, seed)
    return HostInputs(wl, make_hidden(wl, seed), ids, w, make_dout(wl, seed), gu, dn)


# ---------------------------------------------------------------- device
def torch_dtype(wl: Workload):
    import torch
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def device_weights(wl: Workload, device, seed: int = 0):
    """Expert weights drawn directly in device memory (the large workloads).

    Expert e's gate_up and down blocks come from torch generators seeded with
    (seed, kind, e), N(0,0.02) in fp32 then rounded (RNE) to the workload dtype.
    They differ from make_expert_weights' host draws; an oracle that checks a
    device run reads the experts it needs back from device memory.
    """
    import torch
    dt = torch_dtype(wl)
    gu = torch.empty((wl.E, 2 * wl.I, wl.H), dtype=dt, device=device)
    dn = torch.empty((wl.E, wl.H, wl.I), dtype=dt, device=device)
    g = torch.Generator(device=device)
    for e in range(wl.E):
        g.manual_seed(((seed * 1000003 + 1) * 4099 + e) & 0x7FFFFFFFFFFF)
        tmp = torch.randn((2 * wl.I, wl.H), generator=g, device=device, dtype=torch.float32)
        gu[e].copy_(tmp.mul_(WEIGHT_STD))
        g.manual_seed(((seed * 1000003 + 2) * 4099 + e) & 0x7FFFFFFFFFFF)
        tmp = torch.randn((wl.H, wl.I), generator=g, device=device, dtype=torch.float32)
        dn[e].copy_(tmp.mul_(WEIGHT_STD))
    del tmp
    return gu, dn


def to_device(x: np.ndarray, wl: Workload, device):
    """Host fp32 array -> device tensor of the workload dtype (exact for rounded values)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device).to(torch_dtype(wl))
