"""Plain, slow, fp64 CPU definition of the routed MoE expert computation.

TEST INFRASTRUCTURE: only tests, the smoke check and the benchmark's CPU
baseline use this module.  It shares no code with the HIP path.

Sources (kernelindex.com operation pages):

* "Sparse expert dispatch and combine" — description: experts are processed
  one after another; for each, the tokens routed to it are extracted, pass
  through a gate_up projection, a gated GLU with clamping and a down
  projection, and are scattered back into the output with index_add_.
  Workload line: hidden_size, intermediate_size, num_local_experts,
  num_experts_per_tok, and a fused gate_up width of twice intermediate_size.
* "MoE training token repeat and expert computation" — description: each
  token is repeated num_experts_per_tok times, experts select their rows by
  masked indexing and run a SwiGLU FFN, and the routing weights multiply the
  expert outputs before the sum over experts.
* "MoE expert parallel execution backward" — description: gradients with
  respect to hidden_states, topk_weights, gate, up and down weights through
  the SwiGLU expert MLP, with token dispatch and weighted aggregation.

Notation: T tokens, H hidden, I intermediate, E experts, K experts per token,
S = T*K slots.  Slot s = t*K + k is the k-th copy of token t (the "token
repeat").  Weights are stored [out, in]: w_gate_up [E, 2I, H], w_down [E, H, I].

Readings where the pages are silent (all fixed by the workload definitions
that accompany this library, not by the pages):

* the clamped GLU is gate = min(g, limit), up = clip(u, -limit, limit),
  a = (up + 1) * gate * sigmoid(alpha * gate) with limit 7 and alpha 1.702;
  its derivative passes on the closed intervals g <= limit, |u| <= limit;
* the fused gate_up rows are either concatenated ([gate; up]) or interleaved
  (even rows gate, odd rows up);
* no biases;
* ids repeated inside one token are two independent slots.

Every quantity is fp64; inputs are upcast exactly from their stored dtype.
"""
from __future__ import annotations

from typing import Callable, Optional, Tuple

import numpy as np

F64 = np.float64


# ------------------------------------------------------------------ routing
def route(topk_ids: np.ndarray, E: int):
    """Group the T*K slots by expert.

    "Masked indexing" per expert ("MoE training token repeat and expert
    computation", description) selects, for expert e, the slots whose id is
    e, in slot order.  Written as one stable sort of the flattened ids:

    counts[e]       number of slots routed to e (the expert histogram)
    offsets[e]      exclusive prefix sum of counts (length E+1)
    sorted_slot[p]  slots ordered by expert, ascending slot inside an expert
    inv_pos[s]      position p of slot s in sorted_slot
    """
    f = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    if f.size and (f.min() < 0 or f.max() >= E):
        raise ValueError("expert id outside [0, E)")
    counts = np.bincount(f, minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    sorted_slot = np.argsort(f, kind="stable").astype(np.int64)
    inv_pos = np.empty_like(sorted_slot)
    inv_pos[sorted_slot] = np.arange(f.size, dtype=np.int64)
    return counts, offsets, sorted_slot, inv_pos


# ------------------------------------------------------------------ GLU
def router(logits: np.ndarray, K: int):
    """Top-K expert ids and routing weights from router logits [T, E].

    The pages take topk_ids and topk_weights as given inputs ("MoE expert
    parallel execution backward" differentiates topk_weights).  The routing
    that produces them is the one the workloads are defined with: the softmax
    over a token's E logits, its K largest entries, renormalised to sum to
    one.  Written out in that order, in fp64:

    p = softmax(logits[t])        (max subtracted for range)
    ids[t] = the K largest, by descending logit (softmax is increasing, so
             ranking logits ranks p without p's underflow ties); equal
             logits in ascending expert id
    w[t, k] = p[ids[t, k]] / sum_j p[ids[t, j]]
    """
    lg = np.asarray(logits, dtype=F64)
    T, E = lg.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    z = np.exp(lg - lg.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    ids = np.argsort(-lg, axis=1, kind="stable")[:, :K]
    chosen = np.take_along_axis(p, ids, axis=1)
    return ids.astype(np.int64), chosen / chosen.sum(axis=1, keepdims=True)


def router_backward(topk_ids: np.ndarray, topk_weights: np.ndarray, d_topk_weights: np.ndarray, E: int):
    """dL/dlogits [T, E] given dL/dw [T, K], by the chain rule on router().

    With the choice held fixed (it is piecewise constant in the logits),
    w_k = exp(l_{i_k}) / sum_j exp(l_{i_j}), so dw_k/dl_{i_m} =
    w_k (delta_km - w_m) and dL/dl_{i_m} = w_m (g_m - sum_k w_k g_k); logits
    not chosen get zero.  A repeated id adds its terms.
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    w = np.asarray(topk_weights, dtype=F64)
    g = np.asarray(d_topk_weights, dtype=F64)
    T, K = ids.shape
    d = np.zeros((T, E), dtype=F64)
    dot = np.sum(w * g, axis=1)
    for t in range(T):
        for k in range(K):
            if 0 <= ids[t, k] < E:
                d[t, ids[t, k]] += w[t, k] * (g[t, k] - dot[t])
    return d


def split_gate_up(Z: np.ndarray, layout: str):
    """Split gate_up projection outputs [c, 2I] into gate and up [c, I]."""
    I = Z.shape[1] // 2
    if layout == "concat":
        return Z[:, :I], Z[:, I:]
    if layout == "interleaved":
        return Z[:, 0::2], Z[:, 1::2]
    raise ValueError(layout)


def merge_gate_up(g: np.ndarray, u: np.ndarray, layout: str) -> np.ndarray:
    """Inverse of split_gate_up."""
    c, I = g.shape
    Z = np.empty((c, 2 * I), dtype=F64)
    if layout == "concat":
        Z[:, :I], Z[:, I:] = g, u
    elif layout == "interleaved":
        Z[:, 0::2], Z[:, 1::2] = g, u
    else:
        raise ValueError(layout)
    return Z


def _sigmoid(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def glu(g: np.ndarray, u: np.ndarray, act: str, limit: float = 7.0, alpha: float = 1.702):
    """Gated activation a = phi(g, u).

    "swiglu": silu(g) * u = g * sigmoid(g) * u ("MoE training token repeat
    and expert computation", description: SwiGLU FFN).
    "clamped": the "gated GLU with clamping" of "Sparse expert dispatch and
    combine" (description), with the constants stated in the module header.
    """
    g = np.asarray(g, dtype=F64)
    u = np.asarray(u, dtype=F64)
    if act == "swiglu":
        return g * _sigmoid(g) * u
    if act == "clamped":
        gc = np.minimum(g, limit)
        uc = np.clip(u, -limit, limit)
        return (uc + 1.0) * gc * _sigmoid(alpha * gc)
    raise ValueError(act)


def glu_backward(g, u, dA, act: str, limit: float = 7.0, alpha: float = 1.702):
    """(dL/dg, dL/du) given dL/da, by the chain rule on glu()."""
    g = np.asarray(g, dtype=F64)
    u = np.asarray(u, dtype=F64)
    dA = np.asarray(dA, dtype=F64)
    if act == "swiglu":
        sg = _sigmoid(g)
        dsilu = sg * (1.0 + g * (1.0 - sg))          # d/dg [g*sigmoid(g)]
        return dA * u * dsilu, dA * g * sg
    if act == "clamped":
        gc = np.minimum(g, limit)
        uc = np.clip(u, -limit, limit)
        s = _sigmoid(alpha * gc)
        dq = s * (1.0 + alpha * gc * (1.0 - s))     # d/dx [x*sigmoid(alpha*x)]
        pass_g = (g <= limit).astype(F64)
        pass_u = ((u >= -limit) & (u <= limit)).astype(F64)
        return dA * (uc + 1.0) * dq * pass_g, dA * gc * s * pass_u
    raise ValueError(act)


# ------------------------------------------------------------------ weights
ExpertFn = Callable[[int], Tuple[np.ndarray, np.ndarray]]


def expert_accessor(w_gate_up, w_down=None) -> ExpertFn:
    """Normalise expert weights to a function e -> (Wgu[e] [2I,H], Wd[e] [H,I]) in fp64.

    Accepts the two stacked arrays, or a callable that already returns one
    expert's pair (for workloads whose weights are too large to hold in fp64).
    """
    if callable(w_gate_up):
        fn = w_gate_up
        return lambda e: tuple(np.asarray(m, dtype=F64) for m in fn(e))
    return lambda e: (np.asarray(w_gate_up[e], dtype=F64), np.asarray(w_down[e], dtype=F64))


# ------------------------------------------------------------------ forward
def forward(X, topk_ids, topk_weights, experts, E: int, act: str, layout: str,
            limit: float = 7.0, alpha: float = 1.702) -> np.ndarray:
    """out[t] = sum_k w[t,k] * FFN_{ids[t,k]}(x_t), one expert at a time.

    Follows "Sparse expert dispatch and combine" (description): for each
    expert in turn, extract its tokens, gate_up projection, gated GLU, down
    projection, then index_add_ the weighted rows into the output; the
    weighting before the sum is from "MoE training token repeat and expert
    computation" (description).
    """
    X = np.asarray(X, dtype=F64)
    T, H = X.shape
    K = np.asarray(topk_ids).shape[1]
    w = np.asarray(topk_weights, dtype=F64).reshape(-1)
    counts, offsets, sorted_slot, _ = route(topk_ids, E)
    out = np.zeros((T, H), dtype=F64)
    for e in range(E):
        R = sorted_slot[offsets[e]:offsets[e + 1]]
        if R.size == 0:
            continue
        tok = R // K
        Wgu, Wd = experts(e)
        Xe = X[tok]                               # sparse token extraction
        Ze = Xe @ Wgu.T                           # gate_up projection [c, 2I]
        g, u = split_gate_up(Ze, layout)
        A = glu(g, u, act, limit, alpha)          # gated GLU [c, I]
        Ye = A @ Wd.T                             # down projection [c, H]
        np.add.at(out, tok, w[R][:, None] * Ye)   # weighted index_add_
    return out


def slot_outputs(X, topk_ids, experts, E: int, act: str, layout: str,
                 limit: float = 7.0, alpha: float = 1.702) -> np.ndarray:
    """y[s] = FFN_{e_s}(x_{s // K}) for every slot, unweighted, [S, H]."""
    X = np.asarray(X, dtype=F64)
    ids = np.asarray(topk_ids)
    T, K = ids.shape
    Y = np.zeros((T * K, X.shape[1]), dtype=F64)
    counts, offsets, sorted_slot, _ = route(ids, E)
    for e in range(E):
        R = sorted_slot[offsets[e]:offsets[e + 1]]
        if R.size == 0:
            continue
        Wgu, Wd = experts(e)
        g, u = split_gate_up(X[R // K] @ Wgu.T, layout)
        Y[R] = glu(g, u, act, limit, alpha) @ Wd.T
    return Y


# ------------------------------------------------------------------ backward
def backward(X, topk_ids, topk_weights, dY, experts, E: int, act: str, layout: str,
             limit: float = 7.0, alpha: float = 1.702,
             dw_sink: Optional[Callable[[int, np.ndarray, np.ndarray], None]] = None):
    """Gradients of L = <dY, forward(...)> ("MoE expert parallel execution backward").

    Returns (d_hidden [T,H], d_topk_weights [T,K], d_w_gate_up [E,2I,H],
    d_w_down [E,H,I]).  With ``dw_sink`` the weight gradients are handed over
    one expert at a time as dw_sink(e, dWgu_e, dWd_e) instead (None, None is
    returned for them); an expert with no slots gets exact zeros (handed to
    the sink as dw_sink(e, None, None)).

    Per expert, with the forward recomputed:
      r   = dY[tok] @ Wd[e]                 grad of the unweighted expert output
      dTopkW[slot] = <r, a>                 (equals <dY_t, y_s>)
      da  = w * r
      (dg, du) = phi'(g, u) . da            reassembled into dZ in the stored layout
      d_hidden[tok] += dZ @ Wgu[e]
      dWd[e]  = (w * dY[tok])^T @ a,  dWgu[e] = dZ^T @ X[tok]
    """
    X = np.asarray(X, dtype=F64)
    dY = np.asarray(dY, dtype=F64)
    T, H = X.shape
    ids = np.asarray(topk_ids)
    K = ids.shape[1]
    w = np.asarray(topk_weights, dtype=F64).reshape(-1)
    counts, offsets, sorted_slot, _ = route(ids, E)
    dX = np.zeros((T, H), dtype=F64)
    dTopkW = np.zeros(T * K, dtype=F64)
    dWgu_all = dWd_all = None
    for e in range(E):
        R = sorted_slot[offsets[e]:offsets[e + 1]]
        if R.size == 0:
            if dw_sink is not None:
                dw_sink(e, None, None)
            continue
        tok = R // K
        Wgu, Wd = experts(e)
        if dw_sink is None and dWgu_all is None:
            dWgu_all = np.zeros((E,) + Wgu.shape, dtype=F64)
            dWd_all = np.zeros((E,) + Wd.shape, dtype=F64)
        Xe = X[tok]
        Ze = Xe @ Wgu.T
        g, u = split_gate_up(Ze, layout)
        A = glu(g, u, act, limit, alpha)
        dYe = dY[tok]
        Re = dYe @ Wd                               # [c, I]
        dTopkW[R] = (Re * A).sum(axis=1)
        dA = w[R][:, None] * Re
        dg, du = glu_backward(g, u, dA, act, limit, alpha)
        dZe = merge_gate_up(dg, du, layout)         # [c, 2I]
        np.add.at(dX, tok, dZe @ Wgu)
        dWd_e = (w[R][:, None] * dYe).T @ A         # [H, I]
        dWgu_e = dZe.T @ Xe                         # [2I, H]
        if dw_sink is None:
            dWd_all[e] = dWd_e
            dWgu_all[e] = dWgu_e
        else:
            dw_sink(e, dWgu_e, dWd_e)
    if dw_sink is None and dWgu_all is None:        # every expert empty (T == 0)
        Wgu, Wd = experts(0)
        dWgu_all = np.zeros((E,) + Wgu.shape, dtype=F64)
        dWd_all = np.zeros((E,) + Wd.shape, dtype=F64)
    return dX, dTopkW.reshape(T, K), dWgu_all, dWd_all
