"""Dense torch-CPU fp64 formulation of the routed MoE layer (test helper).

Independent of the oracle: every expert is applied to every token, and the
routing enters only through a dense gate matrix G[t, e] = sum_k w[t,k]*[ids[t,k]==e].
The GLU uses torch.nn.functional (silu) and torch.clamp/sigmoid.
"""
import numpy as np
import torch
import torch.nn.functional as F


def t64(x, grad=False):
    return torch.tensor(np.asarray(x, dtype=np.float64), dtype=torch.float64, requires_grad=grad)


def gate_matrix(ids, w, E):
    """Dense [T,E] gate built by a scatter-add (differentiable in w)."""
    ids = torch.as_tensor(np.asarray(ids, dtype=np.int64))
    T = ids.shape[0]
    G = torch.zeros((T, E), dtype=torch.float64)
    return G.scatter_add(1, ids, w)


def act_fn(g, u, act, limit=7.0, alpha=1.702):
    if act == "swiglu":
        return F.silu(g) * u
    gc = torch.clamp(g, max=limit)
    uc = torch.clamp(u, min=-limit, max=limit)
    return (uc + 1.0) * gc * torch.sigmoid(alpha * gc)


def ffn(x, wgu, wd, act, layout, limit=7.0, alpha=1.702):
    """One expert on every row of x: [T,H] -> [T,H]."""
    z = F.linear(x, wgu)
    I = wd.shape[1]
    if layout == "concat":
        g, u = z[:, :I], z[:, I:]
    else:
        g, u = z[:, 0::2], z[:, 1::2]
    return F.linear(act_fn(g, u, act, limit, alpha), wd)


def dense_forward(X, ids, w, Wgu, Wd, act, layout, limit=7.0, alpha=1.702):
    """out[t] = sum_e G[t,e] * FFN_e(x_t) with all torch fp64 tensors."""
    E = Wgu.shape[0]
    G = gate_matrix(ids, w, E)
    out = torch.zeros_like(X)
    for e in range(E):
        out = out + G[:, e:e + 1] * ffn(X, Wgu[e], Wd[e], act, layout, limit, alpha)
    return out
