"""ctypes binding of the C ABI in include/moe.h (argument marshalling only).

Every step of the computation runs in the HIP library; torch supplies device
memory and the current stream.  Loading fails loudly if the library is not
built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_BAD_EXPERT_ID = range(6)
MOE_BF16, MOE_F32 = 0, 1
MOE_SWIGLU, MOE_CLAMPED_GLU = 0, 1
MOE_GU_CONCAT, MOE_GU_INTERLEAVED = 0, 1

EXPORTED = ["moe_workspace_size", "moe_route_workspace_size", "moe_route", "moe_router", "moe_fwd",
            "moe_fwd_logits", "moe_fwd_sep", "moe_bwd", "moe_bwd_sep", "moe_router_bwd", "moe_check_device_status",
            "moe_status_str", "moe_timing_enable", "moe_timing_disable", "moe_timing_read", "moe_fwd_noalloc"]

# Size of the library's per-GPU scratch array behind moe_fwd_noalloc (moe.h).
NOALLOC_SCRATCH_BYTES = 64 << 20


class MoeDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("I", ctypes.c_int64),
                ("E", ctypes.c_int64), ("K", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("act", ctypes.c_int32), ("gu_layout", ctypes.c_int32),
                ("clamp_limit", ctypes.c_float), ("glu_alpha", ctypes.c_float),
                ("grad_dtype", ctypes.c_int32)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double)]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


_lib = None


def library() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"MoE HIP library not built: {LIB_PATH} is missing "
                          "(run `python -m mixture_experts_expert_histogram_amd.build`)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    pd = ctypes.POINTER(MoeDesc)
    psz = ctypes.POINTER(ctypes.c_size_t)
    lib.moe_workspace_size.argtypes = [pd, psz, psz, psz]
    lib.moe_route_workspace_size.argtypes = [pd, psz]
    lib.moe_route.argtypes = [pd, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_router.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_fwd.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]
    lib.moe_fwd_logits.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]
    lib.moe_router_bwd.argtypes = [pd, vp, vp, vp, vp, vp]
    lib.moe_fwd_sep.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]
    lib.moe_bwd_sep.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_bwd.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_fwd_noalloc.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
    lib.moe_check_device_status.argtypes = [vp, vp]
    lib.moe_status_str.argtypes = [ctypes.c_int]
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_timing_enable.argtypes = [ctypes.c_int32]
    lib.moe_timing_disable.argtypes = []
    lib.moe_timing_read.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    for name in ["moe_workspace_size", "moe_route_workspace_size", "moe_route", "moe_router", "moe_fwd",
                 "moe_fwd_logits", "moe_fwd_sep", "moe_bwd", "moe_bwd_sep", "moe_router_bwd",
                 "moe_check_device_status", "moe_timing_enable", "moe_timing_disable", "moe_timing_read",
                 "moe_fwd_noalloc"]:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return library().moe_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def _dt(name) -> int:
    if name in ("bf16", "bfloat16"):
        return MOE_BF16
    if name in ("fp32", "float32"):
        return MOE_F32
    raise ValueError(f"unsupported dtype {name}")


def make_desc(T, H, I, E, K, dtype="bf16", act="swiglu", layout="concat", limit=7.0, alpha=1.702,
              grad_dtype=None) -> MoeDesc:
    return MoeDesc(int(T), int(H), int(I), int(E), int(K), _dt(dtype),
                   MOE_CLAMPED_GLU if act == "clamped" else MOE_SWIGLU,
                   MOE_GU_INTERLEAVED if layout == "interleaved" else MOE_GU_CONCAT,
                   float(limit), float(alpha), _dt(grad_dtype or dtype))


def workspace_size(desc: MoeDesc) -> Tuple[int, int, int]:
    f, b, s = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(library().moe_workspace_size(ctypes.byref(desc), ctypes.byref(f), ctypes.byref(b), ctypes.byref(s)),
           "moe_workspace_size")
    return f.value, b.value, s.value


def route_workspace_size(desc: MoeDesc) -> int:
    r = ctypes.c_size_t()
    _check(library().moe_route_workspace_size(ctypes.byref(desc), ctypes.byref(r)), "moe_route_workspace_size")
    return r.value


# ---------------------------------------------------------------- torch layer
def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ids32(topk_ids):
    import torch
    return topk_ids if topk_ids.dtype == torch.int32 and topk_ids.is_contiguous() else \
        topk_ids.to(torch.int32).contiguous()


def _f32(x):
    import torch
    return x if x.dtype == torch.float32 and x.is_contiguous() else x.to(torch.float32).contiguous()


def _desc_for(hidden, topk_ids, w_gate_up, w_down, act, layout, limit, alpha, grad_dtype=None) -> MoeDesc:
    import torch
    T, H = hidden.shape
    E, I2, H2 = w_gate_up.shape
    if H2 != H or tuple(w_down.shape) != (E, H, I2 // 2) or topk_ids.shape[0] != T:
        raise ValueError("inconsistent MoE shapes")
    for t in (hidden, w_gate_up, w_down):
        if t.dtype != hidden.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("hidden and weights must be contiguous device tensors of one dtype")
    dt = "bf16" if hidden.dtype == torch.bfloat16 else ("fp32" if hidden.dtype == torch.float32 else None)
    if dt is None:
        raise ValueError(f"unsupported dtype {hidden.dtype}")
    return make_desc(T, H, I2 // 2, E, topk_ids.shape[1], dt, act, layout, limit, alpha, grad_dtype)


def empty_workspace(nbytes: int, device):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def route(topk_ids, E: int, ws=None):
    """counts [E], offsets [E+1], sorted_slot [S], inv_pos [S] (int32 device tensors)."""
    import torch
    ids = _ids32(topk_ids)
    T, K = ids.shape
    d = make_desc(T, 8, 8, E, K)
    dev = ids.device
    nbytes = route_workspace_size(d)
    ws = empty_workspace(nbytes, dev) if ws is None else ws
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    ss = torch.empty(T * K, dtype=torch.int32, device=dev)
    ip = torch.empty(T * K, dtype=torch.int32, device=dev)
    _check(library().moe_route(ctypes.byref(d), _ptr(ids), _ptr(counts), _ptr(offsets), _ptr(ss), _ptr(ip),
                               _ptr(ws), ws.numel(), _stream()), "moe_route")
    return counts, offsets, ss, ip, ws


def router(logits, K: int, ws=None, out=None):
    """Top-K of router logits [T,E] (fp32) and their softmax, with the routing.

    Returns (topk_ids int32 [T,K], topk_weights fp32 [T,K], counts [E],
    offsets [E+1], sorted_slot [S], inv_pos [S], ws)."""
    import torch
    lg = _f32(logits)
    if not lg.is_cuda or lg.dim() != 2:
        raise ValueError("router takes device logits [T, E]")
    T, E = lg.shape
    d = make_desc(T, 8, 8, E, K)
    dev = lg.device
    ws = empty_workspace(route_workspace_size(d), dev) if ws is None else ws
    if out is None:
        out = (torch.empty((T, K), dtype=torch.int32, device=dev), torch.empty((T, K), dtype=torch.float32, device=dev))
    ids, w = out
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    ss = torch.empty(T * K, dtype=torch.int32, device=dev)
    ip = torch.empty(T * K, dtype=torch.int32, device=dev)
    _check(library().moe_router(ctypes.byref(d), _ptr(lg), _ptr(ids), _ptr(w), _ptr(counts), _ptr(offsets),
                                _ptr(ss), _ptr(ip), _ptr(ws), ws.numel(), _stream()), "moe_router")
    return ids, w, counts, offsets, ss, ip, ws


def router_bwd(topk_ids, topk_weights, d_topk_weights, E: int, out=None):
    """d_logits fp32 [T,E] from the routing-weight gradient."""
    import torch
    ids, w, g = _ids32(topk_ids), _f32(topk_weights), _f32(d_topk_weights)
    T, K = ids.shape
    if tuple(w.shape) != (T, K) or tuple(g.shape) != (T, K):
        raise ValueError("topk_ids, topk_weights and d_topk_weights must all be [T, K]")
    if not (ids.is_cuda and w.is_cuda and g.is_cuda):
        raise ValueError("router_bwd takes device tensors")
    d = make_desc(T, 8, 8, E, K)
    out = torch.empty((T, E), dtype=torch.float32, device=ids.device) if out is None else out
    _check(library().moe_router_bwd(ctypes.byref(d), _ptr(ids), _ptr(w), _ptr(g), _ptr(out), _stream()),
           "moe_router_bwd")
    return out


def fwd_logits(hidden, logits, K: int, w_gate_up, w_down, act="swiglu", layout="concat", limit=7.0, alpha=1.702,
               save=False, ws=None, out=None, saved=None, routing=None):
    """Forward from router logits [T,E]; returns (out, topk_ids, topk_weights, saved-or-None, ws)."""
    import torch
    lg = _f32(logits)
    T, E = lg.shape
    if T != hidden.shape[0] or E != w_gate_up.shape[0]:
        raise ValueError("logits must be [T, E] for hidden [T, H] and w_gate_up [E, 2I, H]")
    dev = hidden.device
    if routing is None:
        routing = (torch.empty((T, K), dtype=torch.int32, device=dev),
                   torch.empty((T, K), dtype=torch.float32, device=dev))
    ids, w = routing
    d = _desc_for(hidden, ids, w_gate_up, w_down, act, layout, limit, alpha)
    fws, _, sbytes = workspace_size(d)
    ws = empty_workspace(fws, dev) if ws is None else ws
    out = torch.empty_like(hidden) if out is None else out
    if save and saved is None:
        saved = empty_workspace(sbytes, dev)
    _check(library().moe_fwd_logits(ctypes.byref(d), _ptr(hidden), _ptr(lg), _ptr(w_gate_up), _ptr(w_down),
                                    _ptr(out), _ptr(ids), _ptr(w), _ptr(saved) if save else None,
                                    _nbytes(saved) if save else 0, _ptr(ws), ws.numel(), _stream()),
           "moe_fwd_logits")
    return out, ids, w, (saved if save else None), ws


def fwd(hidden, topk_ids, topk_weights, w_gate_up, w_down, act="swiglu", layout="concat", limit=7.0,
        alpha=1.702, save=False, ws=None, out=None, saved=None):
    """Forward pass; returns (out, saved-or-None, ws)."""
    import torch
    d = _desc_for(hidden, topk_ids, w_gate_up, w_down, act, layout, limit, alpha)
    ids, w = _ids32(topk_ids), _f32(topk_weights)
    fws, _, sbytes = workspace_size(d)
    ws = empty_workspace(fws, hidden.device) if ws is None else ws
    out = torch.empty_like(hidden) if out is None else out
    if save and saved is None:
        saved = empty_workspace(sbytes, hidden.device)
    _check(library().moe_fwd(ctypes.byref(d), _ptr(hidden), _ptr(ids), _ptr(w), _ptr(w_gate_up), _ptr(w_down),
                             _ptr(out), _ptr(saved) if save else None, _nbytes(saved) if save else 0, _ptr(ws),
                             ws.numel(), _stream()), "moe_fwd")
    return out, (saved if save else None), ws


def fwd_noalloc(hidden, topk_ids, topk_weights, w_gate_up, w_down, act="swiglu", layout="concat", limit=7.0,
                alpha=1.702, out=None, saved=None, bad_ids=None):
    """Forward with the library's own per-GPU scratch as workspace (moe_fwd_noalloc);
    returns out.  `saved` (optional) receives Z as for fwd(save=True); `bad_ids`
    (optional int32 device tensor of one element) the number of bad-id slots."""
    import torch
    d = _desc_for(hidden, topk_ids, w_gate_up, w_down, act, layout, limit, alpha)
    ids, w = _ids32(topk_ids), _f32(topk_weights)
    out = torch.empty_like(hidden) if out is None else out
    _check(library().moe_fwd_noalloc(ctypes.byref(d), _ptr(hidden), _ptr(ids), _ptr(w), _ptr(w_gate_up),
                                     _ptr(w_down), _ptr(out), _ptr(saved), _nbytes(saved), _ptr(bad_ids),
                                     _stream()), "moe_fwd_noalloc")
    return out


def bwd(hidden, topk_ids, topk_weights, w_gate_up, w_down, d_out, saved=None, act="swiglu", layout="concat",
        limit=7.0, alpha=1.702, ws=None, grads=None, grad_dtype=None):
    """Backward pass; returns (d_hidden, d_topk_weights, d_w_gate_up, d_w_down, ws).

    grad_dtype: "bf16" or "fp32" storage of the weight gradients (default: the
    activation dtype)."""
    import torch
    d = _desc_for(hidden, topk_ids, w_gate_up, w_down, act, layout, limit, alpha, grad_dtype)
    ids, w = _ids32(topk_ids), _f32(topk_weights)
    _, bws, _ = workspace_size(d)
    ws = empty_workspace(bws, hidden.device) if ws is None else ws
    if grads is None:
        gdt = torch.float32 if d.grad_dtype == MOE_F32 else torch.bfloat16
        grads = (torch.empty_like(hidden), torch.empty(ids.shape, dtype=torch.float32, device=hidden.device),
                 torch.empty(w_gate_up.shape, dtype=gdt, device=hidden.device),
                 torch.empty(w_down.shape, dtype=gdt, device=hidden.device))
    dh, dw, dgu, dd = grads
    _check(library().moe_bwd(ctypes.byref(d), _ptr(hidden), _ptr(ids), _ptr(w), _ptr(w_gate_up), _ptr(w_down),
                             _ptr(d_out.contiguous()), _ptr(saved), _nbytes(saved), _ptr(dh), _ptr(dw), _ptr(dgu),
                             _ptr(dd), _ptr(ws), ws.numel(), _stream()), "moe_bwd")
    return dh, dw, dgu, dd, ws


def _sep_desc(hidden, topk_ids, w_gate, w_up, w_down, act, limit, alpha, grad_dtype=None) -> MoeDesc:
    import torch
    T, H = hidden.shape
    E, I, H2 = w_gate.shape
    if (H2 != H or tuple(w_up.shape) != (E, I, H) or tuple(w_down.shape) != (E, H, I)
            or topk_ids.shape[0] != T):
        raise ValueError("inconsistent MoE shapes")
    for t in (hidden, w_gate, w_up, w_down):
        if t.dtype != hidden.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("hidden and weights must be contiguous device tensors of one dtype")
    dt = "bf16" if hidden.dtype == torch.bfloat16 else ("fp32" if hidden.dtype == torch.float32 else None)
    if dt is None:
        raise ValueError(f"unsupported dtype {hidden.dtype}")
    return make_desc(T, H, I, E, topk_ids.shape[1], dt, act, "concat", limit, alpha, grad_dtype)


def fwd_sep(hidden, topk_ids, topk_weights, w_gate, w_up, w_down, act="swiglu", limit=7.0, alpha=1.702, save=False,
            ws=None, out=None, saved=None):
    """Forward with separate gate and up weights [E, I, H]; returns (out, saved-or-None, ws)."""
    import torch
    d = _sep_desc(hidden, topk_ids, w_gate, w_up, w_down, act, limit, alpha)
    ids, w = _ids32(topk_ids), _f32(topk_weights)
    fws, _, sbytes = workspace_size(d)
    ws = empty_workspace(fws, hidden.device) if ws is None else ws
    out = torch.empty_like(hidden) if out is None else out
    if save and saved is None:
        saved = empty_workspace(sbytes, hidden.device)
    _check(library().moe_fwd_sep(ctypes.byref(d), _ptr(hidden), _ptr(ids), _ptr(w), _ptr(w_gate), _ptr(w_up),
                                 _ptr(w_down), _ptr(out), _ptr(saved) if save else None,
                                 _nbytes(saved) if save else 0, _ptr(ws), ws.numel(), _stream()), "moe_fwd_sep")
    return out, (saved if save else None), ws


def bwd_sep(hidden, topk_ids, topk_weights, w_gate, w_up, w_down, d_out, saved=None, act="swiglu", limit=7.0,
            alpha=1.702, ws=None, grads=None, grad_dtype=None):
    """Backward with separate gate and up weights; returns
    (d_hidden, d_topk_weights, d_w_gate, d_w_up, d_w_down, ws)."""
    import torch
    d = _sep_desc(hidden, topk_ids, w_gate, w_up, w_down, act, limit, alpha, grad_dtype)
    ids, w = _ids32(topk_ids), _f32(topk_weights)
    _, bws, _ = workspace_size(d)
    ws = empty_workspace(bws, hidden.device) if ws is None else ws
    if grads is None:
        gdt = torch.float32 if d.grad_dtype == MOE_F32 else torch.bfloat16
        grads = (torch.empty_like(hidden), torch.empty(ids.shape, dtype=torch.float32, device=hidden.device),
                 torch.empty(w_gate.shape, dtype=gdt, device=hidden.device),
                 torch.empty(w_up.shape, dtype=gdt, device=hidden.device),
                 torch.empty(w_down.shape, dtype=gdt, device=hidden.device))
    dh, dw, dg, du, dd = grads
    _check(library().moe_bwd_sep(ctypes.byref(d), _ptr(hidden), _ptr(ids), _ptr(w), _ptr(w_gate), _ptr(w_up),
                                 _ptr(w_down), _ptr(d_out.contiguous()), _ptr(saved), _nbytes(saved), _ptr(dh),
                                 _ptr(dw), _ptr(dg), _ptr(du), _ptr(dd), _ptr(ws), ws.numel(), _stream()),
           "moe_bwd_sep")
    return dh, dw, dg, du, dd, ws


def check_device_status(ws) -> int:
    """Synchronises the current stream; returns the status code of the last routing in ws."""
    return library().moe_check_device_status(_ptr(ws), _stream())


def timing_enable(max_launches: int = 4096):
    _check(library().moe_timing_enable(int(max_launches)), "moe_timing_enable")


def timing_disable():
    _check(library().moe_timing_disable(), "moe_timing_disable")


def timing_read():
    """{kernel name: (launches, total_ms)} of the launches timed since the last read."""
    n = ctypes.c_int32()
    buf = (KernelTime * 64)()
    _check(library().moe_timing_read(buf, 64, ctypes.byref(n)), "moe_timing_read")
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(min(n.value, 64))}
