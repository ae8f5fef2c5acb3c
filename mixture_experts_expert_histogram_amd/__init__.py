"""Routed mixture-of-experts expert computation on AMD Instinct MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI declared in
``include/moe.h``; this package is its thin Python binding.  ``build`` compiles
the library in-tree.
"""
from ._lib import (  # noqa: F401
    EXPORTED, LIB_PATH, MOE_ERR_BAD_EXPERT_ID, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_OK,
    NOALLOC_SCRATCH_BYTES, MoeDesc, MoeError, bwd, bwd_sep, check_device_status, empty_workspace, fwd, fwd_logits,
    fwd_noalloc, fwd_sep, library,
    make_desc, route, route_workspace_size, router, router_bwd, status_str, timing_disable, timing_enable,
    timing_read, workspace_size,
)
