"""The C-ABI library loads on the host and exports every declared entry point;
argument checks fire before any launch (no GPU is touched by these tests)."""
import ctypes
import os
import re

import pytest

import mixture_experts_expert_histogram_amd as moe
from mixture_experts_expert_histogram_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(moe_[a-z_]+)\s*\(", src, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 8
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(_lib.EXPORTED)


def test_status_strings():
    assert moe.status_str(0) == "MOE_OK"
    assert moe.status_str(5) == "MOE_ERR_BAD_EXPERT_ID"
    assert moe.status_str(99) == "MOE_ERR_UNKNOWN"


def test_workspace_sizes_cover_the_buffers():
    d = moe.make_desc(4096, 2880, 2880, 128, 4, "bf16", "clamped", "interleaved")
    f, b, s = moe.workspace_size(d)
    S = 4096 * 4
    assert s == S * 2 * 2880 * 4                    # Z is kept in fp32
    assert f >= S * 2880 * 2 + S * 2880 * 4         # a (bf16) + per-slot down outputs (fp32)
    assert b >= S * 2 * 2880 * 4 + S * 2 * 2880 * 2 + S * 2880 * 2 + S * 2880 * 4
    assert moe.route_workspace_size(d) < f


def _call_fwd(d, ptr=16, ws_bytes=1 << 40):
    lib = moe.library()
    p = ctypes.c_void_p(ptr)
    return lib.moe_fwd(ctypes.byref(d), p, p, p, p, p, p, None, 0, p, ws_bytes, None)


def test_argument_errors_before_launch():
    lib = moe.library()
    good = moe.make_desc(64, 128, 128, 8, 2, "fp32")
    # misaligned pointer
    assert _call_fwd(good, ptr=8) == _lib.MOE_ERR_INVALID_ARG
    # null required pointer
    p = ctypes.c_void_p(16)
    assert lib.moe_fwd(ctypes.byref(good), None, p, p, p, p, p, None, 0, p, 1 << 40, None) == _lib.MOE_ERR_INVALID_ARG
    # workspace too small
    assert _call_fwd(good, ws_bytes=100) == _lib.MOE_ERR_WORKSPACE
    # unsupported shapes
    assert _call_fwd(moe.make_desc(64, 100, 128, 8, 2)) == _lib.MOE_ERR_UNSUPPORTED
    assert _call_fwd(moe.make_desc(64, 128, 12, 8, 2)) == _lib.MOE_ERR_UNSUPPORTED
    assert _call_fwd(moe.make_desc(64, 128, 128, 2000, 2)) == _lib.MOE_ERR_UNSUPPORTED
    # invalid descriptors
    for bad in [moe.make_desc(-1, 128, 128, 8, 2), moe.make_desc(64, 128, 128, 0, 2),
                moe.make_desc(64, 128, 128, 8, 0), moe.make_desc(64, 0, 128, 8, 2)]:
        assert _call_fwd(bad) == _lib.MOE_ERR_INVALID_ARG
    d = moe.make_desc(64, 128, 128, 8, 2)
    d.dtype = 7
    assert _call_fwd(d) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_fwd(None, p, p, p, p, p, p, None, 0, p, 1 << 40, None) == _lib.MOE_ERR_INVALID_ARG
    # (T = 0 passes these checks and then clears the status word on the device:
    # covered by the GPU tests)


def test_bwd_argument_errors():
    lib = moe.library()
    d = moe.make_desc(64, 128, 128, 8, 2)
    p = ctypes.c_void_p(16)
    args = [p] * 11
    assert lib.moe_bwd(ctypes.byref(d), *args[:6], None, 0, *args[6:10], p, 100, None) == _lib.MOE_ERR_WORKSPACE
    assert lib.moe_bwd(ctypes.byref(d), *args[:6], None, 0, p, p, None, p, p, 1 << 40, None) == _lib.MOE_ERR_INVALID_ARG


def test_route_and_status_argument_errors():
    lib = moe.library()
    d = moe.make_desc(64, 8, 8, 8, 2)
    p = ctypes.c_void_p(16)
    assert lib.moe_route(ctypes.byref(d), p, None, None, None, None, p, 10, None) == _lib.MOE_ERR_WORKSPACE
    assert lib.moe_route(ctypes.byref(d), None, None, None, None, None, p, 1 << 30, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_check_device_status(None, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_timing_enable(0) == _lib.MOE_ERR_INVALID_ARG


def test_router_argument_errors():
    lib = moe.library()
    p = ctypes.c_void_p(16)
    d = moe.make_desc(64, 8, 8, 8, 2)
    big = 1 << 30
    # K > E: the router cannot pick K distinct experts
    d9 = moe.make_desc(64, 8, 8, 8, 9)
    assert lib.moe_router(ctypes.byref(d9), p, p, p, None, None, None, None, p, big, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_router(ctypes.byref(d), None, p, p, None, None, None, None, p, big, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_router(ctypes.byref(d), ctypes.c_void_p(8), p, p, None, None, None, None, p, big,
                          None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_router(ctypes.byref(d), p, p, p, None, None, None, None, p, 10, None) == _lib.MOE_ERR_WORKSPACE
    assert lib.moe_fwd_logits(ctypes.byref(d), p, None, p, p, p, p, p, None, 0, p, big, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_fwd_logits(ctypes.byref(d9), p, p, p, p, p, p, p, None, 0, p, big, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_fwd_logits(ctypes.byref(d), p, p, p, p, p, p, p, None, 0, p, 10, None) == _lib.MOE_ERR_WORKSPACE
    assert lib.moe_router_bwd(ctypes.byref(d), p, p, None, p, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_router_bwd(ctypes.byref(d), p, p, p, ctypes.c_void_p(4), None) == _lib.MOE_ERR_INVALID_ARG


def test_separate_weight_argument_errors():
    lib = moe.library()
    p = ctypes.c_void_p(16)
    d = moe.make_desc(64, 8, 8, 8, 2)
    big = 1 << 30
    assert lib.moe_fwd_sep(ctypes.byref(d), p, p, p, p, None, p, p, None, 0, p, big, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_fwd_sep(ctypes.byref(d), p, p, p, p, p, p, p, None, 0, p, 10, None) == _lib.MOE_ERR_WORKSPACE
    assert lib.moe_bwd_sep(ctypes.byref(d), p, p, p, p, p, p, p, None, 0, p, p, p, None, p, p, big,
                           None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_bwd_sep(ctypes.byref(d), p, p, p, p, p, p, p, None, 0, p, p, p, p, p, p, 10,
                           None) == _lib.MOE_ERR_WORKSPACE


def test_saved_buffer_size_is_checked():
    """A `saved` buffer smaller than moe_workspace_size's saved_bytes is
    rejected before any launch, by the forward that fills it and by the
    backward that reads it."""
    lib = moe.library()
    d = moe.make_desc(64, 128, 128, 8, 2)
    _, _, sbytes = moe.workspace_size(d)
    p = ctypes.c_void_p(16)
    big = 1 << 40
    assert lib.moe_fwd(ctypes.byref(d), p, p, p, p, p, p, p, sbytes - 16, p, big, None) == _lib.MOE_ERR_WORKSPACE
    assert lib.moe_fwd_logits(ctypes.byref(d), p, p, p, p, p, p, p, p, sbytes - 16, p, big,
                              None) == _lib.MOE_ERR_WORKSPACE
    assert lib.moe_fwd_sep(ctypes.byref(d), p, p, p, p, p, p, p, p, sbytes - 16, p, big,
                           None) == _lib.MOE_ERR_WORKSPACE
    assert lib.moe_bwd(ctypes.byref(d), p, p, p, p, p, p, p, sbytes - 16, p, p, p, p, p, big,
                       None) == _lib.MOE_ERR_WORKSPACE
    assert lib.moe_bwd_sep(ctypes.byref(d), p, p, p, p, p, p, p, p, sbytes - 16, p, p, p, p, p, p, big,
                           None) == _lib.MOE_ERR_WORKSPACE
