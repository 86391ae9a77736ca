"""ctypes declarations of libptg.so (the C ABI in include/ptg.h).

Loading fails loudly: there is no fallback implementation of any call.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libptg.so")

PTG_OK = 0
STATUS_NAMES = {
    0: "PTG_OK",
    1: "PTG_ERR_INVALID_ARG",
    2: "PTG_ERR_UNSUPPORTED",
    3: "PTG_ERR_WORKSPACE",
    4: "PTG_ERR_HIP",
    5: "PTG_ERR_DEVICE_CHECK",
}

# Every symbol include/ptg.h declares (checked by the CPU tests).
EXPORTS = (
    "ptg_gemm", "ptg_grouped_gemm", "ptg_grouped_gemm_split", "ptg_grouped_gemm_split_workspace",
    "ptg_grouped_gemm_check", "ptg_grouped_gemm_wgrad",
    "ptg_grouped_gemm_wgrad_workspace", "ptg_ikbo_attention",
    "ptg_grouped_gemm_ptr_array_workspace", "ptg_grouped_gemm_ptr_array",
    "ptg_grouped_gemm_ptr_array_prepare", "ptg_grouped_gemm_ptr_array_run",
    "ptg_broadcast_gemm_workspace", "ptg_broadcast_gemm", "ptg_broadcast_gemm_noalloc",
    "ptg_broadcast_gemm_fused_workspace", "ptg_broadcast_gemm_fused",
    "ptg_broadcast_gemm_check",
    "ptg_status_string", "ptg_last_error", "ptg_watchdog", "ptg_version", "ptg_describe_config",
)


class ProblemStruct(ctypes.Structure):
    """Mirror of ptg_problem."""
    _fields_ = [
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p),
        ("bias", ctypes.c_void_p),
        ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldc", ctypes.c_int64),
    ]


_lib = None


def load(path: str = LIB_PATH):
    """Load and declare libptg.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = open_library(path)
    return _lib


def open_library(path: str):
    """A declared handle on a build of the library at `path` (the product build, or a
    test build of the same sources); raises if the file is missing."""
    if not os.path.exists(path):
        raise ImportError(
            f"{os.path.basename(path)} not found at {path}: build it with "
            "`python -m pipelined_tiled_gemm_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(path)
    i64, i32, p, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    e = ctypes.c_int  # enums
    L.ptg_gemm.argtypes = [i64, i64, i64, p, i64, p, i64, e, p, i64, e, p, e, p]
    L.ptg_grouped_gemm.argtypes = [i32, i64, i64, i64, p, p, e, p, p, e, p, e, p]
    L.ptg_grouped_gemm_check.argtypes = [i32, i64, p, p]
    L.ptg_grouped_gemm_split.argtypes = [i32, i64, i64, i64, p, p, e, p, p, e, p, e, p, sz, p]
    L.ptg_grouped_gemm_split_workspace.argtypes = []
    L.ptg_grouped_gemm_split_workspace.restype = sz
    L.ptg_grouped_gemm_wgrad.argtypes = [i32, i64, i64, i64, p, p, p, p, e, p, sz, p]
    L.ptg_ikbo_attention.argtypes = [i64, i64, i64, i64, i64, ctypes.c_float, p, p, p, p, p, e, p]
    L.ptg_grouped_gemm_wgrad_workspace.argtypes = []
    L.ptg_grouped_gemm_wgrad_workspace.restype = sz
    L.ptg_grouped_gemm_ptr_array_workspace.argtypes = [i32]
    L.ptg_grouped_gemm_ptr_array_workspace.restype = sz
    L.ptg_grouped_gemm_ptr_array.argtypes = [i32, ctypes.POINTER(ProblemStruct), e, e, p, sz, p]
    L.ptg_grouped_gemm_ptr_array_prepare.argtypes = [i32, ctypes.POINTER(ProblemStruct), e, e, p, sz, p]
    L.ptg_grouped_gemm_ptr_array_run.argtypes = [i32, p, sz, e, e, p]
    L.ptg_broadcast_gemm_workspace.argtypes = [i64, i64]
    L.ptg_broadcast_gemm_workspace.restype = sz
    L.ptg_broadcast_gemm.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, e, p, e, p, e, p, sz, p]
    L.ptg_broadcast_gemm_check.argtypes = [i64, i64, p, p]
    L.ptg_broadcast_gemm_noalloc.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, e, p, e, p, e, p]
    L.ptg_broadcast_gemm_fused_workspace.argtypes = [i64, i64]
    L.ptg_broadcast_gemm_fused_workspace.restype = sz
    L.ptg_broadcast_gemm_fused.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, e, p, e, p, e, p, sz, p]
    for f in (L.ptg_gemm, L.ptg_grouped_gemm, L.ptg_grouped_gemm_split, L.ptg_grouped_gemm_check, L.ptg_grouped_gemm_wgrad, L.ptg_ikbo_attention,
              L.ptg_grouped_gemm_ptr_array, L.ptg_grouped_gemm_ptr_array_prepare,
              L.ptg_grouped_gemm_ptr_array_run, L.ptg_broadcast_gemm, L.ptg_broadcast_gemm_noalloc,
              L.ptg_broadcast_gemm_fused,
              L.ptg_broadcast_gemm_check):
        f.restype = e
    L.ptg_status_string.argtypes = [e]
    L.ptg_status_string.restype = ctypes.c_char_p
    L.ptg_last_error.argtypes = []
    L.ptg_last_error.restype = ctypes.c_char_p
    L.ptg_watchdog.argtypes = [ctypes.POINTER(ctypes.c_uint32), i32]
    L.ptg_watchdog.restype = e
    L.ptg_version.argtypes = []
    L.ptg_version.restype = i32
    L.ptg_describe_config.argtypes = [i64, i64, i64, e, ctypes.POINTER(ctypes.c_int32)]
    L.ptg_describe_config.restype = e
    return L
