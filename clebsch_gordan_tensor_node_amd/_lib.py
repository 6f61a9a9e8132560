"""ctypes declarations of libcgtp.so (the C ABI in include/cgtp.h).

Loading order matters: torch is imported first so that its HIP runtime
(libamdhip64.so.7) is the one libcgtp binds to; the two then share devices and
streams.  A missing library is an error, never a fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must be loaded before libcgtp: one HIP runtime per process)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcgtp.so")

CGTP_OK = 0
ERRORS = {
    -1: "CGTP_ERR_INVALID_ARG", -2: "CGTP_ERR_PARSE", -3: "CGTP_ERR_UNSUPPORTED",
    -4: "CGTP_ERR_CAPACITY", -5: "CGTP_ERR_WORKSPACE", -6: "CGTP_ERR_HIP", -7: "CGTP_ERR_NO_DEVICE",
}
CGTP_ERR_CAPACITY = -4
CGTP_PATHS_ALL = 0
CGTP_PATHS_PARITY = 1
CGTP_PLAN_HOST_ONLY = 1
CGTP_PLAN_FP64 = 2

EXPORTED = [
    "cgtp_plan_create", "cgtp_plan_info", "cgtp_plan_paths", "cgtp_plan_cg", "cgtp_plan_schedule",
    "cgtp_workspace_size", "cgtp_neighbors_workspace_size", "cgtp_neighbors_build",
    "cgtp_conv_prepare", "cgtp_edge_sh", "cgtp_conv_forward", "cgtp_conv_forward_gated", "cgtp_conv_forward_timed",
    "cgtp_conv_forward_f64", "cgtp_conv_forward_noalloc", "cgtp_backward_workspace_size", "cgtp_conv_backward", "cgtp_plan_destroy",
    "cgtp_last_error", "cgtp_version",
]


class CgtpError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERRORS.get(code, code)}: {message}")
        self.code = code


_lib = None

P = ctypes.c_void_p
I64 = ctypes.c_int64
I32 = ctypes.c_int
SZ = ctypes.c_size_t
FP = ctypes.POINTER(ctypes.c_float)
DP = ctypes.POINTER(ctypes.c_double)


def load():
    """Load libcgtp.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -m clebsch_gordan_tensor_node_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "cgtp_plan_create": ([ctypes.c_char_p, ctypes.c_char_p, I32, I32, ctypes.c_uint, ctypes.POINTER(P)], I32),
        "cgtp_plan_info": ([P, ctypes.POINTER(I64), ctypes.POINTER(I64), ctypes.POINTER(I64),
                            ctypes.POINTER(I32), ctypes.POINTER(I32), ctypes.c_char_p, SZ], I32),
        "cgtp_plan_paths": ([P, ctypes.POINTER(ctypes.c_int32)], I32),
        "cgtp_plan_cg": ([P, I32, FP], I32),
        "cgtp_plan_schedule": ([P, ctypes.POINTER(I32), ctypes.POINTER(I32)], I32),
        "cgtp_workspace_size": ([P, I64, I64, I32, ctypes.POINTER(SZ)], I32),
        "cgtp_neighbors_workspace_size": ([I64, FP, ctypes.c_float, ctypes.POINTER(SZ)], I32),
        "cgtp_neighbors_build": ([P, I64, FP, ctypes.c_float, P, P, P, I64, ctypes.POINTER(I64), P, SZ, P], I32),
        "cgtp_conv_prepare": ([P, P, P, I64, I64, P, P, P, P, SZ, P], I32),
        "cgtp_edge_sh": ([P, P, I64, FP, P, P, P, I64, P, P], I32),
        "cgtp_conv_forward": ([P, P, I64, FP, P, P, P, I64, P, P, P, P, P, SZ, P], I32),
        "cgtp_conv_forward_gated": ([P, P, I64, FP, P, P, P, I64, P, P, P, P, P, P, SZ, P], I32),
        "cgtp_conv_forward_timed": ([P, P, I64, FP, P, P, P, I64, P, P, P, P, P, P, SZ, P, P, P], I32),
        "cgtp_conv_forward_f64": ([P, P, I64, DP, P, P, P, I64, P, P, P, P, P, P, SZ, P, P, P], I32),
        "cgtp_conv_forward_noalloc": ([P, P, I64, FP, P, P, P, I64, P, P, P, P, P, P], I32),
        "cgtp_backward_workspace_size": ([P, I64, I64, ctypes.POINTER(SZ)], I32),
        "cgtp_conv_backward": ([P, P, I64, FP, P, P, P, I64, P, P, P, P, P, P, P, P, P, SZ, P], I32),
        "cgtp_plan_destroy": ([P], None),
        "cgtp_last_error": ([], ctypes.c_char_p),
        "cgtp_version": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def check(rc: int) -> int:
    if rc != CGTP_OK:
        raise CgtpError(rc, load().cgtp_last_error().decode())
    return rc
