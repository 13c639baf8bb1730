"""ctypes view of libi8mm.so (the C ABI declared in include/i8mm.h).

torch is imported first so that the HIP runtime torch ships (SONAME
libamdhip64.so.7) is the one libi8mm binds to: streams and device pointers
then belong to a single runtime.  There is no fallback: if the library is
missing or does not load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads torch's HIP runtime before libi8mm)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libi8mm.so")

c_i64 = ctypes.c_int64
c_ptr = ctypes.c_void_p
c_size = ctypes.c_size_t
c_int = ctypes.c_int
c_float = ctypes.c_float


class WsLayout(ctypes.Structure):
    _fields_ = [
        ("counts", c_size), ("outliers", c_size), ("mask", c_size), ("sx", c_size),
        ("xq", c_size), ("xo", c_size), ("wo", c_size), ("zp", c_size), ("osum", c_size),
        ("part", c_size),
        ("ldq", c_i64), ("ldo", c_i64), ("splits", c_i64), ("total", c_size),
    ]


# name -> (restype, argtypes)
SIGNATURES = {
    "i8mm_status_string": (ctypes.c_char_p, [c_int]),
    "i8mm_abi_version": (c_int, []),
    "i8mm_set_split_override": (c_int, [c_i64]),
    "i8mm_set_tile_override": (c_int, [c_i64]),
    "i8mm_set_row_prep": (c_int, [c_int]),
    "int8_quantize_weight": (c_int, [c_ptr, c_i64, c_i64, c_ptr, c_ptr, c_ptr]),
    "int8_linear_workspace_layout": (c_int, [c_i64, c_i64, c_i64, c_i64, ctypes.POINTER(WsLayout)]),
    "int8_linear_workspace_size": (c_size, [c_i64, c_i64, c_i64, c_i64]),
    "int8_linear_workspace_init": (c_int, [c_ptr, c_i64, c_i64, c_i64, c_i64, c_ptr]),
    "int8_linear_forward": (c_int, [c_ptr, c_i64, c_i64, c_ptr, c_ptr, c_i64, c_ptr, c_float,
                                    c_ptr, c_ptr, c_size, c_i64, c_ptr]),
    "int8_weight_rowsum": (c_int, [c_ptr, c_i64, c_i64, c_ptr, c_ptr]),
    "int8_linear_forward_noalloc": (c_int, [c_ptr, c_i64, c_i64, c_ptr, c_ptr, c_i64, c_ptr,
                                            c_float, c_ptr, c_i64, c_ptr, c_ptr]),
    "int8_linear_forward_zeropoint": (c_int, [c_ptr, c_i64, c_i64, c_ptr, c_ptr, c_ptr, c_i64,
                                              c_ptr, c_float, c_ptr, c_ptr, c_size, c_i64, c_ptr]),
    "int8_linear_forward_fp16w": (c_int, [c_ptr, c_i64, c_i64, c_ptr, c_i64, c_ptr, c_float,
                                          c_ptr, c_ptr, c_ptr, c_ptr, c_size, c_i64, c_ptr]),
    "int8_linear_status": (c_int, [c_ptr, ctypes.POINTER(ctypes.c_int32), c_ptr]),
    "int8_find_outliers": (c_int, [c_ptr, c_i64, c_i64, c_float, c_ptr, c_ptr, c_ptr, c_i64,
                                   c_ptr]),
    "int8_quantize_rows": (c_int, [c_ptr, c_i64, c_i64, c_ptr, c_i64, c_ptr, c_i64, c_ptr,
                                   c_ptr, c_i64, c_ptr]),
    "int8_outlier_weights": (c_int, [c_ptr, c_ptr, c_i64, c_i64, c_ptr, c_i64, c_ptr, c_i64,
                                     c_ptr]),
    "int8_gemm_s32": (c_int, [c_ptr, c_i64, c_ptr, c_i64, c_ptr, c_i64, c_i64, c_i64, c_ptr]),
    "i8mm_profile_enable": (c_int, [c_int]),
    "i8mm_profile_read": (c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_i64)]),
}

# I8MM_NOALLOC_SCRATCH_BYTES: the per-GPU array of the allocation-free forward
NOALLOC_SCRATCH_BYTES = 64 << 20

STATUS = {0: "I8MM_OK", 1: "I8MM_ERR_INVALID_ARG", 2: "I8MM_ERR_WORKSPACE",
          3: "I8MM_ERR_UNSUPPORTED", 4: "I8MM_ERR_HIP", 5: "I8MM_ERR_OUTLIER_OVERFLOW"}


class I8mmError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m int8_mixed_precision_detect_amd.build` (there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(fn: str, code: int) -> None:
    if code != 0:
        raise I8mmError(fn, code)
