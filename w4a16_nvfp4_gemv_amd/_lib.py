"""Loader of libw4a16_nvfp4_gemv.so (the HIP library) with its C signatures.

There is no fallback: if the library is missing, every op raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw4a16_nvfp4_gemv.so")

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int

# name -> (restype, argtypes); mirrors include/w4a16_nvfp4_gemv.h
SIGNATURES = {
    "nvfp4_gemv": (_int, [_p, _i64, _i64, _i64, _p, _p, _p, _i64, _int, _p, _p]),
    "bf16_gemv": (_int, [_p, _i64, _i64, _i64, _p, _i64, _int, _p, _p]),
    "gemv_splitk_workspace_bytes": (_i64, [_int, _i64, _i64, _i64, _int]),
    "nvfp4_gemv_splitk": (_int, [_p, _i64, _i64, _i64, _p, _p, _p, _i64, _int, _p, _i64, _p, _p]),
    "bf16_gemv_splitk": (_int, [_p, _i64, _i64, _i64, _p, _i64, _int, _p, _i64, _p, _p]),
    "nvfp4_gemv_splitk_noalloc": (_int, [_p, _i64, _i64, _i64, _p, _p, _p, _i64, _int, _p, _p]),
    "dequantize_rows": (_int, [_p, _p, _i64, _i64, _p, _p]),
    "nvfp4_dequant_gemm_workspace_bytes": (_i64, [_i64, _i64, _i64]),
    "nvfp4_dequant_gemm": (_int, [_p, _i64, _i64, _i64, _p, _p, _p, _i64, _int, _p, _i64, _p, _p]),
    "nvfp4_unswizzle_scales": (_int, [_p, _i64, _i64, _p, _p]),
    "moe_gate_up": (_int, [_p, _i64, _i64, _p, _i64, _i64, _p, _p, _p, _i64, _p, _p, _p, _p, _i64, _p, _p]),
    "moe_down_combine": (_int, [_p, _p, _p, _i64, _i64, _i64, _p, _p, _p, _i64, _i64, _p, _p, _p, _p, _i64, _p, _p]),
    "w4a16_gemv_kernel_name": (ctypes.c_char_p, [_int, _i64, _i64, _i64, _int]),
    "w4a16_gemv_splitk_kernel_name": (ctypes.c_char_p, [_int, _i64, _i64, _i64, _int]),
    "nvfp4_status_string": (ctypes.c_char_p, [_int]),
    "w4a16_status_string": (ctypes.c_char_p, [_int]),
    "w4a16_last_error": (ctypes.c_char_p, []),
}

_lib = None


class LibraryMissing(RuntimeError):
    pass


def load():
    """The loaded library; raises LibraryMissing if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(
            f"{LIB_PATH} is not built: run `python -m w4a16_nvfp4_gemv_amd.build_ext` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
