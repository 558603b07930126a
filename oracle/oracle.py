"""ctypes front end of the binary64 CPU oracle (test infrastructure only).

Every function takes and returns numpy arrays; BF16 tensors are carried as
their uint16 bit patterns.  No arithmetic of the method happens here: each
call forwards to ``nvfp4_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# A different build of the oracle (the mutation tests compile deliberately
# broken copies) can be selected with W4A16_ORACLE_LIB.
_LIB_PATH = os.environ.get("W4A16_ORACLE_LIB") or os.path.join(_HERE, "liboracle_nvfp4.so")
_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build_oracle

        build_oracle.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_e2m1_value.argtypes = [ctypes.c_int]
    lib.oracle_e2m1_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_int]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_bf16_from_f64.argtypes = [ctypes.c_double]
    lib.oracle_bf16_from_f64.restype = ctypes.c_uint16
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_scale_bytes.argtypes = [_i64, _i64]
    lib.oracle_scale_bytes.restype = _i64
    lib.oracle_scale_offset.argtypes = [_i64, _i64, _i64]
    lib.oracle_scale_offset.restype = _i64
    lib.oracle_swizzle_scales.argtypes = [_u8p, _i64, _i64, _u8p]
    lib.oracle_unswizzle_scales.argtypes = [_u8p, _i64, _i64, _u8p]
    lib.oracle_dequantize_rows.argtypes = [_u8p, _u8p, _i64, _i64, _u16p]
    lib.oracle_dequantize_rows.restype = _i64
    lib.oracle_nvfp4_gemv.argtypes = [
        _u16p, _i64, _i64, _i64, _u8p, _u8p, ctypes.c_float, _i64, ctypes.c_int,
        _u16p, _f64p, _f64p,
    ]
    lib.oracle_bf16_gemv.argtypes = [
        _u16p, _i64, _i64, _i64, _u16p, _i64, ctypes.c_int, _u16p, _f64p, _f64p,
    ]
    lib.oracle_moe_gate_up.argtypes = [
        _u16p, _i64, _i64, _i32p, _i64, _u8p, _u8p, _f32p, _i64, _u16p,
        _u8p, _u8p, _f32p, _i64, _u16p, _f64p, _f64p, _f64p, _f64p,
    ]
    lib.oracle_moe_down_combine.argtypes = [
        _u16p, _i32p, _f32p, _i64, _i64, _u8p, _u8p, _f32p, _i64, _i64,
        _u16p, _u8p, _u8p, _f32p, _i64, _u16p, _f64p, _f64p, _f64p, _f64p,
    ]
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray, typ):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(typ)


def _arr(a, dtype) -> np.ndarray:
    """Host numpy view of an array-like (numpy array or CPU torch tensor)."""
    if hasattr(a, "numpy"):
        import torch

        if a.dtype == torch.bfloat16:
            a = a.view(torch.uint16) if hasattr(torch, "uint16") else a.view(torch.int16)
        a = a.detach().cpu().contiguous().numpy()
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        a = a.view(dtype) if a.dtype.itemsize == np.dtype(dtype).itemsize else a.astype(dtype)
    return a


def set_threads(n: int) -> int:
    """Sets the OpenMP thread count of the oracle; returns the count in use."""
    return _load().oracle_set_threads(int(n))


def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return _load().oracle_e4m3_value(int(byte))


def bf16_from_f64(v: float) -> int:
    return int(_load().oracle_bf16_from_f64(float(v)))


def bf16_to_f64(bits: int) -> float:
    return _load().oracle_bf16_to_f64(int(bits))


def scale_bytes(n: int, k: int) -> int:
    return int(_load().oracle_scale_bytes(n, k))


def scale_offset(n: int, c: int, k: int) -> int:
    return int(_load().oracle_scale_offset(n, c, k))


def swizzle_scales(logical, n: int, k: int) -> np.ndarray:
    logical = _arr(logical, np.uint8).reshape(n, k // 16)
    out = np.empty(scale_bytes(n, k), np.uint8)
    _load().oracle_swizzle_scales(_ptr(logical, _u8p), n, k, _ptr(out, _u8p))
    return out


def unswizzle_scales(flat, n: int, k: int) -> np.ndarray:
    flat = _arr(flat, np.uint8).reshape(-1)
    assert flat.size >= scale_bytes(n, k)
    out = np.empty((n, k // 16), np.uint8)
    _load().oracle_unswizzle_scales(_ptr(flat, _u8p), n, k, _ptr(out, _u8p))
    return out


def dequantize_rows(w, s_flat, rows: int, k: int):
    """Returns (bf16 bits [rows, k], number of inexact products)."""
    w = _arr(w, np.uint8).reshape(rows, k // 2)
    s_flat = _arr(s_flat, np.uint8).reshape(-1)
    out = np.empty((rows, k), np.uint16)
    bad = _load().oracle_dequantize_rows(_ptr(w, _u8p), _ptr(s_flat, _u8p), rows, k, _ptr(out, _u16p))
    return out, int(bad)


def nvfp4_gemv(x, w, s_flat, global_scale: float, n: int, silu_mul: bool = False):
    """Returns (bf16 bits out, acc [M, N] binary64, sum|x*w| [M, N])."""
    w = _arr(w, np.uint8)
    k = w.shape[-1] * 2
    x = np.ascontiguousarray(_arr(x, np.uint16)[:, :k])
    m = x.shape[0]
    s_flat = _arr(s_flat, np.uint8).reshape(-1)
    n_out = n // 2 if silu_mul else n
    out = np.empty((m, n_out), np.uint16)
    acc = np.empty((m, n), np.float64)
    absacc = np.empty((m, n), np.float64)
    _load().oracle_nvfp4_gemv(
        _ptr(x, _u16p), m, k, k, _ptr(w, _u8p), _ptr(s_flat, _u8p), float(global_scale),
        n, int(bool(silu_mul)), _ptr(out, _u16p), _ptr(acc, _f64p), _ptr(absacc, _f64p),
    )
    return out, acc, absacc


def bf16_gemv(x, w, silu_mul: bool = False):
    """Returns (bf16 bits out, acc [M, N] binary64, sum|x*w| [M, N])."""
    x = _arr(x, np.uint16)
    w = _arr(w, np.uint16)
    m, k = x.shape
    n = w.shape[0]
    n_out = n // 2 if silu_mul else n
    out = np.empty((m, n_out), np.uint16)
    acc = np.empty((m, n), np.float64)
    absacc = np.empty((m, n), np.float64)
    _load().oracle_bf16_gemv(
        _ptr(x, _u16p), m, k, k, _ptr(w, _u16p), n, int(bool(silu_mul)),
        _ptr(out, _u16p), _ptr(acc, _f64p), _ptr(absacc, _f64p),
    )
    return out, acc, absacc


def moe_gate_up(x, ids, w1, w1_sf, alpha, wsh, ssh, gssh):
    """Returns dict(act, sact, acc_r, abs_r, acc_s, abs_s)."""
    x = _arr(x, np.uint16)
    ids = _arr(ids, np.int32)
    w1 = _arr(w1, np.uint8)
    w1_sf = _arr(w1_sf, np.uint8).reshape(-1)
    alpha = _arr(alpha, np.float32).reshape(-1)
    wsh = _arr(wsh, np.uint8)
    ssh = _arr(ssh, np.uint8).reshape(-1)
    gssh = _arr(gssh, np.float32).reshape(-1)
    m, h = x.shape
    topk = ids.shape[1]
    inter = w1.shape[1] // 2
    si = wsh.shape[0] // 2
    p = m * topk
    act = np.empty((p, inter), np.uint16)
    sact = np.empty((m, si), np.uint16)
    acc_r = np.empty((p, 2 * inter), np.float64)
    abs_r = np.empty((p, 2 * inter), np.float64)
    acc_s = np.empty((m, 2 * si), np.float64)
    abs_s = np.empty((m, 2 * si), np.float64)
    _load().oracle_moe_gate_up(
        _ptr(x, _u16p), m, h, _ptr(ids, _i32p), topk, _ptr(w1, _u8p), _ptr(w1_sf, _u8p),
        _ptr(alpha, _f32p), inter, _ptr(act, _u16p), _ptr(wsh, _u8p), _ptr(ssh, _u8p),
        _ptr(gssh, _f32p), si, _ptr(sact, _u16p), _ptr(acc_r, _f64p), _ptr(abs_r, _f64p),
        _ptr(acc_s, _f64p), _ptr(abs_s, _f64p),
    )
    return dict(act=act, sact=sact, acc_r=acc_r, abs_r=abs_r, acc_s=acc_s, abs_s=abs_s)


def moe_down_combine(act, ids, tw, w2, w2_sf, alpha2, sact, wsd, ssd, gssd):
    """Returns dict(out, acc_r [M, topk, H], abs_r, acc_s [M, H], abs_s)."""
    act = _arr(act, np.uint16)
    ids = _arr(ids, np.int32)
    tw = _arr(tw, np.float32)
    w2 = _arr(w2, np.uint8)
    w2_sf = _arr(w2_sf, np.uint8).reshape(-1)
    alpha2 = _arr(alpha2, np.float32).reshape(-1)
    sact = _arr(sact, np.uint16)
    wsd = _arr(wsd, np.uint8)
    ssd = _arr(ssd, np.uint8).reshape(-1)
    gssd = _arr(gssd, np.float32).reshape(-1)
    m, topk = ids.shape
    h = w2.shape[1]
    inter = w2.shape[2] * 2
    si = wsd.shape[1] * 2
    out = np.empty((m, h), np.uint16)
    acc_r = np.empty((m, topk, h), np.float64)
    abs_r = np.empty((m, topk, h), np.float64)
    acc_s = np.empty((m, h), np.float64)
    abs_s = np.empty((m, h), np.float64)
    _load().oracle_moe_down_combine(
        _ptr(act, _u16p), _ptr(ids, _i32p), _ptr(tw, _f32p), m, topk, _ptr(w2, _u8p),
        _ptr(w2_sf, _u8p), _ptr(alpha2, _f32p), h, inter, _ptr(sact, _u16p), _ptr(wsd, _u8p),
        _ptr(ssd, _u8p), _ptr(gssd, _f32p), si, _ptr(out, _u16p), _ptr(acc_r, _f64p),
        _ptr(abs_r, _f64p), _ptr(acc_s, _f64p), _ptr(abs_s, _f64p),
    )
    return dict(out=out, acc_r=acc_r, abs_r=abs_r, acc_s=acc_s, abs_s=abs_s)


__all__ = [
    "set_threads", "e2m1_value", "e4m3_value", "bf16_from_f64", "bf16_to_f64",
    "scale_bytes", "scale_offset", "swizzle_scales", "unswizzle_scales",
    "dequantize_rows", "nvfp4_gemv", "bf16_gemv", "moe_gate_up", "moe_down_combine",
]
