"""Test-side helpers: independent references used to pin the oracle, BF16 bit
handling, and the acceptance bounds used by the GPU parity tests.

The references here do NOT reuse the oracle's code: element values come from
the OCP table in tests/golden and from torch's float8_e4m3fn conversion, the
scale layout is written as a tensor reshape/transpose, sums use numpy/torch
binary64 matmuls or exact rationals, and rounding to BF16 picks the nearest
BF16 value by exact rational comparison.
"""
from __future__ import annotations

import math
import os
import struct
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- elements
def e2m1_golden() -> np.ndarray:
    vals = np.zeros(16, np.float64)
    with open(os.path.join(GOLDEN, "e2m1_ocp_mx_v1.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return vals


def e4m3_torch() -> np.ndarray:
    """All 256 E4M3FN byte values via torch's own float8_e4m3fn conversion."""
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return b.view(torch.float8_e4m3fn).to(torch.float32).to(torch.float64).numpy()


# ---------------------------------------------------------------- bf16 bits
def bf16_bits_to_f64(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_bf16_bits_torch(v) -> np.ndarray:
    """torch's float32 -> bfloat16 conversion (round to nearest even)."""
    t = torch.as_tensor(np.asarray(v, np.float32))
    return t.to(torch.bfloat16).view(torch.uint16).numpy()


def to_bits(t) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor/array."""
    if isinstance(t, torch.Tensor):
        return t.detach().cpu().contiguous().view(torch.uint16).numpy()
    return np.asarray(t, np.uint16)


def nearest_bf16_bits(v: Fraction) -> int:
    """BF16 bit pattern nearest to the rational v (ties to even mantissa),
    chosen by exact comparison among neighbouring candidates.  Finite range
    only (the tests never reach overflow)."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = -v if v < 0 else v
    f = float(a)
    base = struct.unpack("<I", struct.pack("<f", f))[0] >> 16
    best, best_d = None, None
    for cand in (base - 1, base, base + 1, base + 2):
        if cand < 0 or cand >= 0x7F80:
            continue
        cv = Fraction(struct.unpack("<f", struct.pack("<I", cand << 16))[0])
        d = abs(cv - a)
        if best is None or d < best_d or (d == best_d and cand % 2 == 0):
            best, best_d = cand, d
    return sign | best


def bits_fraction(bits: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0])


# ---------------------------------------------------------------- layout
def unswizzle_by_reshape(flat, n: int, k: int) -> np.ndarray:
    """Logical [n, k/16] scales from the flat 128x4 buffer, written as a view
    change: the buffer is [row bands, column groups, 32, 4, 4] =
    (band, group, r % 32, r // 32, column-in-group); bring it back to
    [band, r // 32, r % 32, group, column-in-group] = [rows, columns]."""
    flat = np.asarray(flat, np.uint8).reshape(-1)
    cp = (k // 16 + 3) // 4 * 4
    npad = (n + 127) // 128 * 128
    t = flat[: npad * cp].reshape(npad // 128, cp // 4, 32, 4, 4)
    t = t.transpose(0, 3, 2, 1, 4).reshape(npad, cp)
    return np.ascontiguousarray(t[:n, : k // 16])


def swizzle_by_reshape(logical, n: int, k: int) -> np.ndarray:
    logical = np.asarray(logical, np.uint8).reshape(n, k // 16)
    cp = (k // 16 + 3) // 4 * 4
    npad = (n + 127) // 128 * 128
    padded = np.zeros((npad, cp), np.uint8)
    padded[:n, : k // 16] = logical
    t = padded.reshape(npad // 128, 4, 32, cp // 4, 4).transpose(0, 3, 2, 1, 4)
    return np.ascontiguousarray(t).reshape(-1)


# ---------------------------------------------------------------- references
def dequant_reference(w, flat, n: int, k: int) -> np.ndarray:
    """binary64 [n, k] dequantized weights: golden E2M1 x torch E4M3, low
    nibble = even k, scale of block k // 16 read through the reshape layout."""
    w = np.asarray(w, np.uint8).reshape(n, k // 2)
    codes = np.empty((n, k), np.int64)
    codes[:, 0::2] = w & 15
    codes[:, 1::2] = w >> 4
    sc = unswizzle_by_reshape(flat, n, k)
    scale = e4m3_torch()[sc.astype(np.int64)]
    return e2m1_golden()[codes] * np.repeat(scale, 16, axis=1)


# ---------------------------------------------------------------- bounds
def ulp_bf16(v) -> np.ndarray:
    """Spacing of BF16 numbers at |v|: 2^(max(floor(log2|v|), -126) - 7)
    (infinite for infinite or NaN v: such values are compared exactly)."""
    a = np.abs(np.asarray(v, np.float64))
    fin = np.isfinite(a)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where((a > 0) & fin, a, 1.0)))
    e = np.where(a > 0, np.maximum(e, -126), -126)
    return np.where(fin, np.ldexp(1.0, (e - 7).astype(np.int64)), np.inf)


def gemv_bound(ref_value, absacc, gs) -> np.ndarray:
    """Acceptance bound of a GEMV output: one BF16 ulp of the oracle's
    binary64 value plus 1e-3 * sum|x*w| * |global scale|."""
    return ulp_bf16(ref_value) + 1e-3 * np.abs(absacc) * abs(float(gs))


def fp32_order_bound(ref_value, absacc, gs, k: int) -> np.ndarray:
    """Tighter bound that any FP32 summation order satisfies (twice the
    worst-case gamma_K of recursive summation): one ulp + 2 K 2^-24 sum|x*w| |gs|."""
    return ulp_bf16(ref_value) + 2.0 * k * 2.0 ** -24 * np.abs(absacc) * abs(float(gs))


def silu_np(g):
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def silu_bound(out_ref, g, u, bg, bu) -> np.ndarray:
    """Bound for bf16(silu(g) * u) when g and u are each off by at most bg,
    bu: 2 ulp(out) + 1.1 |u| bg + (|silu(g)| + 1.1 bg) bu (|silu'| <= 1.1)."""
    return (2.0 * ulp_bf16(out_ref) + 1.1 * np.abs(u) * bg
            + (np.abs(silu_np(g)) + 1.1 * bg) * bu)


def assert_close_bits(got_bits, want_bits, bound, what: str, nan_ok: bool = False):
    got = bf16_bits_to_f64(got_bits)
    want = bf16_bits_to_f64(want_bits)
    same = (np.isnan(got) & np.isnan(want)) | (got == want)   # includes equal infinities
    with np.errstate(invalid="ignore"):
        diff = np.where(same, 0.0, np.abs(got - want))
    bad = ~(diff <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:8]
        lines = [f"{what}: {int(bad.sum())} of {bad.size} outside the bound"]
        for i in idx:
            i = tuple(i)
            lines.append(f"  at {i}: got {got[i]!r} want {want[i]!r} bound {np.asarray(bound)[i] if np.ndim(bound) else bound!r}")
        raise AssertionError("\n".join(lines))
    return float(np.max(diff / np.maximum(bound, 1e-300))) if diff.size else 0.0


def math_fsum_rows(x: np.ndarray) -> np.ndarray:
    return np.array([math.fsum(r) for r in x])


# ---------------------------------------------------------------- checks used by the GPU parity tests
def check_gemv(gpu_bits, acc, absacc, gs, k, what):
    """GPU BF16 GEMV output against the oracle's binary64 accumulator: the
    acceptance bound (one ulp + 1e-3 sum|xw| |gs|) and the tighter bound every
    FP32 summation order meets.  Returns the worst |diff| / tight bound."""
    ref = acc * float(gs)
    got = bf16_bits_to_f64(gpu_bits)
    diff = np.abs(got - ref)
    bad = ~(diff <= gemv_bound(ref, absacc, gs))
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} outside the acceptance bound; "
                             f"first at {i}: got {got[i]!r} oracle {ref[i]!r}")
    tight = fp32_order_bound(ref, absacc, gs, k)
    bad = ~(diff <= tight)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} outside the FP32-order bound; "
                             f"first at {i}: got {got[i]!r} oracle {ref[i]!r}")
    return float(np.max(diff / tight)) if diff.size else 0.0


def check_silu(gpu_bits, oracle_bits, acc, absacc, gs, what, rounded_gate_up=True):
    """GPU bf16(silu(g) * u) against the oracle, with the GEMV error of g and u
    (rows j and H + j of acc) propagated through silu(g) * u."""
    h = acc.shape[1] // 2
    g_ref = acc[:, :h] * float(gs)
    u_ref = acc[:, h:] * float(gs)
    if rounded_gate_up:
        bg = 1.5 * ulp_bf16(g_ref) + 1e-3 * float(gs) * absacc[:, :h]
        bu = 1.5 * ulp_bf16(u_ref) + 1e-3 * float(gs) * absacc[:, h:]
    else:
        bg = 1e-3 * abs(float(gs)) * absacc[:, :h]
        bu = 1e-3 * abs(float(gs)) * absacc[:, h:]
    want = bf16_bits_to_f64(oracle_bits)
    bound = silu_bound(want, g_ref, u_ref, bg, bu)
    return assert_close_bits(gpu_bits, oracle_bits, bound, what)


def check_routed_act(gpu_bits, oracle_bits, acc_r, abs_r, alpha_per_pair, what):
    """Routed gate_up output: g, u are FP32 accumulators times alpha (not rounded)."""
    h = acc_r.shape[1] // 2
    a = np.asarray(alpha_per_pair, np.float64)[:, None]
    g_ref = acc_r[:, :h] * a
    u_ref = acc_r[:, h:] * a
    bg = 1e-3 * a * abs_r[:, :h] + 2.0 ** -126
    bu = 1e-3 * a * abs_r[:, h:] + 2.0 ** -126
    want = bf16_bits_to_f64(oracle_bits)
    return assert_close_bits(gpu_bits, oracle_bits, silu_bound(want, g_ref, u_ref, bg, bu), what)


def check_down(gpu_bits, oracle_bits, acc_r, abs_r, acc_s, abs_s, tw, alpha2_per_slot, gssd, what):
    """down_combine: out = bf16(bf16(sum_j tw_j y_j) + y_sh); the bound adds the
    propagated GEMV bounds of every y_j and of y_sh, the rounding of the sum and
    the FP32 error of the weighted sum."""
    a2 = np.asarray(alpha2_per_slot, np.float64)[:, :, None]     # [M, topk, 1]
    twv = np.asarray(tw, np.float64)[:, :, None]
    y_ref = acc_r * a2
    b_y = 1.5 * ulp_bf16(y_ref) + 1e-3 * a2 * abs_r
    s_ref = np.sum(twv * y_ref, axis=1)
    ysh_ref = acc_s * float(gssd)
    b_sh = 1.5 * ulp_bf16(ysh_ref) + 1e-3 * float(gssd) * abs_s
    want = bf16_bits_to_f64(oracle_bits)
    bound = (2 * ulp_bf16(want) + 1.5 * ulp_bf16(s_ref) + np.sum(np.abs(twv) * b_y, axis=1)
             + b_sh + 2.0 ** -22 * np.sum(np.abs(twv * y_ref), axis=1))
    return assert_close_bits(gpu_bits, oracle_bits, bound, what)
