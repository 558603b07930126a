"""Pins of the CPU oracle to facts fixed outside it (runs without a GPU).

Each test checks the oracle against something other than itself: the OCP
E2M1 table (tests/golden), torch's float8_e4m3fn and float32->bfloat16
conversions, the scale layout written as a tensor reshape, binary64 matmuls,
exact rational brute force, closed forms and special cases.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (
    bf16_bits_to_f64, bits_fraction, dequant_reference, e2m1_golden, e4m3_torch,
    f32_to_bf16_bits_torch, nearest_bf16_bits, silu_np, swizzle_by_reshape,
    ulp_bf16, unswizzle_by_reshape,
)


def _bits(v: float) -> int:
    return oracle.bf16_from_f64(v)


# ------------------------------------------------------------------ tables
def test_e2m1_table_matches_ocp_mx_spec():
    want = e2m1_golden()
    for c in range(16):
        got = oracle.e2m1_value(c)
        assert got == want[c] and math.copysign(1, got) == math.copysign(1, want[c]), c


def test_e2m1_codes_with_sign_bit_are_negatives():
    for c in range(8):
        assert oracle.e2m1_value(c | 8) == -oracle.e2m1_value(c)
        assert math.copysign(1, oracle.e2m1_value(c | 8)) == -1.0


def test_e4m3_table_matches_torch_float8_e4m3fn():
    want = e4m3_torch()
    for b in range(256):
        got = oracle.e4m3_value(b)
        if math.isnan(want[b]):
            assert math.isnan(got), hex(b)
        else:
            assert got == want[b] and math.copysign(1, got) == math.copysign(1, want[b]), hex(b)
    nan_codes = [b for b in range(256) if math.isnan(oracle.e4m3_value(b))]
    assert nan_codes == [0x7F, 0xFF]
    assert oracle.e4m3_value(0x7E) == 448.0


def test_config_scale_codes_are_the_finite_positive_values_in_range():
    vals = e4m3_torch()
    in_range = [b for b in range(256) if 2.0 ** -4 <= vals[b] <= 2.0 ** 4]
    assert in_range == list(range(synth.SCALE_CODE_LO, synth.SCALE_CODE_HI + 1))
    assert len(in_range) == 65


# ------------------------------------------------------------------ rounding
def test_bf16_rounding_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    # keep values whose rounding cannot overflow the BF16 range
    vals = vals[np.abs(vals) < 3.38e38]
    extra = np.array([1.0, -1.0, 0.0, -0.0, 1.00390625, 1.01171875, 2.0 ** -133, 1.5 * 2.0 ** -133,
                      2.0 ** -126, 3.0 * 2.0 ** -134, 65504.0, 1e-40, -1e-40], np.float32)
    vals = np.concatenate([vals, extra])
    want = f32_to_bf16_bits_torch(vals)
    got = np.array([_bits(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, want)


def test_bf16_rounding_is_direct_from_binary64():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0.
    assert _bits(1.0 + 2.0 ** -8) == 0x3F80
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: even -> 1 + 2^-6.
    assert _bits(1.0 + 3 * 2.0 ** -8) == 0x3F82
    # Just above a tie rounds up; a float32 detour would have landed on the tie.
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert np.float32(v) == np.float32(1.0 + 2.0 ** -8)
    assert _bits(v) == 0x3F81
    assert _bits(-v) == 0xBF81
    # Overflow to infinity at and above max + half ulp.
    max_bf16 = 255.0 * 2.0 ** 120
    assert _bits(max_bf16) == 0x7F7F
    assert _bits(max_bf16 + 2.0 ** 119) == 0x7F80
    assert _bits(max_bf16 + 2.0 ** 119 - 2.0 ** 80) == 0x7F7F
    assert _bits(-1e300) == 0xFF80
    # Subnormal ties: 1.5 * 2^-133 -> 2 * 2^-133 (even), 0.5 * 2^-133 -> 0.
    assert _bits(1.5 * 2.0 ** -133) == 0x0002
    assert _bits(0.5 * 2.0 ** -133) == 0x0000
    assert _bits(-0.5 * 2.0 ** -133) == 0x8000
    assert _bits(0.5 * 2.0 ** -133 + 2.0 ** -180) == 0x0001
    assert _bits(float("nan")) & 0x7FC0 == 0x7FC0


# ------------------------------------------------------------------ layout
def test_scale_buffer_size_formula():
    assert oracle.scale_bytes(256, 512) == 8192
    assert oracle.scale_bytes(4096, 4096) == 1048576
    assert oracle.scale_bytes(6144, 4096) == 1572864
    assert oracle.scale_bytes(28672, 4096) == 7340032
    assert oracle.scale_bytes(3072, 4096) == 786432
    assert oracle.scale_bytes(4096, 1536) == 393216
    assert oracle.scale_bytes(16, 64) == 512
    assert oracle.scale_bytes(130, 80) == 256 * 8
    for n, k in [(256, 512), (4096, 4096), (16, 64), (130, 80)]:
        assert oracle.scale_bytes(n, k) == synth.flat_scale_bytes(n, k)


def test_scale_offsets_of_the_128x4_tile():
    k = 4096  # 256 scale columns, 64 column groups
    assert oracle.scale_offset(0, 0, k) == 0
    assert oracle.scale_offset(0, 1, k) == 1
    assert oracle.scale_offset(0, 3, k) == 3
    assert oracle.scale_offset(0, 4, k) == 512            # next 4-column group
    assert oracle.scale_offset(1, 0, k) == 16             # next 16-byte chunk
    assert oracle.scale_offset(31, 0, k) == 31 * 16
    assert oracle.scale_offset(32, 0, k) == 4             # rows 32 apart share a chunk
    assert oracle.scale_offset(96, 2, k) == 12 + 2
    assert oracle.scale_offset(128, 0, k) == 64 * 512     # next 128-row band


@pytest.mark.parametrize("n,k", [(128, 64), (256, 512), (16, 64), (48, 208), (130, 80), (384, 1536)])
def test_swizzle_matches_the_reshape_layout_and_round_trips(n, k):
    rng = np.random.default_rng(n * 1000 + k)
    logical = rng.integers(0, 256, size=(n, k // 16), dtype=np.uint8)
    flat = oracle.swizzle_scales(logical, n, k)
    assert flat.size == oracle.scale_bytes(n, k)
    assert np.array_equal(flat, swizzle_by_reshape(logical, n, k))
    assert np.array_equal(oracle.unswizzle_scales(flat, n, k), logical)
    assert np.array_equal(unswizzle_by_reshape(flat, n, k), logical)
    # every logical position maps to a distinct in-range byte
    offs = {oracle.scale_offset(r, c, k) for r in range(n) for c in range(k // 16)}
    assert len(offs) == n * (k // 16)
    assert max(offs) < flat.size


# ------------------------------------------------------------------ dequant
def _all_pairs_weight():
    """16 rows x 4096: every block holds codes 0..15 in order, and every row
    walks through all 256 scale codes (NaN scales included)."""
    n, k = 16, 4096
    codes = np.tile(np.arange(16, dtype=np.uint8), (n, k // 16))
    w = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    logical = ((np.arange(k // 16)[None, :] + 16 * np.arange(n)[:, None]) % 256).astype(np.uint8)
    return n, k, w, logical


def test_dequant_all_code_scale_pairs_exact_against_torch():
    n, k, w, logical = _all_pairs_weight()
    flat = swizzle_by_reshape(logical, n, k)
    got, inexact = oracle.dequantize_rows(w, flat, n, k)
    assert inexact == 0
    # torch: e2m1 (golden, exact in f32) * e4m3 (torch) in float32 -> bf16
    ref64 = dequant_reference(w, flat, n, k)
    want = f32_to_bf16_bits_torch(ref64.astype(np.float32))
    finite = ~np.isnan(ref64)
    assert np.array_equal(got[finite], want[finite])
    assert np.isnan(bf16_bits_to_f64(got[~finite])).all()
    # exactness: the BF16 value equals the binary64 product
    assert np.array_equal(bf16_bits_to_f64(got[finite]), ref64[finite])
    # negative zero: code 8 times a positive scale
    assert got[0, 8] == 0x8000 and got[0, 0] == 0x0000


def test_dequant_low_nibble_is_even_k():
    n, k = 16, 64
    w = np.zeros((n, k // 2), np.uint8)
    w[3, 5] = 0x72  # k = 10 -> code 2 (1.0); k = 11 -> code 7 (6.0)
    flat = swizzle_by_reshape(np.full((n, k // 16), 0x38, np.uint8), n, k)  # scale 1.0
    got, _ = oracle.dequantize_rows(w, flat, n, k)
    vals = bf16_bits_to_f64(got)
    assert vals[3, 10] == 1.0 and vals[3, 11] == 6.0
    vals[3, 10] = vals[3, 11] = 0.0
    assert not vals.any()


# ------------------------------------------------------------------ GEMV
@pytest.mark.parametrize("m,n,k", [(1, 256, 512), (3, 48, 128), (5, 160, 320), (2, 128, 64)])
def test_gemv_accumulator_matches_binary64_matmul(m, n, k):
    d = synth.dense_w4a16(m, n, k, seed=11 + m + n + k)
    out, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n)
    x64 = bf16_bits_to_f64(d["x"].view(torch.uint16).numpy())
    wd = dequant_reference(d["w"].numpy(), d["s"].numpy(), n, k)
    ref = x64 @ wd.T
    assert np.all(np.abs(acc - ref) <= 4 * k * 2.0 ** -52 * absacc)
    assert np.allclose(absacc, np.abs(x64) @ np.abs(wd).T, rtol=1e-12, atol=0)
    # the output is the BF16 value nearest to acc * gs
    gs = float(d["gs"][0])
    got = bf16_bits_to_f64(out)
    assert np.all(np.abs(got - ref * gs) <= 0.5 * ulp_bf16(got) * (1 + 1e-9) + 1e-300)


def _exact_gemv_bits(x_bits, wd, gs, silu_mul=False):
    m, k = x_bits.shape
    n = wd.shape[0]
    xf = [[bits_fraction(b) for b in row] for row in x_bits]
    wf = [[Fraction(float(v)) for v in row] for row in wd]
    acc = [[sum((xf[i][kk] * wf[j][kk] for kk in range(k)), Fraction(0)) for j in range(n)]
           for i in range(m)]
    g = Fraction(gs)
    if not silu_mul:
        return np.array([[nearest_bf16_bits(acc[i][j] * g) for j in range(n)] for i in range(m)],
                        np.uint16), acc
    return None, acc


def test_gemv_exact_rational_brute_force():
    m, n, k = 2, 32, 64  # ragged N (< 128 rows): padding rows in the scale tile
    d = synth.dense_w4a16(m, n, k, seed=5)
    gs = 0.3  # not a power of two: the product with the accumulator must round once
    out, _, _ = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], gs, n)
    wd = dequant_reference(d["w"].numpy(), d["s"].numpy(), n, k)
    want, _ = _exact_gemv_bits(d["x"].view(torch.uint16).numpy(), wd, float(np.float32(gs)))
    assert np.array_equal(out, want)


def test_gemv_all_ones_weight_is_scaled_row_sum():
    m, n, k = 3, 128, 256
    d = synth.dense_w4a16(m, n, k, seed=3)
    w = np.full((n, k // 2), 0x22, np.uint8)      # both nibbles code 2 = 1.0
    flat = np.full(oracle.scale_bytes(n, k), 0x38, np.uint8)  # E4M3 1.0
    out, _, _ = oracle.nvfp4_gemv(d["x"], w, flat, 1 / 64, n)
    x64 = bf16_bits_to_f64(d["x"].view(torch.uint16).numpy())
    rowsum = np.array([math.fsum(r) for r in x64]) / 64
    got = bf16_bits_to_f64(out)
    for i in range(m):
        assert np.all(got[i] == got[i, 0])
        assert abs(got[i, 0] - rowsum[i]) <= 0.5 * ulp_bf16(got[i, 0])


def test_gemv_one_hot_weight_is_one_exact_product():
    m, n, k = 2, 128, 128
    d = synth.dense_w4a16(m, n, k, seed=9)
    w = np.zeros((n, k // 2), np.uint8)
    w[77, 20] = 0x0E  # k = 40 -> code 14 (-4.0); k = 41 -> code 0
    logical = np.full((n, k // 16), 0x38, np.uint8)
    logical[77, 2] = 0x4B  # block k // 16 = 2: 2^2 * 1.375 = 5.5
    flat = swizzle_by_reshape(logical, n, k)
    out, _, _ = oracle.nvfp4_gemv(d["x"], w, flat, 1 / 64, n)
    x64 = bf16_bits_to_f64(d["x"].view(torch.uint16).numpy())
    got = bf16_bits_to_f64(out)
    for i in range(m):
        want = x64[i, 40] * -4.0 * 5.5 / 64
        assert abs(got[i, 77] - want) <= 0.5 * ulp_bf16(want)
        others = np.delete(got[i], 77)
        assert not others.any()


def test_silu_mul_pairs_gate_and_up_halves():
    m, n, k = 2, 256, 128
    d = synth.dense_w4a16(m, n, k, seed=21)
    gs = float(d["gs"][0])
    full, _, _ = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], gs, n)
    fused, _, _ = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], gs, n, silu_mul=True)
    assert fused.shape == (m, n // 2)
    g = bf16_bits_to_f64(full[:, : n // 2])
    u = bf16_bits_to_f64(full[:, n // 2:])
    ref = torch.nn.functional.silu(torch.from_numpy(g)).numpy() * u
    got = bf16_bits_to_f64(fused)
    assert np.all(np.abs(got - ref) <= 0.5 * ulp_bf16(got) * (1 + 1e-9) + 1e-300)
    # closed forms of SiLU
    assert silu_np(0.0) == 0.0


def test_bf16_gemv_matches_torch_matmul():
    m, n, k = 4, 96, 320
    d = synth.dense_bf16(m, n, k, seed=4)
    out, acc, absacc = oracle.bf16_gemv(d["x"], d["w"])
    ref = (d["x"].double() @ d["w"].double().T).numpy()
    assert np.all(np.abs(acc - ref) <= 4 * k * 2.0 ** -52 * absacc)
    ref32 = (d["x"].float() @ d["w"].float().T).numpy().astype(np.float64)
    got = bf16_bits_to_f64(out)
    assert np.all(np.abs(got - ref32) <= ulp_bf16(ref) + 2 * k * 2.0 ** -24 * absacc)


def test_bf16_gemv_exact_rational_brute_force():
    m, n, k = 2, 16, 48
    d = synth.dense_bf16(m, n, k, seed=8)
    out, _, _ = oracle.bf16_gemv(d["x"], d["w"])
    wd = bf16_bits_to_f64(d["w"].view(torch.uint16).numpy())
    want, _ = _exact_gemv_bits(d["x"].view(torch.uint16).numpy(), wd, 1.0)
    assert np.array_equal(out, want)


# ------------------------------------------------------------------ MoE
def _tiny_moe(m=3, e=4, topk=2, h=64, inter=32, si=32, seed=17, dup=False):
    wts = synth.moe_weights(e, h, inter, si, seed)
    tok = synth.moe_tokens(m, h, e, topk, seed + 1)
    if dup:
        tok["ids"][0, :] = tok["ids"][0, 0]
    return wts, tok


def test_moe_gate_up_matches_binary64_reference():
    wts, tok = _tiny_moe()
    r = oracle.moe_gate_up(tok["x"], tok["ids"], wts["w1"], wts["w1_sf"], wts["alpha"],
                           wts["wsh"], wts["ssh"], wts["gssh"])
    x64 = bf16_bits_to_f64(tok["x"].view(torch.uint16).numpy())
    ids = tok["ids"].numpy()
    m, topk = ids.shape
    inter = wts["w1"].shape[1] // 2
    h = x64.shape[1]
    for p in range(m * topk):
        t, e = p // topk, ids.reshape(-1)[p]
        wd = dequant_reference(wts["w1"][e].numpy(), wts["w1_sf"][e].numpy(), 2 * inter, h)
        acc = wd @ x64[t]
        g = acc[:inter] * float(wts["alpha"][e])
        u = acc[inter:] * float(wts["alpha"][e])
        ref = silu_np(g) * u
        got = bf16_bits_to_f64(r["act"][p])
        assert np.all(np.abs(got - ref) <= 0.5 * ulp_bf16(got) * (1 + 1e-9) + 2.0 ** -140), p
    # shared expert equals the dense fused GEMV on the shared weights
    dense, _, _ = oracle.nvfp4_gemv(tok["x"], wts["wsh"], wts["ssh"], float(wts["gssh"][0]),
                                    wts["wsh"].shape[0], silu_mul=True)
    assert np.array_equal(r["sact"], dense)


def test_moe_down_combine_exact_rational_brute_force():
    wts, tok = _tiny_moe(m=2, e=4, topk=3, h=32, inter=32, si=48, seed=23)
    gu = oracle.moe_gate_up(tok["x"], tok["ids"], wts["w1"], wts["w1_sf"], wts["alpha"],
                            wts["wsh"], wts["ssh"], wts["gssh"])
    r = oracle.moe_down_combine(gu["act"], tok["ids"], tok["tw"], wts["w2"], wts["w2_sf"],
                                wts["alpha2"], gu["sact"], wts["wsd"], wts["ssd"], wts["gssd"])
    ids = tok["ids"].numpy()
    tw = tok["tw"].numpy()
    m, topk = ids.shape
    h = wts["w2"].shape[1]
    inter = wts["w2"].shape[2] * 2
    si = wts["wsd"].shape[1] * 2
    wsd = dequant_reference(wts["wsd"].numpy(), wts["ssd"].numpy(), h, si)
    gssd = Fraction(float(wts["gssd"][0]))
    for t in range(m):
        sact_f = [bits_fraction(b) for b in gu["sact"][t]]
        for hh in range(h):
            s = Fraction(0)
            for j in range(topk):
                p = t * topk + j
                e = ids[t, j]
                w2 = dequant_reference(wts["w2"][e].numpy(), wts["w2_sf"][e].numpy(), h, inter)[hh]
                a = sum((bits_fraction(gu["act"][p][kk]) * Fraction(float(w2[kk])) for kk in range(inter)),
                        Fraction(0))
                y = bits_fraction(nearest_bf16_bits(a * Fraction(float(wts["alpha2"][e]))))
                s += Fraction(float(tw[t, j])) * y
            a = sum((sact_f[kk] * Fraction(float(wsd[hh, kk])) for kk in range(si)), Fraction(0))
            ysh = bits_fraction(nearest_bf16_bits(a * gssd))
            want = nearest_bf16_bits(bits_fraction(nearest_bf16_bits(s)) + ysh)
            assert r["out"][t, hh] == want, (t, hh)


def test_moe_top1_unit_weight_zero_shared_reduces_to_dense_gemv():
    wts, tok = _tiny_moe(m=2, e=3, topk=1, h=64, inter=64, si=32, seed=31)
    tok["tw"][:] = 1.0
    wts["wsd"][:] = 0  # all codes +0
    gu = oracle.moe_gate_up(tok["x"], tok["ids"], wts["w1"], wts["w1_sf"], wts["alpha"],
                            wts["wsh"], wts["ssh"], wts["gssh"])
    r = oracle.moe_down_combine(gu["act"], tok["ids"], tok["tw"], wts["w2"], wts["w2_sf"],
                                wts["alpha2"], gu["sact"], wts["wsd"], wts["ssd"], wts["gssd"])
    for t in range(2):
        e = int(tok["ids"][t, 0])
        dense, _, _ = oracle.nvfp4_gemv(gu["act"][t:t + 1], wts["w2"][e], wts["w2_sf"][e],
                                        float(wts["alpha2"][e]), wts["w2"].shape[1])
        assert np.array_equal(r["out"][t], dense[0])


def test_moe_duplicate_ids_count_each_slot():
    wts, tok = _tiny_moe(m=1, e=4, topk=2, h=64, inter=32, si=32, seed=41, dup=True)
    tok["tw"][:] = torch.tensor([[0.25, 0.75]])
    gu = oracle.moe_gate_up(tok["x"], tok["ids"], wts["w1"], wts["w1_sf"], wts["alpha"],
                            wts["wsh"], wts["ssh"], wts["gssh"])
    assert np.array_equal(gu["act"][0], gu["act"][1])
    wts["wsd"][:] = 0
    r = oracle.moe_down_combine(gu["act"], tok["ids"], tok["tw"], wts["w2"], wts["w2_sf"],
                                wts["alpha2"], gu["sact"], wts["wsd"], wts["ssd"], wts["gssd"])
    e = int(tok["ids"][0, 0])
    dense, _, _ = oracle.nvfp4_gemv(gu["act"][0:1], wts["w2"][e], wts["w2_sf"][e],
                                    float(wts["alpha2"][e]), wts["w2"].shape[1])
    # 0.25 y + 0.75 y = y exactly
    assert np.array_equal(r["out"][0], dense[0])


# ------------------------------------------------------------------ planted mistakes
def test_pins_detect_planted_mistakes():
    """The pins above reject plausible mistakes: a swapped nibble order, a
    transposed swizzle tile and a dropped sign all change the result."""
    n, k, w, logical = _all_pairs_weight()
    flat = swizzle_by_reshape(logical, n, k)
    good, _ = oracle.dequantize_rows(w, flat, n, k)
    swapped = ((w >> 4) | (w << 4)).astype(np.uint8)
    bad, _ = oracle.dequantize_rows(swapped, flat, n, k)
    assert not np.array_equal(good, bad)
    # a (r % 32, r // 32) transposition of the tile is a different layout
    t = logical.copy()
    alt = np.zeros_like(flat)
    for r in range(n):
        for c in range(k // 16):
            alt[(c // 4) * 512 + (r // 32) * 16 + (r % 32) * 4 + c % 4] = t[r, c]
    assert not np.array_equal(alt, flat)
    assert not np.array_equal(unswizzle_by_reshape(alt, n, k), logical)
