"""GPU parity: every entry point, called through the C ABI (via the thin Python
binding), against the binary64 CPU oracle on the same seeded host inputs.

Bars: bit-exact for dequantize_rows and the scale un-swizzle; for the GEMVs
one BF16 ulp of the oracle's binary64 value plus 1e-3 * sum|x*w| * |gs| (and
the tighter bound any FP32 summation order meets); propagated bounds for the
SiLU epilogues and the MoE combine (tests/helpers.py).  Full-size shapes are
checked element by element at every output.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import synth
import w4a16_nvfp4_gemv_amd as lib
from helpers import (bf16_bits_to_f64, check_down, check_gemv, check_routed_act, check_silu, swizzle_by_reshape,
                     to_bits)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.set_threads(min(16, os.cpu_count() or 1))
    yield


def _say(*a):
    print("[case]", *a, flush=True)


def dev(t):
    return t.to(DEV)


# ------------------------------------------------------------------ bit-exact
@pytest.mark.parametrize("n,k", [(16, 64), (48, 208), (128, 4096), (130, 80), (256, 512), (4096, 4096)])
def test_unswizzle_bit_exact(n, k):
    _say("unswizzle", n, k)
    g = torch.Generator().manual_seed(n + k)
    flat = torch.randint(0, 256, (synth.flat_scale_bytes(n, k),), generator=g, dtype=torch.uint8)
    got = lib.nvfp4_unswizzle_scales(dev(flat), n, k).cpu().numpy()
    assert np.array_equal(got, oracle.unswizzle_scales(flat.numpy(), n, k))


def test_dequantize_rows_every_code_scale_pair_bit_exact():
    n, k = 16, 4096
    codes = np.tile(np.arange(16, dtype=np.uint8), (n, k // 16))
    w = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    logical = ((np.arange(k // 16)[None, :] + 16 * np.arange(n)[:, None]) % 256).astype(np.uint8)
    flat = swizzle_by_reshape(logical, n, k)
    _say("dequantize_rows all pairs")
    got = to_bits(lib.dequantize_rows(dev(torch.from_numpy(w)), dev(torch.from_numpy(flat))).cpu())
    want, _ = oracle.dequantize_rows(w, flat, n, k)
    nan_scale = np.repeat((logical & 0x7F) == 0x7F, 16, axis=1)
    assert np.array_equal(got[~nan_scale], want[~nan_scale])   # includes -0 bit patterns
    assert ((got[nan_scale] & 0x7F80) == 0x7F80).all() and ((got[nan_scale] & 0x7F) != 0).all()


@pytest.mark.parametrize("rows,k", [(16, 256), (48, 512), (272, 1536), (4096, 4096)])
def test_dequantize_rows_random_bit_exact(rows, k):
    _say("dequantize_rows", rows, k)
    d = synth.dense_w4a16(1, rows, k, seed=rows + k)
    got = to_bits(lib.dequantize_rows(dev(d["w"]), dev(d["s"])).cpu())
    want, inexact = oracle.dequantize_rows(d["w"].numpy(), d["s"].numpy(), rows, k)
    assert inexact == 0
    assert np.array_equal(got, want)


# ------------------------------------------------------------------ NVFP4 GEMV
def run_nvfp4(d, n, silu=False):
    out = lib.nvfp4_gemv(dev(d["x"]), dev(d["w"]), dev(d["s"]), dev(d["gs"]), silu_mul=silu)
    torch.cuda.synchronize()
    return to_bits(out.cpu())


SMALL_M = [1, 2, 3, 4, 5, 8, 16, 17, 32]
SMALL_NK = [(256, 512), (48, 64), (144, 192), (400, 320), (128, 4096), (16, 1536)]


PATHS = ["auto", "valu", "mfma", "blk"]


@pytest.fixture
def gemv_path(request, monkeypatch):
    """Forces the kernel family (valu / mfma; valu only where it applies)."""
    monkeypatch.setenv("W4A16_GEMV_PATH", request.param)
    return request.param


@pytest.mark.parametrize("gemv_path", PATHS, indirect=True)
@pytest.mark.parametrize("m", SMALL_M)
@pytest.mark.parametrize("n,k", SMALL_NK)
def test_nvfp4_gemv_small_shapes(m, n, k, gemv_path):
    _say("nvfp4_gemv", m, n, k, gemv_path)
    d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(0, m) + n + k)
    got = run_nvfp4(d, n)
    _, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n)
    check_gemv(got, acc, absacc, d["gs"][0], k, f"nvfp4_gemv M={m} N={n} K={k}")


@pytest.mark.parametrize("gemv_path", PATHS, indirect=True)
@pytest.mark.parametrize("m", [1, 2, 3, 4, 8, 32])
@pytest.mark.parametrize("n,k", [(48, 8192), (32, 14336), (144, 16384), (16, 16448), (32, 20480)])
def test_nvfp4_gemv_long_rows(m, n, k, gemv_path):
    """Rows past 4096 columns: the chunked VALU kernel with 2-4 K slices and
    partly empty chunk slots (up to 16384), the LDS-staged VALU kernel beyond,
    and the MFMA kernel with several steps per wave."""
    _say("nvfp4_gemv long", m, n, k, gemv_path)
    d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(0, m) + n + k)
    got = run_nvfp4(d, n)
    _, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n)
    check_gemv(got, acc, absacc, d["gs"][0], k, f"nvfp4_gemv M={m} N={n} K={k}")


@pytest.mark.parametrize("m", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("n,nq", [(48, 1), (2048, 2), (3072, 3), (4096, 4), (6144, 3)])
@pytest.mark.parametrize("k,c", [(64, 1), (1536, 1), (2560, 2), (4096, 2)])
def test_nvfp4_gemv_4x4_block_kernel(m, n, nq, k, c, monkeypatch):
    """The 4x4 block MFMA kernel at 2..8 tokens (one or two groups of 4):
    every unit size the dispatch picks (1..4 quads, units that cross 128-row
    bands at 3), one or two 512-k segments per lane, ragged K (waves and
    lanes past the end of a row), a partial band (48 rows), every output
    checked.  At 5..8 tokens it serves only where its units fit one round."""
    monkeypatch.delenv("W4A16_GEMV_PATH", raising=False)
    if m > 4 and n == 6144:
        assert lib.gemv_kernel_name(m, n, k) == "k_gemv_mfma_bd<false, 8, 24>"
    else:
        assert lib.gemv_kernel_name(m, n, k) == f"k_gemv_blk<{1 if m <= 4 else 2}, {nq}, {c}, 4, false>"
    _say("nvfp4_gemv blk", m, n, k)
    d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(0, m) + 3 * n + k)
    got = run_nvfp4(d, n)
    _, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n)
    check_gemv(got, acc, absacc, d["gs"][0], k, f"nvfp4_gemv blk M={m} N={n} K={k}")


@pytest.mark.parametrize("m", [2, 3, 4])
@pytest.mark.parametrize("n,nq", [(96, 1), (2 * 2048, 2), (2 * 6144, 3), (2 * 14336, 4)])
@pytest.mark.parametrize("k,c", [(64, 1), (2560, 2), (4096, 2)])
def test_nvfp4_gemv_4x4_block_kernel_silu(m, n, nq, k, c, monkeypatch):
    """The 4x4 block MFMA kernel with silu_mul: units of nq gate quads and
    their up quads (the up rows n/2 further on, in another band), every
    output checked."""
    monkeypatch.delenv("W4A16_GEMV_PATH", raising=False)
    assert lib.gemv_kernel_name(m, n, k, silu_mul=True) == f"k_gemv_blk<1, {nq}, {c}, 4, true>"
    _say("nvfp4_gemv blk silu", m, n, k)
    d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(2, m) + 5 * n + k)
    got = run_nvfp4(d, n, silu=True)
    want, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n, silu_mul=True)
    check_silu(got, want, acc, absacc, d["gs"][0], f"silu blk M={m} N={n} K={k}")


@pytest.mark.parametrize("m", [33, 47, 64])
@pytest.mark.parametrize("n,k,silu", [(256, 512, False), (144, 320, False), (4224, 128, False),
                                      (512, 256, True), (4096, 4096, False)])
def test_nvfp4_gemv_up_to_64_tokens(m, n, k, silu):
    """33..64 tokens: four 16-token tiles staged per step (ragged last tile,
    ragged K, ragged 128-row band, more tiles than compute units, silu_mul,
    the sweep's weight)."""
    _say("nvfp4_gemv 64 tokens", m, n, k, silu)
    d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(0, m) + 3 * n + k)
    got = run_nvfp4(d, n, silu=silu)
    want, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n, silu_mul=silu)
    if silu:
        check_silu(got, want, acc, absacc, d["gs"][0], f"silu M={m} N={n} K={k}")
    else:
        check_gemv(got, acc, absacc, d["gs"][0], k, f"nvfp4_gemv M={m} N={n} K={k}")


@pytest.mark.parametrize("m", [65, 100, 128, 192])
@pytest.mark.parametrize("fp4,n,k,silu", [(True, 256, 512, False), (True, 4096, 4096, False), (True, 144, 320, False),
                                          (True, 512, 256, True), (False, 256, 512, False), (False, 96, 144, True)])
def test_gemv_past_64_tokens(m, fp4, n, k, silu):
    """65..192 tokens: one launch per 64 tokens (the last one ragged), NVFP4
    and BF16 weights, silu_mul."""
    _say("gemv past 64 tokens", m, fp4, n, k, silu)
    if fp4:
        d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(0, m) + 5 * n + k)
        got = run_nvfp4(d, n, silu=silu)
        want, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n, silu_mul=silu)
        gs = d["gs"][0]
    else:
        d = synth.dense_bf16(m, n, k, seed=synth.seed_for(3, m) + 5 * n + k)
        got = run_bf16(d, silu=silu)
        want, acc, absacc = oracle.bf16_gemv(d["x"], d["w"], silu_mul=silu)
        gs = 1.0
    if silu:
        check_silu(got, want, acc, absacc, gs, f"{m} tokens silu N={n} K={k}")
    else:
        check_gemv(got, acc, absacc, gs, k, f"{m} tokens N={n} K={k}")


@pytest.mark.parametrize("m", [100, 192])
def test_gemv_splitk_past_64_tokens(m):
    """The split-K entry point past 64 tokens: every 64-token launch reuses
    the workspace (its counters are zero again after each), strided x."""
    n, k = 1024, 8192
    d = synth.dense_w4a16(m, n, k, seed=1300 + m)
    wide = torch.zeros((m, k + 64), dtype=torch.bfloat16)
    wide[:, :k] = d["x"]
    xv = dev(wide)[:, :k]
    _say("splitk past 64", m, lib.gemv_kernel_name(m, n, k, splitk=True))
    ws = lib.gemv_splitk_workspace(m, n, k, device=DEV)
    out = lib.nvfp4_gemv_splitk(xv, dev(d["w"]), dev(d["s"]), dev(d["gs"]), workspace=ws)
    torch.cuda.synchronize()
    _, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n)
    check_gemv(to_bits(out.cpu()), acc, absacc, d["gs"][0], k, f"splitk {m} tokens")
    assert int(ws[:65536].count_nonzero()) == 0


@pytest.mark.parametrize("m", [40, 64])
@pytest.mark.parametrize("n,k,silu", [(256, 512, False), (96, 144, False), (512, 256, True)])
def test_bf16_gemv_up_to_64_tokens(m, n, k, silu):
    _say("bf16_gemv 64 tokens", m, n, k, silu)
    d = synth.dense_bf16(m, n, k, seed=synth.seed_for(3, m) + 5 * n + k)
    got = run_bf16(d, silu=silu)
    want, acc, absacc = oracle.bf16_gemv(d["x"], d["w"], silu_mul=silu)
    if silu:
        check_silu(got, want, acc, absacc, 1.0, f"bf16 silu M={m} N={n} K={k}")
    else:
        check_gemv(got, acc, absacc, 1.0, k, f"bf16_gemv M={m} N={n} K={k}")


@pytest.mark.parametrize("m,n,k,silu", [
    (1, 256, 512, False),
    (33, 256, 512, False),       # past the pages' 32-token GEMV
    (64, 144, 768, False),       # ragged 128-row band
    (200, 384, 1024, False),
    (48, 512, 512, True),
    (96, 4096, 4096, False),     # the sweep's weight at 96 tokens
])
def test_nvfp4_dequant_gemm(m, n, k, silu):
    """Large-M path (dequantize into a BF16 copy, library GEMM with FP32 sums,
    scale epilogue) against the GEMV oracle, whose definition it shares."""
    _say("dequant_gemm", m, n, k, silu)
    d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(0, m) + 7 * n + k)
    out = lib.dequant_gemm(dev(d["x"]), dev(d["w"]), dev(d["s"]), dev(d["gs"]), silu_mul=silu)
    torch.cuda.synchronize()
    got = to_bits(out.cpu())
    want, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n, silu_mul=silu)
    if silu:
        check_silu(got, want, acc, absacc, d["gs"][0], f"dequant_gemm silu M={m} N={n} K={k}")
    else:
        check_gemv(got, acc, absacc, d["gs"][0], k, f"dequant_gemm M={m} N={n} K={k}")


def test_nvfp4_dequant_gemm_strided_x_and_reuse():
    """x with a row stride past K; a second call with other sizes on a fresh
    workspace gives the same results as a call of its own."""
    m, n, k = 40, 256, 768
    d = synth.dense_w4a16(m, n, k, seed=4242)
    xpad = torch.zeros((m, k + 64), dtype=torch.bfloat16)
    xpad[:, :k] = d["x"]
    x = dev(xpad)[:, :k]
    assert x.stride(0) == k + 64
    out = lib.dequant_gemm(x, dev(d["w"]), dev(d["s"]), dev(d["gs"]))
    torch.cuda.synchronize()
    _, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n)
    check_gemv(to_bits(out.cpu()), acc, absacc, d["gs"][0], k, "dequant_gemm strided x")
    d2 = synth.dense_w4a16(5, 128, 256, seed=4243)
    a = to_bits(lib.dequant_gemm(dev(d2["x"]), dev(d2["w"]), dev(d2["s"]), dev(d2["gs"])).cpu())
    b = to_bits(lib.dequant_gemm(dev(d2["x"]), dev(d2["w"]), dev(d2["s"]), dev(d2["gs"])).cpu())
    np.testing.assert_array_equal(a, b)  # the sums do not depend on timing (no atomics)


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("n,k,silu", [(4112, 128, False), (4176, 320, False), (6144, 1024, False), (8448, 128, True),
                                      (8256, 64, True)])
def test_nvfp4_gemv_24_row_units(m, n, k, silu, monkeypatch):
    """Up to 8 tokens with more 16-row tiles than compute units but at most
    one 24-row unit per compute unit: the block-diagonal MFMA kernels (4- and
    8-token forms), with ragged last units, partial super-steps and
    silu_mul."""
    _say("nvfp4_gemv 24-row units", m, n, k, silu)
    monkeypatch.setenv("W4A16_GEMV_PATH", "mfma")  # also at 1 and 2 tokens
    assert lib.gemv_kernel_name(m, n, k, silu_mul=silu).startswith("k_gemv_mfma_bd<")
    d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(0, m) + n + k + 7)
    got = run_nvfp4(d, n, silu=silu)
    want, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n, silu_mul=silu)
    if silu:
        check_silu(got, want, acc, absacc, d["gs"][0], f"silu M={m} N={n} K={k}")
    else:
        check_gemv(got, acc, absacc, d["gs"][0], k, f"nvfp4_gemv M={m} N={n} K={k}")


@pytest.mark.parametrize("m", [5, 7, 8])
@pytest.mark.parametrize("n,k,silu", [(14336, 256, False), (14000, 192, False), (28672, 128, True)])
def test_nvfp4_gemv_56_row_units(m, n, k, silu):
    """5..8 tokens where only 56-row units fit the compute units (14336 rows
    and the fused silu call on 2 x 14336), including a ragged last unit."""
    _say("nvfp4_gemv 56-row units", m, n, k, silu)
    assert lib.gemv_kernel_name(m, n, k, silu_mul=silu) == f"k_gemv_mfma_bd<{'true' if silu else 'false'}, 8, 56>"
    d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(0, m) + n + k + 13)
    got = run_nvfp4(d, n, silu=silu)
    want, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n, silu_mul=silu)
    if silu:
        check_silu(got, want, acc, absacc, d["gs"][0], f"silu M={m} N={n} K={k}")
    else:
        check_gemv(got, acc, absacc, d["gs"][0], k, f"nvfp4_gemv M={m} N={n} K={k}")


@pytest.mark.parametrize("m", [3, 8])
def test_nvfp4_gemv_24_row_units_long_rows(m):
    """The block-diagonal kernels over many super-steps per wave (K = 16448:
    the ring refills, ragged last super-step)."""
    n, k = 4176, 16448
    _say("nvfp4_gemv 24-row units long", m, n, k)
    assert lib.gemv_kernel_name(m, n, k).startswith("k_gemv_mfma_bd<")
    d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(0, m) + 11)
    got = run_nvfp4(d, n)
    _, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n)
    check_gemv(got, acc, absacc, d["gs"][0], k, f"nvfp4_gemv M={m} N={n} K={k}")


@pytest.mark.parametrize("m", [8, 17, 32])
@pytest.mark.parametrize("n,k,silu", [(4224, 128, False), (4176, 192, False), (8448, 128, True), (8256, 64, True)])
def test_nvfp4_gemv_many_row_tiles(m, n, k, silu):
    """More 16-row tiles than compute units: the MFMA workgroups take two
    tiles each, including ragged last bands."""
    _say("nvfp4_gemv many tiles", m, n, k, silu)
    d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(0, m) + n + k)
    got = run_nvfp4(d, n, silu=silu)
    want, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n, silu_mul=silu)
    if silu:
        check_silu(got, want, acc, absacc, d["gs"][0], f"silu M={m} N={n} K={k}")
    else:
        check_gemv(got, acc, absacc, d["gs"][0], k, f"nvfp4_gemv M={m} N={n} K={k}")


@pytest.mark.parametrize("gemv_path", PATHS, indirect=True)
@pytest.mark.parametrize("m", [1, 2, 4, 5, 16, 32])
@pytest.mark.parametrize("n,k", [(256, 512), (96, 128), (288, 256), (512, 1536), (64, 12288)])
def test_nvfp4_gemv_silu_small_shapes(m, n, k, gemv_path):
    _say("nvfp4_gemv silu", m, n, k, gemv_path)
    d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(2, m) + n + k)
    got = run_nvfp4(d, n, silu=True)
    want, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n, silu_mul=True)
    check_silu(got, want, acc, absacc, d["gs"][0], f"silu M={m} N={n} K={k}")


@pytest.mark.parametrize("gemv_path", PATHS, indirect=True)
@pytest.mark.parametrize("m", [1, 2, 4, 8, 16, 32])
@pytest.mark.parametrize("n,k,variant", [(4096, 4096, 0), (6144, 4096, 1)])
def test_nvfp4_gemv_dense_sweep_full_size(m, n, k, variant, gemv_path):
    _say("nvfp4_gemv full", m, n, k, gemv_path)
    d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(1, m, variant))
    got = run_nvfp4(d, n)
    _, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n)
    check_gemv(got, acc, absacc, d["gs"][0], k, f"nvfp4_gemv M={m} N={n} K={k}")


@pytest.mark.parametrize("m", [1, 8, 32])
def test_nvfp4_gemv_gate_up_silu_full_size(m):
    """The fused gate|up call at its full size, every output element."""
    n, k = 2 * 14336, 4096
    _say("nvfp4_gemv silu full", m, n, k)
    d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(2, m))
    got = run_nvfp4(d, n, silu=True)
    want, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n, silu_mul=True)
    check_silu(got, want, acc, absacc, d["gs"][0], f"silu full M={m}")


def test_nvfp4_gemv_row_stride_and_zero_tokens():
    m, n, k = 3, 256, 512
    d = synth.dense_w4a16(m, n, k, seed=77)
    wide = torch.zeros((m, k + 64), dtype=torch.bfloat16)
    wide[:, :k] = d["x"]
    xv = dev(wide)[:, :k]
    assert xv.stride(0) == k + 64
    out = to_bits(lib.nvfp4_gemv(xv, dev(d["w"]), dev(d["s"]), dev(d["gs"])).cpu())
    _, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n)
    check_gemv(out, acc, absacc, d["gs"][0], k, "strided x")
    empty = lib.nvfp4_gemv(dev(d["x"][:0]), dev(d["w"]), dev(d["s"]), dev(d["gs"]))
    assert tuple(empty.shape) == (0, n)


def at_offset(t, off):
    """A device copy of `t` whose data pointer is `off` bytes past a 256-byte
    boundary (a 4- but not 16-byte aligned view for off = 4)."""
    raw = t.contiguous().view(torch.uint8).reshape(-1)
    buf = torch.zeros(raw.numel() + 512, dtype=torch.uint8, device=DEV)
    start = (-buf.data_ptr()) % 256 + off
    view = buf[start:start + raw.numel()]
    view.copy_(dev(raw))
    assert view.data_ptr() % 256 == off
    return view.view(t.dtype).reshape(t.shape)


@pytest.mark.parametrize("off", [4, 8, 12])
@pytest.mark.parametrize("m,n,k,silu", [(1, 256, 512, False), (2, 272, 1088, False), (1, 512, 1024, True),
                                        (3, 256, 512, False), (8, 6144, 256, False), (32, 512, 1024, True),
                                        (2, 64, 20480, False)])
def test_nvfp4_gemv_scale_buffer_4_byte_aligned(m, n, k, silu, off):
    """Scale buffers need only 4-byte alignment (a row's 4 scales of a 64-k
    tile are one 32-bit word): a view 4, 8 or 12 bytes past a 16-byte
    boundary gives results within the bound at token counts and shapes of
    every kernel family (the calls whose default kernel reads 16-byte scale
    chunks run the MFMA kernels)."""
    _say("nvfp4_gemv 4-byte scales", m, n, k, silu, off)
    d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(0, m) + n + k + off)
    s_view = at_offset(d["s"], off)
    out = to_bits(lib.nvfp4_gemv(dev(d["x"]), dev(d["w"]), s_view, dev(d["gs"]), silu_mul=silu).cpu())
    want, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n, silu_mul=silu)
    if silu:
        check_silu(out, want, acc, absacc, d["gs"][0], f"4-byte scales silu M={m} N={n} K={k}")
    else:
        check_gemv(out, acc, absacc, d["gs"][0], k, f"4-byte scales M={m} N={n} K={k}")


@pytest.mark.parametrize("m", [1, 2, 5])
def test_moe_scale_buffers_4_byte_aligned(m):
    """The MoE pair with every scale buffer 4 bytes past a 16-byte boundary
    (one and two tokens then run the MFMA forms)."""
    e, topk, h, inter, si = 6, 3, 256, 128, 192
    wts = synth.moe_weights(e, h, inter, si, seed=500 + m)
    tok = synth.moe_tokens(m, h, e, topk, seed=510 + m)
    _say("moe 4-byte scales", m)
    gw = {k: dev(v) for k, v in wts.items()}
    for name in ("w1_sf", "ssh", "w2_sf", "ssd"):
        gw[name] = at_offset(wts[name], 4)
    act = torch.empty((m * topk, inter), dtype=torch.bfloat16, device=DEV)
    sact = torch.empty((m, si), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((m, h), dtype=torch.bfloat16, device=DEV)
    ids = dev(tok["ids"])
    lib.moe_gate_up(dev(tok["x"]), ids, gw["w1"], gw["w1_sf"], gw["alpha"], act, gw["wsh"], gw["ssh"], gw["gssh"],
                    sact)
    lib.moe_down_combine(act, ids, dev(tok["tw"]), gw["w2"], gw["w2_sf"], gw["alpha2"], sact, gw["wsd"], gw["ssd"],
                         gw["gssd"], out)
    torch.cuda.synchronize()
    moe_check(wts, tok, act.cpu(), sact.cpu(), to_bits(out.cpu()), list(range(m)), f"moe 4-byte scales M={m}")


@pytest.mark.parametrize("m", [3, 7])
@pytest.mark.parametrize("k", [1040, 2560, 5120])
def test_bf16_gemv_block_kernel_strided_activations(m, k, monkeypatch):
    """The BF16 4x4 block kernel (forced) reads its activations straight from
    x: a row stride past K (ldx = K + 64), one and two token groups, every
    wave's pieces up front (K = 1040, 2560) and in rounds (K = 5120)."""
    monkeypatch.setenv("W4A16_GEMV_PATH", "blk")
    n = 272
    assert lib.gemv_kernel_name(m, n, k, weight_fp4=False).startswith(f"k_gemv_blkh<{1 if m <= 4 else 2},")
    b = synth.dense_bf16(m, n, k, seed=97 + m + k)
    wide = torch.zeros((m, k + 64), dtype=torch.bfloat16)
    wide[:, :k] = b["x"]
    wide[:, k:] = float("nan")  # never read
    xv = dev(wide)[:, :k]
    out = to_bits(lib.bf16_gemv(xv, dev(b["w"])).cpu())
    _, acc, absacc = oracle.bf16_gemv(b["x"], b["w"])
    check_gemv(out, acc, absacc, 1.0, k, f"strided x bf16 blkh M={m} K={k}")


@pytest.mark.parametrize("m", [1, 2, 5, 17, 40])
def test_gemv_row_strided_activations_every_family(m):
    """x with a row stride past K (ldx = K + 64) on each kernel family: the
    VALU kernels (1, 2 tokens), and the MFMA tiles staging 8, 32 and 64
    tokens; NVFP4 and BF16 weights."""
    n, k = 272, 1088
    d = synth.dense_w4a16(m, n, k, seed=90 + m)
    wide = torch.zeros((m, k + 64), dtype=torch.bfloat16)
    wide[:, :k] = d["x"]
    xv = dev(wide)[:, :k]
    out = to_bits(lib.nvfp4_gemv(xv, dev(d["w"]), dev(d["s"]), dev(d["gs"])).cpu())
    _, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n)
    check_gemv(out, acc, absacc, d["gs"][0], k, f"strided x nvfp4 M={m}")
    b = synth.dense_bf16(m, n, k, seed=95 + m)
    wide[:, :k] = b["x"]
    xv = dev(wide)[:, :k]
    out = to_bits(lib.bf16_gemv(xv, dev(b["w"])).cpu())
    _, acc, absacc = oracle.bf16_gemv(b["x"], b["w"])
    check_gemv(out, acc, absacc, 1.0, k, f"strided x bf16 M={m}")


@pytest.mark.parametrize("m", [1, 4, 8, 32])
def test_gemv_and_moe_in_hip_graph_replays(m):
    """The calls captured in a HIP graph give the eager results bit for bit on
    every replay, with eager work and synchronisation between the replays;
    the eager results are checked against the oracle."""
    n, k = 512, 1024
    d = synth.dense_w4a16(m, n, k, seed=60 + m)
    x, w, sc, gs = dev(d["x"]), dev(d["w"]), dev(d["s"]), dev(d["gs"])
    e, topk, h, inter, si = 8, 4, 256, 128, 128
    wts = {kk: dev(v) for kk, v in synth.moe_weights(e, h, inter, si, seed=70 + m).items()}
    tok = {kk: dev(v) for kk, v in synth.moe_tokens(m, h, e, topk, seed=80 + m).items()}
    out = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    fused = torch.empty((m, n // 2), dtype=torch.bfloat16, device=DEV)
    act = torch.empty((m * topk, inter), dtype=torch.bfloat16, device=DEV)
    sact = torch.empty((m, si), dtype=torch.bfloat16, device=DEV)
    mo = torch.empty((m, h), dtype=torch.bfloat16, device=DEV)

    def calls():
        out.copy_(lib.nvfp4_gemv(x, w, sc, gs))
        fused.copy_(lib.nvfp4_gemv(x, w, sc, gs, silu_mul=True))
        lib.moe_gate_up(tok["x"], tok["ids"], wts["w1"], wts["w1_sf"], wts["alpha"], act, wts["wsh"],
                        wts["ssh"], wts["gssh"], sact)
        lib.moe_down_combine(act, tok["ids"], tok["tw"], wts["w2"], wts["w2_sf"], wts["alpha2"], sact,
                             wts["wsd"], wts["ssd"], wts["gssd"], mo)

    calls()
    torch.cuda.synchronize()
    want = [to_bits(t.cpu()) for t in (out, fused, act, sact, mo)]
    # the eager results against the oracle, so that every replay below is too
    _, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n)
    check_gemv(want[0], acc, absacc, d["gs"][0], k, f"graph test gemv M={m}")
    ref, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n, silu_mul=True)
    check_silu(want[1], ref, acc, absacc, d["gs"][0], f"graph test silu M={m}")
    moe_check({kk: v.cpu() for kk, v in wts.items()}, {kk: v.cpu() for kk, v in tok.items()}, act.cpu(), sact.cpu(),
              want[4], list(range(m)), f"graph test moe M={m}")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):  # warm the allocator on the capture stream
        calls()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        calls()
    for rep in range(3):
        for t in (out, fused, act, sact, mo):
            t.zero_()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [to_bits(t.cpu()) for t in (out, fused, act, sact, mo)]
        for name, a, b in zip(("gemv", "silu", "act", "sact", "moe out"), got, want):
            assert np.array_equal(a, b), f"graph replay {rep}: {name} differs from the eager call (M={m})"


@pytest.mark.parametrize("m", [1, 8, 32])
def test_nvfp4_gemv_is_deterministic(m):
    """Split-K partials are added in split order, so repeated calls agree bit for bit."""
    d = synth.dense_w4a16(m, 4096, 4096, seed=5)
    a = run_nvfp4(d, 4096)
    for _ in range(3):
        assert np.array_equal(a, run_nvfp4(d, 4096))


def test_nvfp4_gemv_rejects_bad_shapes():
    d = synth.dense_w4a16(193, 256, 512, seed=1)  # one token past the limit
    with pytest.raises(lib.W4A16Error):
        lib.nvfp4_gemv(dev(d["x"]), dev(d["w"]), dev(d["s"]), dev(d["gs"]))


# ------------------------------------------------------------------ BF16 GEMV
def run_bf16(d, silu=False):
    out = lib.bf16_gemv(dev(d["x"]), dev(d["w"]), silu_mul=silu)
    torch.cuda.synchronize()
    return to_bits(out.cpu())


@pytest.mark.parametrize("gemv_path", PATHS, indirect=True)
@pytest.mark.parametrize("m", [1, 2, 4, 5, 16, 32])
@pytest.mark.parametrize("n,k", [(48, 64), (256, 512), (144, 1040), (64, 4096), (32, 336)])
def test_bf16_gemv_small_shapes(m, n, k, gemv_path):
    _say("bf16_gemv", m, n, k, gemv_path)
    d = synth.dense_bf16(m, n, k, seed=synth.seed_for(3, m) + n + k)
    got = run_bf16(d)
    _, acc, absacc = oracle.bf16_gemv(d["x"], d["w"])
    check_gemv(got, acc, absacc, 1.0, k, f"bf16_gemv M={m} N={n} K={k}")


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("n,nq", [(48, 1), (2048, 2), (3072, 3), (4096, 4)])
@pytest.mark.parametrize("k", [16, 1040, 1536, 2560, 4096, 14336])
def test_bf16_gemv_4x4_block_kernel(m, n, nq, k, monkeypatch):
    """The BF16 4x4 block kernel (forced) at 1..8 tokens: every unit size,
    one and two token groups, a piece cut by the end of the row (K % 128 !=
    0), waves without pieces (K = 16), every wave's pieces loaded up front
    (R = 4 up to 4 pieces per wave, 8 up to 8) and in rounds of 4 (K = 14336,
    28 pieces per wave, a last round of fewer), every output checked."""
    monkeypatch.setenv("W4A16_GEMV_PATH", "blk")
    pw = (-(-k // 128) + 3) // 4  # 128-k pieces per wave
    r, one = (4, "true") if pw <= 4 else ((8, "true") if pw <= 8 else (4, "false"))
    g = 1 if m <= 4 else 2
    assert lib.gemv_kernel_name(m, n, k, weight_fp4=False) == f"k_gemv_blkh<{g}, {nq}, {r}, 4, {one}>"
    _say("bf16_gemv blkh", m, n, k)
    d = synth.dense_bf16(m, n, k, seed=synth.seed_for(3, m) + 7 * n + k)
    got = run_bf16(d)
    _, acc, absacc = oracle.bf16_gemv(d["x"], d["w"])
    check_gemv(got, acc, absacc, 1.0, k, f"bf16_gemv blkh M={m} N={n} K={k}")


@pytest.mark.parametrize("gemv_path", PATHS, indirect=True)
@pytest.mark.parametrize("m", [1, 3, 4, 8, 17])
@pytest.mark.parametrize("k", [144, 336, 1040])
def test_bf16_gemv_nonfinite_next_row(m, k, gemv_path):
    """K % 128 != 0, and every odd row starts with 128 infinite weights: a
    kernel whose last 128-k piece read past the end of an even row would
    pick them up (times zero activations: NaN).  The even rows must match
    the oracle; the odd rows' own sums are not finite and are not compared."""
    n = 64
    _say("bf16_gemv nonfinite next row", m, n, k, gemv_path)
    d = synth.dense_bf16(m, n, k, seed=synth.seed_for(3, m) + 11 * k)
    w = d["w"].clone()
    w[1::2, :128] = float("inf")
    d = dict(x=d["x"], w=w)
    got = run_bf16(d)
    _, acc, absacc = oracle.bf16_gemv(d["x"], d["w"])
    check_gemv(got[:, 0::2], acc[:, 0::2], absacc[:, 0::2], 1.0, k, f"bf16_gemv M={m} N={n} K={k} even rows")


@pytest.mark.parametrize("m", [1, 4, 16, 32])
@pytest.mark.parametrize("n,k,variant", [(4096, 4096, 0), (4096, 14336, 1)])
def test_bf16_gemv_full_size(m, n, k, variant):
    """The BF16-weight calls at their full sizes, every output element."""
    _say("bf16_gemv full", m, n, k)
    d = synth.dense_bf16(m, n, k, seed=synth.seed_for(3, m, variant))
    got = run_bf16(d)
    _, acc, absacc = oracle.bf16_gemv(d["x"], d["w"])
    check_gemv(got, acc, absacc, 1.0, k, f"bf16_gemv M={m} N={n} K={k}")


@pytest.mark.parametrize("m", [4, 17])
@pytest.mark.parametrize("n,k,silu", [(4112, 64, False), (4144, 32, False), (8256, 64, True)])
def test_bf16_gemv_many_row_tiles(m, n, k, silu):
    """More 16-row tiles than compute units, an odd number of them: the last
    two-tile workgroup has one tile past the end."""
    _say("bf16_gemv many tiles", m, n, k, silu)
    d = synth.dense_bf16(m, n, k, seed=synth.seed_for(3, m) + n + k)
    got = run_bf16(d, silu=silu)
    want, acc, absacc = oracle.bf16_gemv(d["x"], d["w"], silu_mul=silu)
    if silu:
        check_silu(got, want, acc, absacc, 1.0, f"bf16 silu M={m} N={n} K={k}")
    else:
        check_gemv(got, acc, absacc, 1.0, k, f"bf16_gemv M={m} N={n} K={k}")


@pytest.mark.parametrize("gemv_path", PATHS, indirect=True)
@pytest.mark.parametrize("m", [1, 3, 8, 32])
def test_bf16_gemv_silu(m, gemv_path):
    n, k = 512, 1024
    d = synth.dense_bf16(m, n, k, seed=900 + m)
    got = run_bf16(d, silu=True)
    want, acc, absacc = oracle.bf16_gemv(d["x"], d["w"], silu_mul=True)
    check_silu(got, want, acc, absacc, 1.0, f"bf16 silu M={m}")


# ------------------------------------------------------------------ MoE
def moe_run(wts, tok, m, topk, inter, si, h):
    x = dev(tok["x"])
    ids = dev(tok["ids"])
    act = torch.empty((m * topk, inter), dtype=torch.bfloat16, device=DEV)
    sact = torch.empty((m, si), dtype=torch.bfloat16, device=DEV)
    gw = {k: dev(v) for k, v in wts.items()}
    lib.moe_gate_up(x, ids, gw["w1"], gw["w1_sf"], gw["alpha"], act, gw["wsh"], gw["ssh"], gw["gssh"], sact)
    out = torch.empty((m, h), dtype=torch.bfloat16, device=DEV)
    lib.moe_down_combine(act, ids, dev(tok["tw"]), gw["w2"], gw["w2_sf"], gw["alpha2"], sact, gw["wsd"],
                         gw["ssd"], gw["gssd"], out)
    torch.cuda.synchronize()
    return act.cpu(), sact.cpu(), to_bits(out.cpu())


def moe_check(wts, tok, act, sact, out, tokens, what):
    """Stage-wise: gate_up against the oracle; down_combine against the oracle
    fed with the GPU's own act / sact (so stage errors do not compound)."""
    topk = tok["ids"].shape[1]
    pairs = np.concatenate([np.arange(t * topk, (t + 1) * topk) for t in tokens])
    ids = tok["ids"][tokens].contiguous()
    r = oracle.moe_gate_up(tok["x"][tokens].contiguous(), ids, wts["w1"], wts["w1_sf"], wts["alpha"],
                           wts["wsh"], wts["ssh"], wts["gssh"])
    alpha_pp = wts["alpha"].numpy()[ids.numpy().reshape(-1)]
    check_routed_act(to_bits(act[pairs]), r["act"], r["acc_r"], r["abs_r"], alpha_pp, what + " act")
    check_silu(to_bits(sact[tokens]), r["sact"], r["acc_s"], r["abs_s"], wts["gssh"][0], what + " sact")
    d = oracle.moe_down_combine(act[pairs].contiguous(), ids, tok["tw"][tokens].contiguous(), wts["w2"],
                                wts["w2_sf"], wts["alpha2"], sact[tokens].contiguous(), wts["wsd"],
                                wts["ssd"], wts["gssd"])
    a2 = wts["alpha2"].numpy()[ids.numpy()]
    check_down(out[tokens], d["out"], d["acc_r"], d["abs_r"], d["acc_s"], d["abs_s"],
               tok["tw"][tokens].numpy(), a2, wts["gssd"][0], what + " out")


@pytest.mark.parametrize("m,e,topk,h,inter,si", [
    (1, 4, 2, 256, 128, 128),
    (2, 6, 3, 192, 64, 128),      # two tokens: the VALU forms with token pairs
    (3, 6, 3, 128, 192, 64),      # I not a multiple of 128: unaligned up quad
    (5, 8, 4, 512, 256, 320),
    (16, 12, 4, 320, 448, 192),   # H, I, SI not multiples of 128; shared expert in two token groups
    (32, 16, 8, 256, 128, 128),
])
def test_moe_small_shapes(m, e, topk, h, inter, si):
    _say("moe", m, e, topk, h, inter, si)
    wts = synth.moe_weights(e, h, inter, si, seed=300 + m)
    tok = synth.moe_tokens(m, h, e, topk, seed=400 + m)
    act, sact, out = moe_run(wts, tok, m, topk, inter, si, h)
    moe_check(wts, tok, act, sact, out, list(range(m)), f"moe M={m}")


@pytest.mark.parametrize("m,ids", [
    (1, [[3, 3, 1, 3]]),
    (2, [[0, 5, 0, 2], [5, 5, 5, 5]]),
    (4, [[1, 2, 3, 4], [4, 3, 2, 1], [0, 0, 5, 5], [2, 2, 2, 2]]),
])
def test_moe_duplicate_experts_up_to_four_tokens(m, ids):
    """Up to four tokens (the forms with one job per pair): pairs routed to
    the same expert, within a token and across tokens."""
    e, topk, h, inter, si = 6, 4, 256, 192, 128
    wts = synth.moe_weights(e, h, inter, si, seed=353 + m)
    tok = synth.moe_tokens(m, h, e, topk, seed=354 + m)
    tok["ids"] = torch.tensor(ids, dtype=torch.int32)
    _say("moe duplicates", m, e, topk)
    act, sact, out = moe_run(wts, tok, m, topk, inter, si, h)
    moe_check(wts, tok, act, sact, out, list(range(m)), f"moe duplicates M={m}")


@pytest.mark.parametrize("m", [1, 2, 4, 8])
@pytest.mark.parametrize("h,inter,si", [
    (128, 512, 64),       # down_combine: one wave
    (192, 1024, 512),     # two waves
    (2048, 1536, 1536),   # three waves, one chunk per lane; gate_up one chunk per lane
    (128, 4096, 256),     # four waves, two chunks per lane
    (4160, 1024, 1024),   # gate_up: two chunks per lane, two K blocks
    (128, 4160, 64),      # I beyond the one-block down_combine: the MFMA form
])
def test_moe_up_to_four_tokens_k_extents(m, h, inter, si):
    """The K extents that select the waves and chunks of the one-job-per-pair
    forms (and the fallback past them), top-8 of 16 experts."""
    e, topk = 16, 8
    wts = synth.moe_weights(e, h, inter, si, seed=380 + m + inter)
    tok = synth.moe_tokens(m, h, e, topk, seed=390 + m + inter)
    _say("moe K extents", m, h, inter, si)
    act, sact, out = moe_run(wts, tok, m, topk, inter, si, h)
    moe_check(wts, tok, act, sact, out, list(range(m)), f"moe K extents M={m} H={h} I={inter} SI={si}")


@pytest.mark.parametrize("m", [1, 3])
def test_moe_more_row_quads_than_workgroups(m):
    """H = 33024: 8256 quads of H rows, more than the 8192 workgroups of the
    one-job-per-pair down_combine, so some workgroups take a second quad
    (its unit loop); gate_up's rows are 33024 columns long (9 K blocks)."""
    e, topk, h, inter, si = 4, 2, 33024, 64, 64
    wts = synth.moe_weights(e, h, inter, si, seed=395 + m)
    tok = synth.moe_tokens(m, h, e, topk, seed=396 + m)
    _say("moe many quads", m, h)
    act, sact, out = moe_run(wts, tok, m, topk, inter, si, h)
    moe_check(wts, tok, act, sact, out, list(range(m)), f"moe many quads M={m}")


@pytest.mark.parametrize("m,topk", [(4, 16), (5, 16), (8, 16), (9, 16)])
def test_moe_most_pairs_of_the_pair_forms(m, topk):
    """The token counts around the limits of the one-job-per-pair forms:
    down_combine takes up to 4 tokens (64 pairs), gate_up up to 8 (128
    pairs); beyond, the MFMA forms."""
    e, h, inter, si = 24, 256, 128, 192
    wts = synth.moe_weights(e, h, inter, si, seed=357 + m)
    tok = synth.moe_tokens(m, h, e, topk, seed=358 + m)
    _say("moe pair-form pairs", m, topk)
    act, sact, out = moe_run(wts, tok, m, topk, inter, si, h)
    moe_check(wts, tok, act, sact, out, list(range(m)), f"moe pairs M={m} topk={topk}")


def test_moe_duplicate_experts_within_a_token():
    """A token routed twice to one expert: both slots count (two act rows,
    two weighted terms of the combine)."""
    m, e, topk, h, inter, si = 5, 6, 4, 128, 128, 64
    wts = synth.moe_weights(e, h, inter, si, seed=351)
    tok = synth.moe_tokens(m, h, e, topk, seed=352)
    ids = torch.tensor([[3, 3, 1, 5], [0, 0, 0, 0], [2, 4, 2, 4], [5, 1, 3, 3], [1, 2, 3, 4]], dtype=torch.int32)
    tok["ids"] = ids
    _say("moe duplicates", m, e, topk)
    act, sact, out = moe_run(wts, tok, m, topk, inter, si, h)
    moe_check(wts, tok, act, sact, out, list(range(m)), "moe duplicates")


def test_moe_most_pairs():
    """32 tokens x 16 slots: the largest routing table, experts shared by
    many tokens."""
    m, e, topk, h, inter, si = 32, 40, 16, 128, 64, 128
    wts = synth.moe_weights(e, h, inter, si, seed=361)
    tok = synth.moe_tokens(m, h, e, topk, seed=362)
    _say("moe most pairs", m, e, topk)
    act, sact, out = moe_run(wts, tok, m, topk, inter, si, h)
    moe_check(wts, tok, act, sact, out, [0, 1, 15, 30, 31], "moe most pairs")


def test_moe_many_experts():
    """More experts than the routing kernels' LDS table holds: the scan
    fallback finds each expert's first pair."""
    m, e, topk, h, inter, si = 3, 2100, 4, 64, 64, 64
    wts = synth.moe_weights(e, h, inter, si, seed=371)
    tok = synth.moe_tokens(m, h, e, topk, seed=372)
    tok["ids"][1] = torch.tensor([2099, 7, 2099 - 64, 7], dtype=torch.int32)  # a repeat and high ids
    _say("moe many experts", m, e, topk)
    act, sact, out = moe_run(wts, tok, m, topk, inter, si, h)
    moe_check(wts, tok, act, sact, out, list(range(m)), "moe many experts")


@pytest.fixture(scope="module")
def moe_block_weights():
    return synth.moe_weights(synth.MOE_EXPERTS, synth.MOE_HIDDEN, synth.MOE_INTER,
                             synth.MOE_SHARED_INTER, seed=synth.seed_for(4, 0))


@pytest.mark.parametrize("m", [1, 8, 32])
def test_moe_decode_block_full_size(m, moe_block_weights):
    _say("moe full", m)
    wts = moe_block_weights
    tok = synth.moe_tokens(m, synth.MOE_HIDDEN, synth.MOE_EXPERTS, synth.MOE_TOPK, seed=synth.seed_for(4, m))
    act, sact, out = moe_run(wts, tok, m, synth.MOE_TOPK, synth.MOE_INTER, synth.MOE_SHARED_INTER,
                             synth.MOE_HIDDEN)
    moe_check(wts, tok, act, sact, out, list(range(m)), f"moe full M={m}")


# ------------------------------------------------------------------ split-K (workspace entry points)
SPLIT_FORMS = ["1,2", "2,2", "3,2", "4,2", "1,4", "2,4", "4,4"]


def run_splitk(d, n, silu=False, ws=None, fp4=True):
    if fp4:
        out = lib.nvfp4_gemv_splitk(dev(d["x"]), dev(d["w"]), dev(d["s"]), dev(d["gs"]), silu_mul=silu, workspace=ws)
    else:
        out = lib.bf16_gemv_splitk(dev(d["x"]), dev(d["w"]), silu_mul=silu, workspace=ws)
    torch.cuda.synchronize()
    return to_bits(out.cpu())


@pytest.mark.parametrize("form", SPLIT_FORMS)
@pytest.mark.parametrize("m", [1, 4, 9, 16, 17, 32, 40, 64])
@pytest.mark.parametrize("n,k,silu", [(256, 512, False), (400, 320, False), (4224, 128, False), (144, 4096, False),
                                      (512, 1024, True), (288, 192, True)])
def test_nvfp4_gemv_splitk_forms(form, m, n, k, silu, monkeypatch):
    """Every built split-K form (row tiles per unit, splits) forced at token
    counts of every staged tile size: ragged 128-row bands, more tiles than
    compute units, splits with no K steps (K = 128 and 192 over 2 or 4
    splits), silu_mul.  The counters are zero again after the call."""
    monkeypatch.setenv("W4A16_SPLITK", form)
    rt, s = map(int, form.split(","))
    name = lib.gemv_kernel_name(m, n, k, silu_mul=silu, splitk=True)
    split = name.endswith(f", {rt}, {s}>") and s > 1
    _say("splitk", form, m, n, k, silu, name)
    if name.startswith("k_gemv_mfma<") and lib._lib.load().gemv_splitk_workspace_bytes(1, m, n, k, int(silu)) > 0:
        assert split, name  # the MFMA path takes the forced form whenever it fits
    d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(0, m) + 17 * n + k + rt)
    ws = lib.gemv_splitk_workspace(m, n, k, silu, device=DEV)
    got = run_splitk(d, n, silu, ws)
    want, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n, silu_mul=silu)
    if silu:
        check_silu(got, want, acc, absacc, d["gs"][0], f"splitk {form} silu M={m} N={n} K={k}")
    else:
        check_gemv(got, acc, absacc, d["gs"][0], k, f"splitk {form} M={m} N={n} K={k}")
    if not split:
        assert int(ws.count_nonzero()) == 0, "workspace written without a split"
    else:
        assert int(ws[:65536].count_nonzero()) == 0, "arrival counters left non-zero"


@pytest.mark.parametrize("form", ["2,2", "3,2", "4,4"])
@pytest.mark.parametrize("m", [16, 32, 64])
@pytest.mark.parametrize("n,k,silu", [(4096, 1024, False), (256, 4096, True), (96, 1040, False)])
def test_bf16_gemv_splitk_forms(form, m, n, k, silu, monkeypatch):
    monkeypatch.setenv("W4A16_SPLITK", form)
    _say("bf16 splitk", form, m, n, k, silu)
    d = synth.dense_bf16(m, n, k, seed=synth.seed_for(3, m) + 19 * n + k)
    got = run_splitk(d, n, silu, None, fp4=False)
    want, acc, absacc = oracle.bf16_gemv(d["x"], d["w"], silu_mul=silu)
    if silu:
        check_silu(got, want, acc, absacc, 1.0, f"bf16 splitk {form} silu M={m} N={n} K={k}")
    else:
        check_gemv(got, acc, absacc, 1.0, k, f"bf16 splitk {form} M={m} N={n} K={k}")


@pytest.mark.parametrize("fp4,m,n,k,silu", [
    (True, 16, 4096, 4096, False), (True, 32, 6144, 4096, False),   # the sweep: no split, same as nvfp4_gemv
    (True, 32, 4096, 14336, False), (True, 16, 1024, 8192, False), (True, 32, 1024, 8192, False),
    (True, 4, 1024, 8192, False), (True, 32, 2048, 4096, False), (True, 32, 4096, 4096, True),
    (False, 32, 4096, 14336, False), (False, 4, 2048, 8192, False), (False, 16, 1024, 4096, False)])
def test_gemv_splitk_default_plan_full_size(fp4, m, n, k, silu, monkeypatch):
    """The default split plan: every output element against the oracle, the
    same bits on repeated calls that reuse the workspace, and where the plan
    does not split, the same bits as the entry point without a workspace."""
    monkeypatch.delenv("W4A16_SPLITK", raising=False)
    name = lib.gemv_kernel_name(m, n, k, silu_mul=silu, weight_fp4=fp4, splitk=True)
    _say("splitk default", fp4, m, n, k, silu, name)
    if fp4:
        d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(1, m) + n + 3 * k)
    else:
        d = synth.dense_bf16(m, n, k, seed=synth.seed_for(3, m) + n + 3 * k)
    ws = lib.gemv_splitk_workspace(m, n, k, silu, weight_fp4=fp4, device=DEV)
    got = run_splitk(d, n, silu, ws, fp4=fp4)
    if fp4:
        want, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n, silu_mul=silu)
        gs = d["gs"][0]
    else:
        want, acc, absacc = oracle.bf16_gemv(d["x"], d["w"], silu_mul=silu)
        gs = 1.0
    if silu:
        check_silu(got, want, acc, absacc, gs, f"splitk {name} M={m} N={n} K={k}")
    else:
        check_gemv(got, acc, absacc, gs, k, f"splitk {name} M={m} N={n} K={k}")
    for _ in range(3):
        assert np.array_equal(got, run_splitk(d, n, silu, ws, fp4=fp4)), "split-K result depends on the call"
    split = name.startswith("k_gemv_mfma<") and name.rsplit(",", 1)[1].strip(" >") != "1"
    if not split:
        assert name == lib.gemv_kernel_name(m, n, k, silu_mul=silu, weight_fp4=fp4), name
        plain = run_nvfp4(d, n, silu) if fp4 else run_bf16(d, silu)
        assert np.array_equal(got, plain)


def test_gemv_splitk_one_workspace_across_plans(monkeypatch):
    """One workspace, sized for the largest call, through default plans with
    different unit counts and splits (the counters of every plan sit in the
    same fixed region, so partial sums of one call never land on counters of
    the next), NVFP4 and BF16, each call against the oracle."""
    monkeypatch.delenv("W4A16_SPLITK", raising=False)
    calls = [(True, 32, 1024, 8192, False), (True, 32, 4096, 4096, True), (True, 16, 512, 4096, False),
             (False, 32, 4096, 14336, False), (True, 4, 1024, 8192, False), (True, 32, 1024, 8192, False)]
    need = max(lib._lib.load().gemv_splitk_workspace_bytes(int(f), m, n, k, int(si)) for f, m, n, k, si in calls)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for i, (fp4, m, n, k, silu) in enumerate(calls):
        _say("splitk across plans", i, fp4, m, n, k, silu, lib.gemv_kernel_name(m, n, k, silu, fp4, splitk=True))
        if fp4:
            d = synth.dense_w4a16(m, n, k, seed=900 + i)
            got = run_splitk(d, n, silu, ws)
            want, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n, silu_mul=silu)
            gs = d["gs"][0]
        else:
            d = synth.dense_bf16(m, n, k, seed=900 + i)
            got = run_splitk(d, n, silu, ws, fp4=False)
            want, acc, absacc = oracle.bf16_gemv(d["x"], d["w"], silu_mul=silu)
            gs = 1.0
        if silu:
            check_silu(got, want, acc, absacc, gs, f"splitk across plans call {i}")
        else:
            check_gemv(got, acc, absacc, gs, k, f"splitk across plans call {i}")
        assert int(ws[:65536].count_nonzero()) == 0, f"call {i} left a counter non-zero"


def test_nvfp4_gemv_splitk_workspace_reuse_and_strided_x(monkeypatch):
    """One workspace through calls of different sizes and forms (each leaves
    its counters zero for the next), x with a row stride past K, and a
    misaligned workspace rejected."""
    monkeypatch.setenv("W4A16_SPLITK", "4,4")
    big = lib.gemv_splitk_workspace(32, 4096, 1024, device=DEV)  # the largest call below
    for m, n, k in ((32, 4096, 1024), (17, 256, 512), (64, 400, 320)):
        d = synth.dense_w4a16(m, n, k, seed=700 + m)
        wide = torch.zeros((m, k + 64), dtype=torch.bfloat16)
        wide[:, :k] = d["x"]
        xv = dev(wide)[:, :k]
        out = lib.nvfp4_gemv_splitk(xv, dev(d["w"]), dev(d["s"]), dev(d["gs"]), workspace=big)
        torch.cuda.synchronize()
        _, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n)
        check_gemv(to_bits(out.cpu()), acc, absacc, d["gs"][0], k, f"splitk reuse M={m} N={n} K={k}")
    d = synth.dense_w4a16(32, 256, 512, seed=777)
    with pytest.raises(lib.W4A16Error):
        lib.nvfp4_gemv_splitk(dev(d["x"]), dev(d["w"]), dev(d["s"]), dev(d["gs"]), workspace=big[16:])
    with pytest.raises(lib.W4A16Error):
        lib.nvfp4_gemv_splitk(dev(d["x"]), dev(d["w"]), dev(d["s"]), dev(d["gs"]), workspace=big[:256])


@pytest.mark.parametrize("form", ["2,2", "4,4"])
def test_nvfp4_gemv_splitk_alternating_inputs_share_a_workspace(form, monkeypatch):
    """Two different input sets alternate on one workspace, 12 calls each:
    every result equals that input's first (oracle-checked) result bit for
    bit, so no call reads partial sums left by the previous one."""
    monkeypatch.setenv("W4A16_SPLITK", form)
    m, n, k = 32, 4096, 2048
    ws = lib.gemv_splitk_workspace(m, n, k, device=DEV)
    sets = [synth.dense_w4a16(m, n, k, seed=810 + i) for i in range(2)]
    gpu = [{kk: dev(v) for kk, v in d.items()} for d in sets]
    first = []
    for d, g in zip(sets, gpu):
        out = to_bits(lib.nvfp4_gemv_splitk(g["x"], g["w"], g["s"], g["gs"], workspace=ws).cpu())
        _, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n)
        check_gemv(out, acc, absacc, d["gs"][0], k, f"splitk alternating {form}")
        first.append(out)
    outs = []
    for i in range(24):
        g = gpu[i % 2]
        outs.append(lib.nvfp4_gemv_splitk(g["x"], g["w"], g["s"], g["gs"], workspace=ws))
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert np.array_equal(to_bits(o.cpu()), first[i % 2]), f"call {i} differs from its input's first result"
    assert int(ws[:65536].count_nonzero()) == 0, "arrival counters left non-zero"



# ------------------------------------------------------------------ split-K in HIP graphs
@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
def test_gemv_splitk_in_hip_graph_replays(entry):
    """The split-K calls captured in a HIP graph (no memset is recorded: the
    counters clear themselves): every replay equals the eager result, which
    is checked against the oracle."""
    m, n, k = 32, 1024, 8192
    d = synth.dense_w4a16(m, n, k, seed=1200)
    x, w, sc, gs = dev(d["x"]), dev(d["w"]), dev(d["s"]), dev(d["gs"])
    ws = lib.gemv_splitk_workspace(m, n, k, device=DEV)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    cl = lib._lib.load()

    def call():
        h = torch.cuda.current_stream().cuda_stream
        if entry == "workspace":
            st = cl.nvfp4_gemv_splitk(x.data_ptr(), m, k, k, w.data_ptr(), sc.data_ptr(), gs.data_ptr(), n, 0,
                                      ws.data_ptr(), ws.numel(), out.data_ptr(), h)
        else:
            st = cl.nvfp4_gemv_splitk_noalloc(x.data_ptr(), m, k, k, w.data_ptr(), sc.data_ptr(), gs.data_ptr(), n,
                                              0, out.data_ptr(), h)
        assert st == 0, cl.w4a16_last_error()

    _say("splitk graph", entry, lib.gemv_kernel_name(m, n, k, splitk=True))
    call()
    torch.cuda.synchronize()
    want = to_bits(out.cpu())
    _, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n)
    check_gemv(want, acc, absacc, d["gs"][0], k, f"splitk graph {entry}")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(3):
            call()
    for rep in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(out.cpu()), want), f"graph replay {rep} differs from the eager call"


# ------------------------------------------------------------------ scale and magnitude edges
EDGE_SHAPES = [(256, 1024, False), (6144, 512, False), (512, 1024, True)]


@pytest.mark.parametrize("gemv_path", PATHS, indirect=True)
@pytest.mark.parametrize("m", [1, 2, 4, 8, 16, 32])
@pytest.mark.parametrize("n,k,silu", EDGE_SHAPES)
def test_nvfp4_gemv_every_finite_scale_and_wide_activations(m, n, k, silu, gemv_path):
    """Scales drawn from all 254 finite E4M3 codes (zero, subnormal, up to
    448, negative) with activations spread over 2^-30 .. 2^100 (N(0,1) times
    2^e): the VALU kernels' block-sum-times-scale order and the MFMA kernels'
    exact dequant both stay within the bound; sums stay below the FP32 range."""
    _say("edge scales", m, n, k, silu, gemv_path)
    d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(0, m) + 31 * n + k, scales="all_finite", x_exp=(-30, 100))
    got = run_nvfp4(d, n, silu=silu)
    want, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n, silu_mul=silu)
    assert np.isfinite(acc).all()
    if silu:
        check_silu(got, want, acc, absacc, d["gs"][0], f"edge scales silu M={m} N={n} K={k}")
    else:
        check_gemv(got, acc, absacc, d["gs"][0], k, f"edge scales M={m} N={n} K={k}")


@pytest.mark.parametrize("gemv_path", PATHS, indirect=True)
@pytest.mark.parametrize("m", [1, 2, 4, 32])
def test_nvfp4_gemv_subnormal_activations(m, gemv_path):
    """Activations in the BF16 subnormal range (2^-140 .. 2^-127): every
    product is an FP32 subnormal or underflows, and the outputs are BF16
    subnormals; the kernels keep them (no flush to zero) within the bound."""
    n, k = 256, 1024
    _say("subnormal x", m, gemv_path)
    d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(0, m) + 77, x_exp=(-140, -127))
    d["gs"] = torch.tensor([1.0], dtype=torch.float32)
    got = run_nvfp4(d, n)
    _, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], 1.0, n)
    assert (np.abs(acc) > 0).mean() > 0.9
    check_gemv(got, acc, absacc, 1.0, k, f"subnormal x M={m}")


@pytest.mark.parametrize("gemv_path", PATHS, indirect=True)
@pytest.mark.parametrize("m", [1, 4, 32])
def test_nvfp4_gemv_epilogue_overflow_to_inf(m, gemv_path):
    """Rows whose FP32 sum is finite but whose product with the global scale
    exceeds the BF16 range round to +-inf (as the oracle's direct rounding
    does); the other rows stay finite and within the bound."""
    n, k = 256, 64
    codes = np.full((n, k), 7, np.uint8)                    # +6.0
    codes[n // 2:] = 15                                     # -6.0 in the second half
    w = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    logical = np.full((n, k // 16), 0x7E, np.uint8)         # 448
    logical[::4] = 0x38                                     # 1.0 on every fourth row: stays finite
    flat = swizzle_by_reshape(logical, n, k)
    x = torch.full((m, k), 2.0 ** 108, dtype=torch.float32).to(torch.bfloat16)
    gs = torch.tensor([8.0], dtype=torch.float32)
    d = dict(x=x, w=torch.from_numpy(w), s=torch.from_numpy(flat), gs=gs)
    _say("overflow", m, gemv_path)
    got = run_nvfp4(d, n)
    want, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], 8.0, n)
    assert np.isfinite(acc).all() and (np.abs(acc) < 2.0 ** 128).all()   # the FP32 sums are finite
    ref = bf16_bits_to_f64(want)
    inf = np.isinf(ref)
    assert inf.sum() == m * (n - n // 4) and (~inf).sum() == m * (n // 4)
    assert np.array_equal(got[inf], want[inf]), "an overflowing row is not +-inf"
    fin = ~inf
    check_gemv(got[fin].reshape(m, -1), acc[fin].reshape(m, -1), absacc[fin].reshape(m, -1), 8.0, k,
               f"overflow finite rows M={m}")


@pytest.mark.parametrize("m", [1, 2, 5, 32])
def test_moe_every_finite_scale_and_wide_activations(m):
    """The MoE pair with all finite E4M3 scale codes and activations spread
    over 2^-20 .. 2^20."""
    e, topk, h, inter, si = 8, 4, 512, 256, 192
    wts = synth.moe_weights(e, h, inter, si, seed=600 + m, scales="all_finite")
    tok = synth.moe_tokens(m, h, e, topk, seed=610 + m)
    g = torch.Generator().manual_seed(620 + m)
    tok["x"] = synth.activations_wide(m, h, g, -20, 20)
    _say("moe edge scales", m)
    act, sact, out = moe_run(wts, tok, m, topk, inter, si, h)
    moe_check(wts, tok, act, sact, out, list(range(m)), f"moe edge scales M={m}")
