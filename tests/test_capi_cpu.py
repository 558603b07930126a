"""C-ABI checks that run without a GPU: the library loads, exports every
function the header declares, and rejects bad arguments before any HIP call."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

from w4a16_nvfp4_gemv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16_nvfp4_gemv.h")

OK, INVALID, MISALIGNED, UNSUPPORTED = 0, 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ["nvfp4_gemv", "bf16_gemv", "dequantize_rows", "moe_gate_up", "moe_down_combine",
                 "nvfp4_unswizzle_scales", "nvfp4_dequant_gemm", "nvfp4_dequant_gemm_workspace_bytes",
                 "nvfp4_status_string", "w4a16_status_string", "w4a16_last_error",
                 "nvfp4_gemv_splitk", "bf16_gemv_splitk", "gemv_splitk_workspace_bytes",
                 "nvfp4_gemv_splitk_noalloc"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None
        assert name in _lib.SIGNATURES


def test_status_strings():
    lib = _lib.load()
    assert lib.w4a16_status_string(OK) == b"ok"
    assert lib.w4a16_status_string(UNSUPPORTED) == b"unsupported shape"
    for st in range(-1, 6):  # the boundary's name and the library's name are one function
        assert lib.nvfp4_status_string(st) == lib.w4a16_status_string(st)


FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced: calls fail validation first


def gemv(**kw):
    a = dict(x=FAKE, M=1, K=4096, ldx=4096, w=FAKE, s=FAKE, gs=FAKE, N=4096, silu=0, out=FAKE)
    a.update(kw)
    return _lib.load().nvfp4_gemv(a["x"], a["M"], a["K"], a["ldx"], a["w"], a["s"], a["gs"], a["N"],
                                  a["silu"], a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=193), UNSUPPORTED),
    (dict(M=-1), INVALID),
    (dict(K=4032 + 32), UNSUPPORTED),    # K % 64 != 0
    (dict(K=0), INVALID),
    (dict(N=4100), UNSUPPORTED),         # N % 16 != 0
    (dict(N=0), INVALID),
    (dict(N=48, silu=1), UNSUPPORTED),   # silu needs N % 32 == 0
    (dict(silu=2), INVALID),
    (dict(ldx=4000), INVALID),           # ldx < K
    (dict(ldx=4100), MISALIGNED),        # ldx % 8 != 0
    (dict(x=FAKE + 2), MISALIGNED),
    (dict(w=FAKE + 8), MISALIGNED),
    (dict(s=FAKE + 2), MISALIGNED),      # scales need 4-byte alignment (4-byte views run on the GPU tests)
    (dict(s=FAKE + 1), MISALIGNED),
    (dict(gs=FAKE + 2), MISALIGNED),
    (dict(out=FAKE + 1), MISALIGNED),
    (dict(x=None), INVALID),
    (dict(s=None), INVALID),
    (dict(gs=None), INVALID),
    (dict(M=0, x=None, w=None, s=None, gs=None, out=None), OK),  # M == 0: no-op
])
def test_nvfp4_gemv_argument_errors(kw, status):
    assert gemv(**kw) == status
    if status != OK:
        assert _lib.load().w4a16_last_error()


def test_bf16_gemv_argument_errors():
    lib = _lib.load()
    assert lib.bf16_gemv(FAKE, 193, 4096, 4096, FAKE, 4096, 0, FAKE, None) == UNSUPPORTED
    assert lib.bf16_gemv(FAKE, 1, 4104, 4104, FAKE, 4096, 0, FAKE, None) == UNSUPPORTED  # K % 16
    assert lib.bf16_gemv(FAKE, 0, 4096, 4096, None, 4096, 0, None, None) == OK


def test_dequantize_rows_argument_errors():
    lib = _lib.load()
    assert lib.dequantize_rows(FAKE, FAKE, 24, 4096, FAKE, None) == UNSUPPORTED  # rows % 16
    assert lib.dequantize_rows(FAKE, FAKE, 32, 4160, FAKE, None) == UNSUPPORTED  # K % 256
    assert lib.dequantize_rows(FAKE + 4, FAKE, 32, 4096, FAKE, None) == MISALIGNED
    assert lib.dequantize_rows(None, FAKE, 32, 4096, FAKE, None) == INVALID
    assert lib.dequantize_rows(None, None, 0, 4096, None, None) == OK


def dgemm(**kw):
    lib = _lib.load()
    a = dict(x=FAKE, M=64, K=4096, ldx=4096, w=FAKE, s=FAKE, gs=FAKE, N=4096, silu=0, ws=FAKE, wsb=None, out=FAKE)
    a.update(kw)
    wsb = a["wsb"] if a["wsb"] is not None else lib.nvfp4_dequant_gemm_workspace_bytes(a["M"], a["N"], a["K"])
    return lib.nvfp4_dequant_gemm(a["x"], a["M"], a["K"], a["ldx"], a["w"], a["s"], a["gs"], a["N"], a["silu"],
                                  a["ws"], wsb, a["out"], None)


def test_dequant_gemm_workspace_size():
    lib = _lib.load()
    # BF16 weight copy rounded up to 256 bytes, then the FP32 sums
    assert lib.nvfp4_dequant_gemm_workspace_bytes(64, 4096, 4096) == 4096 * 4096 * 2 + 64 * 4096 * 4
    assert lib.nvfp4_dequant_gemm_workspace_bytes(3, 16, 256) == 16 * 256 * 2 + 3 * 16 * 4
    assert lib.nvfp4_dequant_gemm_workspace_bytes(1, 16, 264) == (16 * 264 * 2 + 255) // 256 * 256 + 16 * 4
    assert lib.nvfp4_dequant_gemm_workspace_bytes(-1, 16, 256) == -1


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), INVALID),
    (dict(K=4096 + 64, ldx=4096 + 64), UNSUPPORTED),  # K % 256 != 0
    (dict(N=4100), UNSUPPORTED),         # N % 16 != 0
    (dict(N=48, silu=1), UNSUPPORTED),   # silu needs N % 32 == 0
    (dict(silu=3), INVALID),
    (dict(ldx=4000), INVALID),           # ldx < K
    (dict(wsb=1024), INVALID),           # workspace too small
    (dict(ws=None), INVALID),
    (dict(gs=None), INVALID),
    (dict(ws=FAKE + 16), MISALIGNED),    # workspace 256-byte aligned
    (dict(w=FAKE + 8), MISALIGNED),
    (dict(x=FAKE + 1), MISALIGNED),
    (dict(M=0, x=None, w=None, s=None, gs=None, ws=None, out=None), OK),  # M == 0: no-op
])
def test_dequant_gemm_argument_errors(kw, status):
    assert dgemm(**kw) == status
    if status != OK:
        assert _lib.load().w4a16_last_error()


def test_unswizzle_argument_errors():
    lib = _lib.load()
    assert lib.nvfp4_unswizzle_scales(FAKE, 16, 40, FAKE, None) == UNSUPPORTED
    assert lib.nvfp4_unswizzle_scales(None, 16, 64, FAKE, None) == INVALID
    assert lib.nvfp4_unswizzle_scales(None, 0, 64, None, None) == OK


def test_moe_argument_errors():
    lib = _lib.load()
    gu = lambda **kw: lib.moe_gate_up(*[kw.get(k, v) for k, v in dict(
        x=FAKE, M=1, H=4096, ids=FAKE, topk=8, E=128, w1=FAKE, s1=FAKE, alpha=FAKE, I=1536,
        act=FAKE, wsh=FAKE, ssh=FAKE, gssh=FAKE, SI=1536, sact=FAKE, st=None).items()])
    assert gu(M=33) == UNSUPPORTED
    assert gu(topk=17) == UNSUPPORTED
    assert gu(topk=0) == INVALID
    assert gu(H=4000) == UNSUPPORTED
    assert gu(I=1544 - 1) == UNSUPPORTED
    assert gu(ids=None) == INVALID
    assert gu(w1=FAKE + 4) == MISALIGNED
    assert gu(s1=FAKE + 2) == MISALIGNED
    assert gu(ssh=FAKE + 1) == MISALIGNED
    assert gu(M=0, x=None, ids=None) == OK
    dc = lambda **kw: lib.moe_down_combine(*[kw.get(k, v) for k, v in dict(
        act=FAKE, ids=FAKE, tw=FAKE, M=1, topk=8, E=128, w2=FAKE, s2=FAKE, alpha2=FAKE, H=4096,
        I=1536, sact=FAKE, wsd=FAKE, ssd=FAKE, gssd=FAKE, SI=1536, out=FAKE, st=None).items()])
    assert dc(I=1568) == UNSUPPORTED   # I % 64
    assert dc(SI=1552) == UNSUPPORTED
    assert dc(H=4104) == UNSUPPORTED   # H % 16
    assert dc(tw=None) == INVALID
    assert dc(act=FAKE + 8) == MISALIGNED
    assert dc(s2=FAKE + 2) == MISALIGNED
    assert dc(ssd=FAKE + 2) == MISALIGNED
    assert dc(M=0, act=None) == OK


def test_gemv_kernel_name_query(monkeypatch):
    """The host-only query names the kernel family each dense sweep shape
    dispatches to, and rejects what the entry points reject."""
    from w4a16_nvfp4_gemv_amd import W4A16Error, gemv_kernel_name
    monkeypatch.delenv("W4A16_GEMV_PATH", raising=False)
    assert gemv_kernel_name(1, 4096, 4096).startswith("k_gemv_vchunk<1, false,")
    assert gemv_kernel_name(1, 28672, 4096, silu_mul=True).startswith("k_gemv_vchunk<1, true,")
    assert gemv_kernel_name(2, 4096, 8192).startswith("k_gemv_vchunk<2, false,")  # K > 4096
    # 2..4 tokens without silu_mul: the 4x4 block MFMA kernel, with the quads per
    # unit that balance the compute units (the host-only query assumes 256 compute
    # units when no GPU is present) and one or two 512-k segments per lane
    for m in (2, 3, 4):
        assert gemv_kernel_name(m, 4096, 4096) == "k_gemv_blk<1, 4, 2, 4, false>"
        assert gemv_kernel_name(m, 6144, 4096) == "k_gemv_blk<1, 3, 2, 4, false>"
    assert gemv_kernel_name(2, 2048, 4096) == "k_gemv_blk<1, 2, 2, 4, false>"
    assert gemv_kernel_name(3, 1024, 2048) == "k_gemv_blk<1, 1, 1, 4, false>"
    assert gemv_kernel_name(4, 4096, 8192).startswith("k_gemv_mfma<true, 4, false,")  # K > 4096
    for m in (2, 4):  # with silu_mul: units of 4 or 3 gate quads and their up quads
        assert gemv_kernel_name(m, 28672, 4096, silu_mul=True) == "k_gemv_blk<1, 4, 2, 4, true>"
        assert gemv_kernel_name(m, 2 * 6144, 4096, silu_mul=True) == "k_gemv_blk<1, 3, 2, 4, true>"
    # 5..8 tokens: the 4x4 kernel with two token groups where its units fill the
    # compute units in one round
    for m in (5, 8):
        assert gemv_kernel_name(m, 4096, 4096) == "k_gemv_blk<2, 4, 2, 4, false>"
        assert gemv_kernel_name(m, 256, 1024) == "k_gemv_blk<2, 1, 1, 4, false>"
    assert gemv_kernel_name(8, 4096, 4096, silu_mul=True).startswith("k_gemv_mfma<true, 8, true,")
    # the MFMA kernels are named by the token rows they stage per step
    for m, xt in ((9, 16), (16, 16), (17, 32), (32, 32), (33, 64), (64, 64)):
        assert gemv_kernel_name(m, 4096, 4096).startswith(f"k_gemv_mfma<true, {xt}, false,")
    assert gemv_kernel_name(8, 4096, 8192).startswith("k_gemv_mfma<true, 8, false,")  # K > 4096
    for m, xt in ((9, 16), (16, 16), (17, 32), (32, 32), (33, 64), (64, 64)):
        assert gemv_kernel_name(m, 6144, 4096).startswith(f"k_gemv_mfma<true, {xt}, false,")
    # 5..8 tokens where 24-row units fit the compute units and 16-row tiles do not
    for m in (5, 8):
        assert gemv_kernel_name(m, 6144, 4096) == "k_gemv_mfma_bd<false, 8, 24>"
    assert gemv_kernel_name(8, 2 * 6144, 4096, silu_mul=True) == "k_gemv_mfma_bd<true, 8, 24>"
    # 5..8 tokens where only 56-row units fit (the fused silu call on 2 x 14336 rows)
    assert gemv_kernel_name(8, 28672, 4096, silu_mul=True) == "k_gemv_mfma_bd<true, 8, 56>"
    assert gemv_kernel_name(4, 28672, 8192, silu_mul=True).startswith("k_gemv_mfma<true, 4, true,")
    assert gemv_kernel_name(32, 4096, 14336, weight_fp4=False).startswith("k_gemv_mfma<false, 32, false,")
    # BF16 without silu_mul: the 4x4 block kernel at 1..4 tokens, and at 5..8
    # for rows longer than 2048 columns; up to 8 pieces of 128 k per wave all
    # loaded up front (R = 4 or 8), longer rows in rounds of 4
    for m in (1, 4):
        assert gemv_kernel_name(m, 4096, 4096, weight_fp4=False) == "k_gemv_blkh<1, 4, 8, 4, true>"
        assert gemv_kernel_name(m, 4096, 14336, weight_fp4=False) == "k_gemv_blkh<1, 4, 4, 4, false>"
        assert gemv_kernel_name(m, 4096, 16384, weight_fp4=False) == "k_gemv_blkh<1, 4, 4, 4, false>"
    assert gemv_kernel_name(2, 1024, 14336, weight_fp4=False) == "k_gemv_blkh<1, 1, 4, 4, false>"
    assert gemv_kernel_name(3, 4096, 1024, weight_fp4=False) == "k_gemv_blkh<1, 4, 4, 4, true>"
    for m in (5, 8):
        assert gemv_kernel_name(m, 4096, 4096, weight_fp4=False) == "k_gemv_blkh<2, 4, 8, 4, true>"
        assert gemv_kernel_name(m, 2048, 8192, weight_fp4=False) == "k_gemv_blkh<2, 2, 4, 4, false>"
        assert gemv_kernel_name(m, 4096, 2048, weight_fp4=False).startswith("k_gemv_mfma<false, 8, false,")
        assert gemv_kernel_name(m, 4096, 2064, weight_fp4=False) == "k_gemv_blkh<2, 4, 8, 4, true>"  # K > 2048
    assert gemv_kernel_name(9, 4096, 4096, weight_fp4=False).startswith("k_gemv_mfma<false, 16, false,")
    assert gemv_kernel_name(4, 4096, 4096, weight_fp4=False, silu_mul=True).startswith("k_gemv_mfma<false, 4, true,")
    assert gemv_kernel_name(1, 8192, 16384, weight_fp4=False, silu_mul=True).startswith("k_gemv_valu<false, 1, 64, true,")
    monkeypatch.setenv("W4A16_GEMV_PATH", "mfma")
    assert gemv_kernel_name(1, 4096, 4096).startswith("k_gemv_mfma<true, 4, false,")
    for m, tk in ((3, 4), (4, 4)):
        assert gemv_kernel_name(m, 6144, 4096) == f"k_gemv_mfma_bd<false, {tk}, 24>"
    assert gemv_kernel_name(4, 2 * 6144, 4096, silu_mul=True) == "k_gemv_mfma_bd<true, 4, 24>"
    monkeypatch.setenv("W4A16_GEMV_PATH", "blk")
    assert gemv_kernel_name(1, 4096, 4096) == "k_gemv_blk<1, 4, 2, 4, false>"
    assert gemv_kernel_name(8, 4096, 4096) == "k_gemv_blk<2, 4, 2, 4, false>"
    assert gemv_kernel_name(9, 4096, 4096).startswith("k_gemv_mfma<true, 16, false,")  # beyond 8 tokens
    assert gemv_kernel_name(2, 28672, 4096, silu_mul=True) == "k_gemv_blk<1, 4, 2, 4, true>"
    assert gemv_kernel_name(8, 28672, 4096, silu_mul=True) == "k_gemv_blk<2, 4, 2, 4, true>"
    monkeypatch.setenv("W4A16_GEMV_PATH", "valu")
    assert gemv_kernel_name(4, 4096, 4096).startswith("k_gemv_vchunk<4, false,")
    assert gemv_kernel_name(64, 6144, 4096).endswith(", 2, 1>")  # two row tiles per workgroup
    assert gemv_kernel_name(64, 2 * 6144, 4096, silu_mul=True).endswith(", 1, 1>")  # LDS: one with silu_mul
    # past 64 tokens a call launches the 64-token kernel once per 64 tokens
    assert gemv_kernel_name(192, 4096, 4096) == gemv_kernel_name(64, 4096, 4096)
    assert gemv_kernel_name(100, 6144, 4096) == gemv_kernel_name(64, 6144, 4096)
    for bad in (dict(m=0, n=16, k=64), dict(m=193, n=16, k=64), dict(m=1, n=16, k=60), dict(m=1, n=8, k=64)):
        with pytest.raises(W4A16Error):
            gemv_kernel_name(bad["m"], bad["n"], bad["k"])


def splitk(**kw):
    lib = _lib.load()
    a = dict(x=FAKE, M=32, K=8192, ldx=8192, w=FAKE, s=FAKE, gs=FAKE, N=1024, silu=0, ws=FAKE, wsb=None, out=FAKE)
    a.update(kw)
    wsb = a["wsb"] if a["wsb"] is not None else lib.gemv_splitk_workspace_bytes(1, a["M"], a["N"], a["K"], a["silu"])
    return lib.nvfp4_gemv_splitk(a["x"], a["M"], a["K"], a["ldx"], a["w"], a["s"], a["gs"], a["N"], a["silu"],
                                 a["ws"], wsb, a["out"], None)


def test_splitk_plan_and_workspace_size(monkeypatch):
    """The split plan (256 compute units assumed without a GPU): no split at
    the sweep's shapes; one row tile per unit and 2 or 4 splits where the row
    tiles would fill less than half the compute units; units of two tiles
    over 2 splits where a workgroup would stream >= 768 KB of activations.
    The workspace holds 64 KiB of counters (whatever the plan) and the FP32
    partials of every unit and split."""
    from w4a16_nvfp4_gemv_amd import gemv_kernel_name
    monkeypatch.delenv("W4A16_SPLITK", raising=False)
    monkeypatch.delenv("W4A16_GEMV_PATH", raising=False)
    lib = _lib.load()
    for m in (1, 2, 4, 8, 16, 32, 64):
        for n in (4096, 6144):
            assert lib.gemv_splitk_workspace_bytes(1, m, n, 4096, 0) == 0
            assert gemv_kernel_name(m, n, 4096, splitk=True) == gemv_kernel_name(m, n, 4096)
    # 64 tiles, 4 splits: 64 KiB of counters, 64 units x 4 splits x 1 A operand x NT x 1 KB
    for m, xt in ((4, 4), (16, 16), (32, 32)):
        nt = max(1, xt // 16)
        assert gemv_kernel_name(m, 1024, 8192, splitk=True) == f"k_gemv_mfma<true, {xt}, false, 1, 4>"
        assert lib.gemv_splitk_workspace_bytes(1, m, 1024, 8192, 0) == 65536 + 64 * 4 * nt * 1024
    assert gemv_kernel_name(9, 1024, 2048, splitk=True) == "k_gemv_mfma<true, 16, false, 1, 1>"  # too little work
    assert gemv_kernel_name(8, 1024, 4096, splitk=True) == "k_gemv_blk<2, 1, 2, 4, false>"  # the 4x4 kernel: no split
    assert gemv_kernel_name(4, 1024, 4096, splitk=True) == "k_gemv_blk<1, 1, 2, 4, false>"  # the 4x4 kernel: no split
    assert gemv_kernel_name(32, 1024, 4096, splitk=True) == "k_gemv_mfma<true, 32, false, 1, 2>"
    assert gemv_kernel_name(32, 4096, 14336, splitk=True) == "k_gemv_mfma<true, 32, false, 2, 2>"
    assert lib.gemv_splitk_workspace_bytes(1, 32, 4096, 14336, 0) == 65536 + 128 * 2 * 2 * 2 * 1024
    assert gemv_kernel_name(16, 4096, 14336, splitk=True) == "k_gemv_mfma<true, 16, false, 1, 1>"
    assert gemv_kernel_name(32, 4096, 14336, weight_fp4=False, splitk=True) == "k_gemv_mfma<false, 32, false, 2, 2>"
    assert gemv_kernel_name(32, 4096, 4096, silu_mul=True, splitk=True) == "k_gemv_mfma<true, 32, true, 1, 2>"
    assert lib.gemv_splitk_workspace_bytes(1, 193, 4096, 4096, 0) == -1
    # past 64 tokens: the plan of the 64-token launches
    assert lib.gemv_splitk_workspace_bytes(1, 192, 1024, 8192, 0) == lib.gemv_splitk_workspace_bytes(1, 64, 1024, 8192, 0)
    assert lib.gemv_splitk_workspace_bytes(2, 32, 4096, 4096, 0) == -1
    monkeypatch.setenv("W4A16_SPLITK", "off")
    assert lib.gemv_splitk_workspace_bytes(1, 32, 1024, 8192, 0) == 0
    assert gemv_kernel_name(32, 1024, 8192, splitk=True) == gemv_kernel_name(32, 1024, 8192)
    monkeypatch.setenv("W4A16_SPLITK", "4,4")
    assert gemv_kernel_name(32, 4096, 4096, splitk=True) == "k_gemv_mfma<true, 32, false, 4, 4>"
    monkeypatch.setenv("W4A16_SPLITK", "5,3")  # not a built form: no split
    assert lib.gemv_splitk_workspace_bytes(1, 32, 4096, 4096, 0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None), INVALID),                 # the plan splits: a workspace is needed
    (dict(wsb=4096), INVALID),                # too small
    (dict(ws=FAKE + 64), MISALIGNED),         # 256-byte alignment
    (dict(M=193), UNSUPPORTED),
    (dict(s=FAKE + 2), MISALIGNED),
    (dict(M=0, x=None, w=None, s=None, gs=None, ws=None, out=None), OK),
])
def test_nvfp4_gemv_splitk_argument_errors(kw, status, monkeypatch):
    monkeypatch.delenv("W4A16_SPLITK", raising=False)
    assert splitk(**kw) == status
    if status != OK:
        assert _lib.load().w4a16_last_error()


def test_bf16_gemv_splitk_argument_errors(monkeypatch):
    monkeypatch.delenv("W4A16_SPLITK", raising=False)
    lib = _lib.load()
    need = lib.gemv_splitk_workspace_bytes(0, 32, 4096, 14336, 0)
    assert need > 0
    assert lib.bf16_gemv_splitk(FAKE, 32, 14336, 14336, FAKE, 4096, 0, None, need, FAKE, None) == INVALID
    assert lib.bf16_gemv_splitk(FAKE, 32, 14336, 14336, FAKE, 4096, 0, FAKE, need - 1, FAKE, None) == INVALID
    assert lib.bf16_gemv_splitk(FAKE, 32, 14344, 14344, FAKE, 4096, 0, FAKE, need, FAKE, None) == UNSUPPORTED
    assert lib.bf16_gemv_splitk(FAKE, 0, 4096, 4096, None, 4096, 0, None, 0, None, None) == OK


def test_noalloc_rejects_plans_beyond_its_scratch(monkeypatch):
    """The entry point that allocates nothing checks the split plan's scratch
    against the library's fixed size before any HIP call."""
    lib = _lib.load()
    monkeypatch.setenv("W4A16_SPLITK", "1,4")
    # 65536 rows at 64 tokens over 4 splits: 4096 units x 4 x 4 token tiles x 1 KB = 64 MiB
    assert lib.gemv_splitk_workspace_bytes(1, 64, 65536, 4096, 0) > (8 << 20)
    st = lib.nvfp4_gemv_splitk_noalloc(FAKE, 64, 4096, 4096, FAKE, FAKE, FAKE, 65536, 0, FAKE, None)
    assert st == UNSUPPORTED
    assert b"scratch" in lib.w4a16_last_error()
    assert lib.nvfp4_gemv_splitk_noalloc(FAKE, 193, 4096, 4096, FAKE, FAKE, FAKE, 4096, 0, FAKE, None) == UNSUPPORTED
    assert lib.nvfp4_gemv_splitk_noalloc(None, 0, 4096, 4096, None, None, None, 4096, 0, None, None) == OK
