"""The entry point that allocates nothing (nvfp4_gemv_splitk_noalloc), called
through the C ABI: its results equal those of nvfp4_gemv_splitk with a
caller workspace (same kernels, same split plan) and meet the oracle's
bound, on calls in a row that share the library's scratch, the second with
a smaller input."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import check_gemv, check_silu, to_bits
from w4a16_nvfp4_gemv_amd import _lib, gemv_kernel_name

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def call(entry, d, m, n, k, silu):
    """One call of `entry` ("noalloc" or "workspace") through the C ABI."""
    lib = _lib.load()
    x, w, s, gs = (d[key].to(DEV) for key in ("x", "w", "s", "gs"))
    out = torch.empty((m, n // 2 if silu else n), dtype=torch.bfloat16, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    if entry == "noalloc":
        st = lib.nvfp4_gemv_splitk_noalloc(x.data_ptr(), m, k, k, w.data_ptr(), s.data_ptr(), gs.data_ptr(), n,
                                           int(silu), out.data_ptr(), stream)
    else:
        need = lib.gemv_splitk_workspace_bytes(1, m, n, k, int(silu))
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=DEV)
        st = lib.nvfp4_gemv_splitk(x.data_ptr(), m, k, k, w.data_ptr(), s.data_ptr(), gs.data_ptr(), n, int(silu),
                                   ws.data_ptr(), ws.numel(), out.data_ptr(), stream)
    assert st == 0, lib.w4a16_last_error().decode()
    torch.cuda.synchronize()
    return to_bits(out.cpu())


# (M, N, K, silu_mul): split plans with 4 and 2 splits, the second call smaller
SEQUENCES = [
    [(32, 1024, 8192, False), (16, 512, 4096, False)],
    [(32, 4096, 4096, True), (17, 2048, 4096, True)],
    [(32, 4096, 14336, False), (4, 1024, 8192, False), (1, 256, 512, False)],
]


@pytest.mark.parametrize("seq", range(len(SEQUENCES)))
def test_noalloc_matches_the_workspace_entry_point(seq):
    for i, (m, n, k, silu) in enumerate(SEQUENCES[seq]):
        name = gemv_kernel_name(m, n, k, silu_mul=silu, splitk=True)
        print(f"[case] noalloc seq={seq} call={i} M={m} N={n} K={k} silu={silu} {name}", flush=True)
        d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(7, m) + n + k + i)
        got = call("noalloc", d, m, n, k, silu)
        want = call("workspace", d, m, n, k, silu)
        assert np.array_equal(got, want), f"call {i}: the no-allocation entry point differs from the workspace one"
        ref, acc, absacc = oracle.nvfp4_gemv(d["x"], d["w"], d["s"], float(d["gs"][0]), n, silu_mul=silu)
        if silu:
            check_silu(got, ref, acc, absacc, d["gs"][0], f"noalloc M={m} N={n} K={k}")
        else:
            check_gemv(got, acc, absacc, d["gs"][0], k, f"noalloc M={m} N={n} K={k}")
