"""Builds the HIP library libw4a16_nvfp4_gemv.so in-tree for gfx950.

    python -m w4a16_nvfp4_gemv_amd.build_ext

Every source under csrc/ is compiled by hipcc into one shared library that
exports the C ABI declared in include/w4a16_nvfp4_gemv.h.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw4a16_nvfp4_gemv.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


PROBE = os.path.join(HERE, "probe", "read_floor.hip")
PROBE_LIB = os.path.join(HERE, "libw4a16_read_floor.so")


def build_probe(verbose: bool = False) -> str:
    """The streaming-read reference the benchmark times beside the GEMV (a
    library of its own: nothing in the GEMV library uses it)."""
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
           PROBE, "-o", PROBE_LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return PROBE_LIB


# Code-generation flags of the library (also part of the benchmark's source
# digest: counter figures taken on code built otherwise are stale).
CODEGEN_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17",
    # packed FP32 instructions stay off (only scalar / non-packed FP32 code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs rather than AccVGPRs: the kernels read them with
    # ordinary VALU instructions (block scales, reductions, epilogues), and
    # each AccVGPR read costs a v_accvgpr_read (measured: the fused silu call
    # at 32 tokens 29.3 -> 28.4 us, the 4x4 block kernel 0.06-0.3 us faster)
    "-mllvm", "--amdgpu-mfma-vgpr-form",
]


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    cmd = [
        hipcc(), *CODEGEN_FLAGS, "-fPIC", "-shared",
        "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
        "-I", os.path.join(ROOT, "include"),
        *sources(), "-o", LIB + ".tmp",
        # the library GEMM of the dequant + GEMM path
        "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lrocblas",
    ]
    if extra:
        cmd[1:1] = extra
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probe(verbose="-v" in sys.argv))
