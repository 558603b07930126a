"""The oracle pins must reject a broken oracle.

Each case compiles a copy of oracle/nvfp4_oracle.c with one plausible mistake
planted in it (on the CPU, in a temporary directory), points the oracle
front end at that copy and runs the pin tests in a subprocess: at least one
pin has to fail for every planted mistake.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "nvfp4_oracle.c")

# (name, text in the oracle, replacement, occurrence index or None for all)
MUTANTS = [
    ("nibble_order", "(k % 2 == 0) ? (byte & 15) : (byte >> 4)", "(k % 2 == 0) ? (byte >> 4) : (byte & 15)", None),
    ("e2m1_bias", "ldexp(1.0 + 0.5 * mantissa, exponent - 1)", "ldexp(1.0 + 0.5 * mantissa, exponent - 2)", None),
    ("e2m1_subnormal", "magnitude = 0.5 * mantissa;", "magnitude = 1.0 * mantissa;", None),
    ("e4m3_bias", "ldexp(1.0 + mantissa / 8.0, exponent - 7)", "ldexp(1.0 + mantissa / 8.0, exponent - 8)", None),
    ("e4m3_sign_dropped", "return sign ? -magnitude : magnitude;", "return magnitude;", 1),
    ("swizzle_chunk_slot_swapped", "(r % 32) * 16 + (r / 32) * 4", "(r / 32) * 16 + (r % 32) * 4", None),
    ("swizzle_tile_order", "band * col_groups + c / 4", "(c / 4) * 1024 + band", None),
    ("block_of_32", "s_flat[oracle_scale_offset(n, k / 16, K)]", "s_flat[oracle_scale_offset(n, k / 32, K)]", None),
    ("ties_away", "(fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0", "fl + 1.0", None),
    ("truncate", "if (frac > 0.5)", "if (frac > 2.0)", None),
    ("x_reversed", "x[m * ldx + k]", "x[m * ldx + (K - 1 - k)]", None),
    ("global_scale_dropped", "oracle_bf16_from_f64(acc[m * N + n] * gs)", "oracle_bf16_from_f64(acc[m * N + n])", None),
    ("silu_pairs_interleaved", "acc[m * N + half + j] * gs", "acc[m * N + 2 * j + 1] * gs", None),
    ("silu_gate_unrounded", "double g = oracle_bf16_to_f64(oracle_bf16_from_f64(acc[m * N + j] * gs));", "double g = acc[m * N + j] * gs;", None),
    ("routed_alpha_dropped", "double u = au * (double)alpha[e];", "double u = au;", None),
    ("routed_gate_up_swapped", "dequant_row_nvfp4(we, se, H, I + i, row_u);", "dequant_row_nvfp4(we, se, H, i, row_u);", None),
    ("tw_dropped", "s += (double)tw[p] * y;", "s += y;", None),
    ("combine_inner_rounding_dropped", "double s_rounded = oracle_bf16_to_f64(oracle_bf16_from_f64(s));", "double s_rounded = s;", None),
    ("shared_down_dropped", "out[t * H + h] = oracle_bf16_from_f64(s_rounded + ysh);", "out[t * H + h] = oracle_bf16_from_f64(s_rounded);", None),
]


def _mutate(text: str, old: str, new: str, occurrence):
    assert old in text, old
    if occurrence is None:
        return text.replace(old, new)
    parts = text.split(old)
    assert len(parts) > occurrence + 1
    return old.join(parts[: occurrence + 1]) + new + old.join(parts[occurrence + 1:])


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_planted_mistake(name, old, new, occ):
    text = open(SRC).read()
    mutated = _mutate(text, old, new, occ)
    assert mutated != text
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "mutant.c")
        lib = os.path.join(d, "libmutant.so")
        with open(src, "w") as f:
            f.write(mutated)
        subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                        "-ffp-contract=off", src, "-o", lib, "-lm"], check=True)
        env = dict(os.environ, W4A16_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout, r.stdout[-2000:]
