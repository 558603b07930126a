"""Host logic of bench.py (no GPU): the counter-ingest arithmetic, the
source digest that marks counter figures stale, and the one-GPU guard."""
from __future__ import annotations

import csv
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (kernel, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def test_ingest_scales_each_counter_by_the_calibration_copy(tmp_path):
    k1 = "void w4a16::k_gemv_mfma<true, 4, false, 1>(w4a16::GemvParams)"
    k2 = "void w4a16::k_gemv_vchunk<1, false, 2, 4>(w4a16::GemvParams)"
    copy = "__amd_rocclr_copyBuffer"
    half = bench.CALIB_BYTES / 1024 / 2  # the copy's read counted at half its size
    _write_csv(tmp_path / "f.csv", "FETCH_SIZE", [(k1, 100.0), (k1, 300.0), (k2, 50.0), (copy, half), (copy, half),
                                                   (copy, half)])
    _write_csv(tmp_path / "w.csv", "WRITE_SIZE", [(k1, 10.0), (k1, 10.0), (k2, 5.0), (copy, bench.CALIB_BYTES / 1024)] * 1
               + [(copy, bench.CALIB_BYTES / 1024)] * 2)
    out = tmp_path / "traffic.json"
    assert bench.ingest_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(out)) == 0
    rec = json.loads(out.read_text())
    assert rec["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert rec["calibration"]["write_scale"] == pytest.approx(1.0)
    a = rec["kernels"]["k_gemv_mfma<true, 4, false, 1>"]
    assert a["fetch_kib_raw"] == pytest.approx(200.0)  # mean over launches
    assert a["bytes_per_launch"] == round(200.0 * 2 * 1024) + round(10.0 * 1024)
    assert rec["kernels"]["k_gemv_vchunk<1, false, 2, 4>"]["bytes_per_launch"] == round(50 * 2 * 1024) + 5 * 1024
    assert rec["source_digest"] == bench.source_digest()


def test_ingest_needs_the_three_calibration_copies(tmp_path):
    k = "void w4a16::k_gemv_mfma<true, 4, false, 1>(w4a16::GemvParams)"
    _write_csv(tmp_path / "f.csv", "FETCH_SIZE", [(k, 1.0), ("__amd_rocclr_copyBuffer", 1.0)])
    _write_csv(tmp_path / "w.csv", "WRITE_SIZE", [(k, 1.0)])
    with pytest.raises(SystemExit):
        bench.ingest_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "t.json"))


def test_source_digest_ignores_comments_and_tracks_code(tmp_path):
    src = os.path.join(ROOT, "w4a16_nvfp4_gemv_amd", "csrc")
    dst = tmp_path / "csrc"
    shutil.copytree(src, dst)
    base = bench.source_digest(str(dst))
    assert base == bench.source_digest()
    gemv = dst / "gemv.hip"
    text = gemv.read_text()
    gemv.write_text(text.replace("namespace w4a16 {", "// a remark\n\nnamespace w4a16 {  // another", 1))
    assert bench.source_digest(str(dst)) == base
    gemv.write_text(text.replace("namespace w4a16 {", "namespace w4a16 {\nconstexpr int kUnused = 1;", 1))
    assert bench.source_digest(str(dst)) != base


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
