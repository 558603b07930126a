"""Benchmark of the small-M W4A16 NVFP4 GEMV on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the dense W4A16 GEMV sweep: M in {1,2,4,8,16,32} on
the (N, K) = (4096, 4096) and (6144, 4096) weights, 12 nvfp4_gemv calls.
Every call reads its own copy of the weight and scales: 60 copies of each
weight rotate (566 MB and 849 MB, each more than the 256 MB Infinity Cache),
so weights come from HBM.  The
12 launches of a step are captured once into a HIP graph per copy set and
replayed, so the host's launch overhead does not throttle the GPU.

value = algorithmic bytes of a step (packed weight + flat scale bytes of the
12 calls) / wall time per step, in GB/s.  Activation and output bytes are not
counted.  Each per-call figure comes from HIP events around a graph of 64
back-to-back launches of that one call shape.  The roofline object reports the
kernel with the largest share of the step.  The CPU baseline is the binary64
oracle on the host cores over a bounded sample of the same workload.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/call and achieved HBM GB/s (% of MI355X peak) at M=1,8,32"
PEAK_GBPS = 8000.0
SWEEP_M = [1, 2, 4, 8, 16, 32]
SHAPES = [(4096, 4096, 0), (6144, 4096, 1)]
COPY_SETS = 10  # step graphs; each reads 6 fresh copies of each weight


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_name(m: int, k: int, silu: bool = False) -> str:
    """Kernel instantiation the library launches for an NVFP4 call with M tokens
    and K columns (mirrors the library's dispatch: the VALU path for M <= 2
    while M activation rows fit 64 KB, the straight-line form when each lane
    of a 64-lane group owns one 64-k tile; the MFMA path otherwise)."""
    sl = str(silu).lower()
    tiles = k // 64
    if m <= 2 and m * k * 2 <= 65536:
        lpq = 64 if tiles > 32 else 32 if tiles > 16 else 16 if tiles > 8 else 8
        mt = 1 if m <= 1 else 2
        if tiles <= lpq:
            return f"k_gemv_valu1<true, {mt}, {lpq}, {sl}>"
        return f"k_gemv_valu<true, {mt}, {lpq}, {sl}, false>"
    return f"k_gemv_mfma<true, {1 if m <= 16 else 2}, {sl}>"


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w4a16_nvfp4_gemv_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(n: int, k: int) -> int:
    import synth

    return n * k // 2 + synth.flat_scale_bytes(n, k)


def cpu_baseline(budget_s: float = 15.0) -> dict:
    """The binary64 oracle, as it is, on the host cores, over the same sweep:
    whole 128-row bands of both weights for every M of the step; the number
    of bands is sized from a one-band trial so the sample takes about
    budget_s seconds (a band is a contiguous slice of codes and scales)."""
    import oracle
    import synth

    threads = min(len(os.sched_getaffinity(0)), 64)
    oracle.set_threads(threads)
    data = {(n, m): synth.dense_w4a16(m, n, k, seed=synth.seed_for(1, m, v))
            for n, k, v in SHAPES for m in SWEEP_M}

    def run(bands: int) -> tuple:
        t0 = time.perf_counter()
        nbytes = 0
        for n, k, _ in SHAPES:
            b = min(bands, n // 128)
            for m in SWEEP_M:
                d = data[(n, m)]
                w = d["w"][: 128 * b].contiguous()
                s = d["s"][: b * (k // 64) * 512].contiguous()
                oracle.nvfp4_gemv(d["x"], w, s, float(d["gs"][0]), 128 * b)
                nbytes += 128 * b * k // 2 + b * (k // 64) * 512
        return time.perf_counter() - t0, nbytes

    t1, _ = run(1)
    bands = int(max(1, min(48, budget_s / max(t1, 1e-6))))
    t, nbytes = run(bands)
    return {"value": round(nbytes / t / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the M={SWEEP_M} sweep on the first {bands} 128-row bands of the (4096,4096) and "
                      f"(6144,4096) weights ({nbytes / 1e6:.1f} MB of weight+scale bytes in {t:.1f} s, "
                      f"binary64, {threads} threads)"}


def traffic_record(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when they are missing or were taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest():
        return None
    ent = rec.get("kernels", {}).get(kernel)
    return None if ent is None else ent.get("bytes_per_launch")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--per-call-launches", type=int, default=64)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (--gpus {args.gpus} "
              "requested).  Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    import synth
    from w4a16_nvfp4_gemv_amd import _lib

    lib = _lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---------------------------------------------------------------- inputs
    calls = []  # (n, k, m, x, w_copies, s_copies, gs, out)
    for n, k, variant in SHAPES:
        base = synth.dense_w4a16(1, n, k, seed=synth.seed_for(1, 1, variant))
        w0 = base["w"].to(dev)
        s0 = base["s"].to(dev)
        copies_w = [w0] + [w0.clone() for _ in range(COPY_SETS * len(SWEEP_M) - 1)]
        copies_s = [s0] + [s0.clone() for _ in range(COPY_SETS * len(SWEEP_M) - 1)]
        for j, m in enumerate(SWEEP_M):
            d = synth.dense_w4a16(m, n, k, seed=synth.seed_for(1, m, variant))
            x = d["x"].to(dev)
            out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            calls.append(dict(n=n, k=k, m=m, j=j, x=x, gs=d["gs"].to(dev), out=out,
                              w=copies_w, s=copies_s))
    resident = sum(c["w"][0].numel() + c["s"][0].numel() for c in calls[::len(SWEEP_M)]) * COPY_SETS * len(SWEEP_M)
    log(f"weight copies resident: {resident / 1e6:.0f} MB")

    def launch(c, copy_idx, stream):
        st = lib.nvfp4_gemv(c["x"].data_ptr(), c["m"], c["k"], c["x"].stride(0),
                            c["w"][copy_idx].data_ptr(), c["s"][copy_idx].data_ptr(),
                            c["gs"].data_ptr(), c["n"], 0, c["out"].data_ptr(), stream)
        if st != 0:
            raise RuntimeError(f"nvfp4_gemv failed: {lib.w4a16_last_error().decode()}")

    step_bytes = sum(algorithmic_bytes(c["n"], c["k"]) for c in calls)

    # ---------------------------------------------------------------- graphs
    cap = torch.cuda.Stream()
    # eager run once on the capture stream: checks every call is accepted and
    # sets up the library's split-K workspace of that stream outside capture
    for c in calls:
        launch(c, 0, cap.cuda_stream)
    torch.cuda.synchronize()
    graphs = []
    for cs in range(COPY_SETS):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            h = torch.cuda.current_stream().cuda_stream
            for c in calls:
                launch(c, cs * len(SWEEP_M) + c["j"], h)
        graphs.append(g)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed steps
    for i in range(args.warmup):
        graphs[i % COPY_SETS].replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        graphs[i % COPY_SETS].replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"{args.steps} steps: {ms_per_step * 1e3:.2f} us/step wall, {gpu_ms * 1e3 / args.steps:.2f} us/step events")

    # ---------------------------------------------------------------- per call
    per_call = []
    L = args.per_call_launches
    for c in calls:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            h = torch.cuda.current_stream().cuda_stream
            for i in range(L):
                launch(c, i % (COPY_SETS * len(SWEEP_M)), h)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (reps * L)
        nbytes = algorithmic_bytes(c["n"], c["k"])
        per_call.append({"N": c["n"], "K": c["k"], "M": c["m"], "kernel": kernel_name(c["m"], c["k"]),
                         "us": round(us, 3), "GBps": round(nbytes / us / 1e3, 1),
                         "frac_peak": round(nbytes / us / 1e3 / PEAK_GBPS, 4), "bytes": nbytes})
        log(f"N={c['n']} K={c['k']} M={c['m']:2d}: {us:7.3f} us/call {nbytes / us / 1e3:8.1f} GB/s")
        del g

    # dominant kernel: largest share of the step's time
    share = {}
    for pc in per_call:
        s = share.setdefault(pc["kernel"], {"us": 0.0, "bytes": 0, "launches": 0})
        s["us"] += pc["us"]
        s["bytes"] += pc["bytes"]
        s["launches"] += 1
    dom = max(share, key=lambda k: share[k]["us"])
    d = share[dom]
    avg_us = d["us"] / d["launches"]
    avg_bytes = d["bytes"] / d["launches"]
    achieved = avg_bytes / avg_us / 1e3
    traffic = traffic_record(dom)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic,
                "kernel": dom, "avg_us_per_launch": round(avg_us, 3),
                "algorithmic_bytes_per_launch": int(avg_bytes), "launches_per_step": d["launches"]}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = cpu_baseline(args.cpu_budget)

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dense W4A16 NVFP4 GEMV sweep M in {1,2,4,8,16,32} x (N,K) in "
                               "{(4096,4096),(6144,4096)}, bf16 x ~N(0,1), uniform codes, E4M3 "
                               "scales in [2^-4,2^4], gs=1/64; 12 calls per step",
                   "calls_per_step": len(calls), "algorithmic_bytes_per_step": step_bytes,
                   "weight_copies_MB": round(resident / 1e6)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_call": per_call,
        "source_digest": source_digest(),
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
