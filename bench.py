#!/usr/bin/env python3
"""Benchmark of the fused block-dequantize GEMV on one MI355X.

Step = one pass of the dense-GEMV workload: 7168 x 7168 weights in each of
FP2 (10 B / 32 weights), FP3 (14 B) and FP4 (17 B), each run with q = 1 and
q = 4 activation columns (six GEMVs). Weights are N(0, 0.02) with 1%
outliers x10 (seeds 0 / 10 / 20); columns N(0, 1), seeds 1..q. Every format
keeps R copies of its matrix at distinct addresses (R x size >= 512 MB, twice
the 256 MB last-level cache) and each launch uses the next copy, so weights
stream from HBM. Inputs are resident in HBM before timing starts.

value = algorithmic bytes of the step (packed weights + quantized
activations read) / step time, in GB/s.

Prints one JSON line. Only one GPU is supported.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
N = K = 7168
FORMATS = (2, 3, 4)
SEEDS = {2: 0, 3: 10, 4: 20}
LLC_BYTES = 256 << 20


def algorithmic_bytes(R, fmt, q, n=N, k=K):
    weights = n * (k // 32) * R.block_bytes(fmt)
    acts = q * k + q * (k // 32) * 8  # int8 codes + fp32 scale + int32 sum per block
    return weights, acts, q * n * 4


def build_workload(torch, R, inputgen):
    work = {}
    for fmt in FORMATS:
        W = inputgen.dense_weight(N, K, seed=SEEDS[fmt], outliers=True)
        tiled = R.quantize_matrix(fmt, W)
        nbytes = tiled.nbytes
        copies = max(2, -(-2 * LLC_BYTES // nbytes))
        base = torch.empty(copies * nbytes, dtype=torch.uint8, device="cuda")
        one = torch.from_numpy(tiled).cuda()
        for c in range(copies):
            base[c * nbytes:(c + 1) * nbytes].copy_(one)
        mats = [R.DeviceQMat(fmt, N, K, base[c * nbytes:(c + 1) * nbytes]) for c in range(copies)]
        work[fmt] = {"W": W, "mats": mats, "base": base}
    acts = {}
    for q in (1, 4):
        x = inputgen.activations(q, K, seed=1)
        xd = torch.from_numpy(x).cuda()
        xq = torch.empty((q, K), dtype=torch.int8, device="cuda")
        xs = torch.empty((q, K // 32), dtype=torch.float32, device="cuda")
        xsum = torch.empty((q, K // 32), dtype=torch.int32, device="cuda")
        R.quantize_act(xd, xq, xs, xsum)
        y = torch.empty((q, N), dtype=torch.float32, device="cuda")
        acts[q] = {"x": x, "xq": xq, "xs": xs, "xsum": xsum, "y": y}
    ws = {}
    for fmt in FORMATS:
        for q in (1, 4):
            n = R.gemv_workspace_bytes(work[fmt]["mats"][0], q)
            ws[(fmt, q)] = torch.zeros(n, dtype=torch.uint8, device="cuda") if n else None
    torch.cuda.synchronize()
    return work, acts, ws


def launch(R, work, acts, ws, fmt, q, i, stream):
    mats = work[fmt]["mats"]
    a = acts[q]
    R.gemv(mats[i % len(mats)], a["xq"], a["xs"], a["xsum"], q, a["y"], ws[(fmt, q)], stream)


def time_kernel(torch, R, work, acts, ws, fmt, q, iters, stream):
    for i in range(20):
        launch(R, work, acts, ws, fmt, q, i, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(iters):
        launch(R, work, acts, ws, fmt, q, i, stream)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / iters  # us per launch


def hbm_reference(torch):
    """Device-to-device copy of 2 GiB: (read + write) bytes / time."""
    n = 1 << 31
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 10
    del a, b
    return 2 * n / us / 1e3


def cpu_baseline(R, work, rows=2048, repeats=2):
    """The CPU oracle on a bounded sample: the first `rows` rows of every
    matrix, all six (format, q) products, `repeats` times, one thread."""
    import oracle as O
    blocks = {fmt: O.quantize_matrix(fmt, work[fmt]["W"][:rows]) for fmt in FORMATS}
    xq = {}
    for q in (1, 4):
        import inputgen
        x = inputgen.activations(q, K, seed=1)
        xq[q] = O.quantize_act(x)
    t0 = time.perf_counter()
    nbytes = 0
    for _ in range(repeats):
        for fmt in FORMATS:
            for q in (1, 4):
                O.gemv(fmt, blocks[fmt], xq[q][0], xq[q][1])
                w, a, _ = algorithmic_bytes(R, fmt, q, n=rows)
                nbytes += w + a
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of each 7168x7168 matrix, FP2/FP3/FP4 x q=1,4, "
                      f"{repeats} repeats, single thread, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--kernel-iters", type=int, default=300)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None, help="fmt,q: time only this GEMV (for profiling)")
    ap.add_argument("--no-split", action="store_true",
                    help="run without a workspace (no split of K across workgroups)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only (the hot path has no multi-GPU part); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_block_quantized_amd as R
    import inputgen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    R.lib()
    stream = torch.cuda.current_stream()
    work, acts, ws = build_workload(torch, R, inputgen)
    if args.no_split:
        ws = {k: None for k in ws}
    print(f"# workload ready: copies {[len(work[f]['mats']) for f in FORMATS]}", file=sys.stderr, flush=True)

    if args.only:
        fmt, q = (int(v) for v in args.only.split(","))
        us = time_kernel(torch, R, work, acts, ws, fmt, q, args.kernel_iters, stream)
        w, a, _ = algorithmic_bytes(R, fmt, q)
        print(json.dumps({"only": [fmt, q], "us": us, "GBps": (w + a) / us / 1e3}), flush=True)
        return

    per = []
    for fmt in FORMATS:
        for q in (1, 4):
            us = time_kernel(torch, R, work, acts, ws, fmt, q, args.kernel_iters, stream)
            w, a, wr = algorithmic_bytes(R, fmt, q)
            per.append({"fmt": f"FP{fmt}", "q": q, "us": round(us, 3), "weight_bytes": w,
                        "act_bytes": a, "write_bytes": wr, "GBps": round((w + a) / us / 1e3, 1),
                        "frac_hbm": round((w + a) / us / 1e3 / HBM_PEAK_GBPS, 4)})
            print(f"# FP{fmt} q={q}: {us:.2f} us  {(w + a) / us / 1e3:.0f} GB/s", file=sys.stderr, flush=True)

    # whole step: the six GEMVs back to back
    step_bytes = sum(p["weight_bytes"] + p["act_bytes"] for p in per)

    def step(i):
        for fmt in FORMATS:
            for q in (1, 4):
                launch(R, work, acts, ws, fmt, q, i, stream)

    for i in range(args.warmup):
        step(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    value = step_bytes / (ms * 1e-3) / 1e9

    dom = max(per, key=lambda p: p["us"])
    ach = (dom["weight_bytes"] + dom["act_bytes"]) / dom["us"] / 1e3
    out = {
        "metric": "packed-weight GB/s & % HBM peak for q=1/q=4 GEMV and MoE decode layer",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "dense GEMV 7168x7168, FP2/FP3/FP4 x q=1,4 per step, rotated copies",
                   "rows": N, "cols": K, "formats": ["FP2", "FP3", "FP4"], "q": [1, 4],
                   "copies": {f"FP{f}": len(work[f]["mats"]) for f in FORMATS}},
        "frac_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": f"gemv FP{dom['fmt'][-1]} q={dom['q']}",
                     "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": None,
                     "bytes_per_launch": dom["weight_bytes"] + dom["act_bytes"],
                     "avg_launch_us": dom["us"]},
        "per_kernel": per,
    }
    try:
        out["hbm_copy_GBps"] = round(hbm_reference(torch), 1)
    except Exception as e:  # pragma: no cover
        out["hbm_copy_GBps"] = f"failed: {e}"
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(R, work)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
