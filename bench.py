#!/usr/bin/env python3
"""Benchmark of the fused block-dequantize GEMV and the MoE decode layer on
one MI355X.

Step (the headline `value`) = one pass of the dense-GEMV workload: 7168 x
7168 weights in each of FP2 (10 B / 32 weights), FP3 (14 B) and FP4 (17 B),
each with q = 1 and q = 4 activation columns (six GEMVs), run as one
grouped launch (rfx_gemv_grouped). Weights are N(0, 0.02) with 1% outliers
x10 (seeds 0 / 10 / 20); columns N(0, 1), seeds 1..q. Each format keeps R
copies of its matrix at distinct addresses (R x size >= 512 MB, twice the
256 MB last-level cache); in step i the q = 1 GEMV uses copy 2i mod R and
the q = 4 GEMV copy 2i + 1 mod R, so no two GEMVs of a step share weights
and every byte counted streams from HBM. Inputs are resident in HBM before the timed region; steps are replayed
from a HIP graph. The same step as six separate launches is reported too.

value = algorithmic bytes of the step (packed weights + quantized
activations read) / step time, in GB/s.

Extra fields: per-kernel timings, the MoE decode layer (256 experts, hidden
4096, intermediate 2048, FP2 gate/up, FP3 down, FP4 shared, q = 4, top-6)
and the 8-layer stack (top-4, Zipf(1.1) router bias, q = 1 and q = 4), the
HBM copy reference and the CPU oracle on a bounded sample. The FP2M
variant (fp16 scale + fp16 minimum, 12 B / 32 weights, seed 30) and the Q8
tier (int8 codes + fp16 scale, 34 B, seed 40) are timed per kernel beside
the named formats; they are not part of the step.

Prints one JSON line. Only one GPU is supported.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
N = K = 7168
FORMATS = (2, 3, 4)
VARIANTS = (12, 8, 16, 13)  # FP2M, Q8, FP2S and FP3E: timed per kernel, not part of the step
SEEDS = {2: 0, 3: 10, 4: 20, 12: 30, 8: 40, 16: 50, 13: 60}
FMT_NAME = {2: "FP2", 3: "FP3", 4: "FP4", 12: "FP2M", 8: "Q8", 16: "FP2S", 13: "FP3E"}
LLC_BYTES = 256 << 20
MOE_H, MOE_I, MOE_E = 4096, 2048, 256


def log(*a):
    print("#", *a, file=sys.stderr, flush=True)


def algorithmic_bytes(R, fmt, q, n=N, k=K):
    weights = n * (k // 32) * R.block_bytes(fmt)
    acts = q * k + q * (k // 32) * 8  # int8 codes + fp32 scale + int32 sum per block
    return weights, acts, q * n * 4


# ------------------------------------------------------------------ GEMV

def build_gemv(torch, R, inputgen):
    work = {}
    for fmt in FORMATS + VARIANTS:
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
        acts[q] = {"xq": xq, "xs": xs, "xsum": xsum,
                   "y": torch.empty((q, N), dtype=torch.float32, device="cuda")}
    ws = {}
    for fmt in FORMATS + VARIANTS:
        for q in (1, 4):
            n = R.gemv_workspace_bytes(work[fmt]["mats"][0], q)
            ws[(fmt, q)] = torch.zeros(n, dtype=torch.uint8, device="cuda") if n else None
    torch.cuda.synchronize()
    return work, acts, ws


def copy_index(q, i):
    """Weight copy of the q-column GEMV in step i (distinct for q = 1, 4)."""
    return 2 * i + (q > 1)


def gemv_launch(R, work, acts, ws, fmt, q, i):
    mats = work[fmt]["mats"]
    a = acts[q]
    R.gemv(mats[i % len(mats)], a["xq"], a["xs"], a["xsum"], q, a["y"], ws[(fmt, q)])


def grouped_step_jobs(torch, R, work, acts):
    """Job arrays of the grouped step, one per rotation index, and their
    (shared, zero-filled) workspace. Each job writes its own output and
    reads its own weight copy."""
    rot = max(len(work[f]["mats"]) for f in FORMATS)
    ys = {(f, q): torch.empty((q, N), dtype=torch.float32, device="cuda") for f in FORMATS for q in (1, 4)}
    arrs = []
    for i in range(rot):
        jobs = []
        for fmt in FORMATS:
            mats = work[fmt]["mats"]
            for q in (1, 4):
                a = acts[q]
                jobs.append((mats[copy_index(q, i) % len(mats)], q, a["xq"], a["xs"], a["xsum"], ys[(fmt, q)]))
        arrs.append(R.gemv_jobs(jobs))
    n = R.gemv_grouped_workspace_bytes(arrs[0])
    gws = torch.zeros(max(n, 256), dtype=torch.uint8, device="cuda")
    return arrs, gws, ys


def graph_of(torch, fn, n):
    """Capture fn(0..n-1) into one graph (after a warm-up on a side stream)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(min(n, 3)):
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, reps, prewarm=True):
    """ms per replay of g over reps timed replays, after an untimed pre-warm
    (prewarm_graph) or, with prewarm=False, one untimed replay."""
    if prewarm:
        prewarm_graph(torch, g)
    else:
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps  # ms per replay


PREWARM_S = 0.2


def prewarm_graph(torch, g):
    """Replay g until at least PREWARM_S seconds have passed; returns the
    number of replays (untimed)."""
    torch.cuda.synchronize()
    t0 = time.time()
    n = 0
    while time.time() - t0 < PREWARM_S:
        for _ in range(8):
            g.replay()
        n += 8
        torch.cuda.synchronize()
    return n


def time_eager(torch, fn, n):
    for i in range(10):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


# ------------------------------------------------------------------- MoE

def build_moe_layers(torch, R, inputgen, n_layers):
    """n_layers distinct seeded layers; each carries both routers (no bias
    for the single-layer top-6 workload, Zipf bias for the stack)."""
    layers = []
    for l in range(n_layers):
        t0 = time.time()
        wfn = (lambda layer: (lambda e, m, r, c: inputgen.expert_weight(layer, e, m, r, c)))(l)
        dev = R.DeviceMoeLayer.build(MOE_H, MOE_I, MOE_E, wfn, inputgen.router_weight(l, MOE_E, MOE_H),
                                     None, workers=16)
        zb = torch.from_numpy(inputgen.zipf_router_bias(l, MOE_E)).cuda()
        zipf = R.DeviceMoeLayer(MOE_H, MOE_I, MOE_E, dev.gate, dev.up, dev.down, dev.sh,
                                dev.router_w, zb)
        layers.append((dev, zipf))
        log(f"moe layer {l} built in {time.time() - t0:.1f} s")
    return layers


def moe_bytes(R, layer, topk_idx, q):
    """Algorithmic bytes of one layer call: router weights, shared expert,
    every distinct routed expert once, token activations and h~ read."""
    w = layer.weight_bytes(topk_idx.reshape(-1).tolist())
    k = topk_idx.shape[1]
    acts = q * MOE_H * 4 + q * MOE_H + (q * MOE_H // 32) * 8  # fp32 x (router) + x~
    acts += (q * k + q) * (MOE_I + (MOE_I // 32) * 8)          # h~ into down
    return w + acts


def bench_moe(torch, R, inputgen, layers, reps):
    out = {}
    # every layer through rfx_moe_forward (at q = 1 the gate/up workgroups
    # route themselves; at q = 4 the router launch and the FFN launches)
    # single layer, q = 4, top-6, rotated over the distinct layers
    q, k = 4, 6
    bufs = [R.MoeBuffers(lay[0], q, k) for lay in layers]
    xs = [torch.from_numpy(inputgen.tokens(l, 7, q, MOE_H)).cuda() for l in range(len(layers))]

    def one(i):
        l = i % len(layers)
        bufs[l].forward(layers[l][0], xs[l])

    for l in range(len(layers)):
        one(l)
    torch.cuda.synchronize()
    nbytes = [moe_bytes(R, layers[l][0], bufs[l].topk_idx.cpu().numpy(), q) for l in range(len(layers))]
    distinct = [len(set(bufs[l].topk_idx.cpu().numpy().reshape(-1).tolist())) for l in range(len(layers))]
    g = graph_of(torch, one, len(layers))
    ms = time_graph(torch, g, reps) / len(layers)
    avg_bytes = sum(nbytes) / len(nbytes)
    out["layer_q4_top6"] = {"us": round(ms * 1e3, 2), "bytes": int(avg_bytes),
                            "GBps": round(avg_bytes / (ms * 1e-3) / 1e9, 1),
                            "frac_hbm": round(avg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                            "distinct_experts": distinct, "rotated_layers": len(layers),
                            "eager_us": round(time_eager(torch, one, 4 * len(layers)) * 1e3, 2)}
    log(f"moe layer q=4 top-6: {ms * 1e3:.1f} us")
    # 8-layer stack, top-4, Zipf bias, residual fused into the combine
    for q in (1, 4):
        k = 4
        sb = [R.MoeBuffers(lay[1], q, k) for lay in layers]
        x0 = torch.from_numpy(inputgen.tokens(100, 0, q, MOE_H)).cuda()
        xbuf = [x0] + [torch.empty((q, MOE_H), dtype=torch.float32, device="cuda") for _ in layers]

        def step(i):
            for l, lay in enumerate(layers):
                sb[l].forward(lay[1], xbuf[l], resid=xbuf[l], out=xbuf[l + 1])

        step(0)
        torch.cuda.synchronize()
        nb = sum(moe_bytes(R, lay[1], sb[l].topk_idx.cpu().numpy(), q) for l, lay in enumerate(layers))
        hist = [len(set(sb[l].topk_idx.cpu().numpy().reshape(-1).tolist())) for l in range(len(layers))]
        g = graph_of(torch, step, 1)
        ms = time_graph(torch, g, reps)
        out[f"stack{len(layers)}_q{q}_top4_zipf"] = {
            "us_per_step": round(ms * 1e3, 2), "bytes_per_step": int(nb),
            "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "distinct_experts_per_layer": hist,
            "steps_per_s": round(1e3 / ms, 1)}
        log(f"moe stack q={q}: {ms * 1e3:.1f} us/step, {nb / (ms * 1e-3) / 1e9:.0f} GB/s")
    # the same workloads through the single-launch layer kernel
    # (rfx_moe_forward with RFX_FORWARD_ONE_LAUNCH): same results, timed
    # beside the three launches
    one = {}
    for q, k, zipf in ((1, 4, True), (4, 4, True), (4, 6, False)):
        sel = [lay[1] if zipf else lay[0] for lay in layers]
        fb = [R.MoeBuffers(d, q, k) for d in sel]
        x0 = torch.from_numpy(inputgen.tokens(100, 0, q, MOE_H) if zipf else inputgen.tokens(0, 7, q, MOE_H)).cuda()
        xb = [x0] + [torch.empty((q, MOE_H), dtype=torch.float32, device="cuda") for _ in sel]

        def fwd_step(i, sel=sel, fb=fb, xb=xb, zipf=zipf):
            for l, d in enumerate(sel):
                fb[l].forward(d, xb[l], resid=xb[l] if zipf else None, out=xb[l + 1], one_launch=True)

        fwd_step(0)
        torch.cuda.synchronize()
        ms = time_graph(torch, graph_of(torch, fwd_step, 1), reps) / len(sel)
        for l, d in enumerate(sel):
            R.moe_forward_status(d, q, k, fb[l].ws)
        one[f"q{q}_top{k}{'_zipf' if zipf else ''}_us_per_layer"] = round(ms * 1e3, 2)
        log(f"moe one launch q={q} top-{k}: {ms * 1e3:.1f} us per layer")
    out["one_launch"] = one
    f = profile_summary("moe_decode_pmc", MOE_SOURCES)
    out["traffic"] = ({k: int(v.split()[0]) for k, v in f.items() if k.endswith("_bytes")}
                      if f else None)
    return out


def bench_placement(torch, R, inputgen, layers, n_hot=64, steps=16, n_layers=2):
    """Expert placement on one GPU: the first n_layers of the Zipf(1.1)
    stack at q = 1, top-4, decoding `steps` fresh tokens; per layer the
    n_hot experts the router bias ranks highest stay in HBM and the others
    sit in pinned host memory, read by the kernels over the host link. The
    same steps with every expert in HBM for comparison. Reports us per step,
    the share of routed picks that hit host memory and the host bytes read
    per step."""
    from bit_block_quantized_amd.layer import hot_experts_by_frequency
    sel = [lay[1] for lay in layers[:n_layers]]
    placed = [R.PlacedMoeLayer(z, hot_experts_by_frequency(np.exp(z.router_b.cpu().numpy().astype(np.float64)),
                                                            n_hot)) for z in sel]
    xs = [torch.from_numpy(inputgen.tokens(100, s, 1, MOE_H)).cuda() for s in range(steps)]
    per_expert = placed[0].hbm_bytes()[0] // max(1, len(placed[0].hot))

    def measure(lays, cold_sets):
        bufs = [R.MoeBuffers(l, 1, 4) for l in lays]
        xb = [torch.empty((1, MOE_H), dtype=torch.float32, device="cuda") for _ in lays]

        def step(s):
            x = xs[s]
            for l, lay in enumerate(lays):
                bufs[l].run(lay, x, resid=x, out=xb[l])
                x = xb[l]

        cold = picks = 0
        for s in range(steps):
            step(s)
            torch.cuda.synchronize()
            for l in range(len(lays)):
                idx = bufs[l].topk_idx.cpu().numpy().reshape(-1)
                picks += idx.size
                cold += int(np.isin(idx, cold_sets[l]).sum())
        g = graph_of(torch, step, steps)
        ms = time_graph(torch, g, 3) / steps
        del g
        return ms, cold, picks

    ms_hbm, _, _ = measure(sel, [[] for _ in sel])
    ms_pl, cold, picks = measure(placed, [p.cold for p in placed])
    hb, cb = placed[0].hbm_bytes()
    host_bytes = cold * per_expert / steps
    out = {"workload": f"first {n_layers} layers of the Zipf(1.1) stack, q=1, top-4, {steps} fresh tokens; "
                       f"{n_hot} of {MOE_E} routed experts per layer in HBM, the rest in pinned host memory",
           "us_per_step_all_hbm": round(ms_hbm * 1e3, 2), "us_per_step_placed": round(ms_pl * 1e3, 2),
           "cold_pick_share": round(cold / max(1, picks), 4),
           "hbm_GiB_per_layer": round(hb / 2**30, 2), "host_GiB_per_layer": round(cb / 2**30, 2),
           "host_bytes_per_step": int(host_bytes),
           "host_link_GBps": round(host_bytes / max(1e-9, (ms_pl - ms_hbm) * 1e-3) / 1e9, 1) if ms_pl > ms_hbm
           else None}
    del placed
    torch.cuda.empty_cache()
    log(f"placement: {out}")
    return out


def bench_prefill(torch, R, inputgen, layer, reps, tokens=2048, k=6):
    """The prefill-sized layer: 2048 tokens N(0,1), top-6 over 256 experts,
    shared expert, grouped int8-MFMA FFN. Reports the whole layer's time,
    tokens/s, int8 MFMA throughput (2 ops per MAC, of the block dots) and
    the packed-weight stream."""
    buf = R.MoeBuffers(layer, tokens, k)
    x = torch.from_numpy(inputgen.tokens(0, 1000, tokens, MOE_H)).cuda()

    def one(i):
        buf.run(layer, x)

    one(0)
    torch.cuda.synchronize()
    idx = buf.topk_idx.cpu().numpy()
    g = graph_of(torch, one, 1)
    ms = time_graph(torch, g, reps)
    n_pairs = tokens * k
    macs = (n_pairs + tokens) * 3 * MOE_I * MOE_H  # gate, up, down per (token, expert)
    wbytes = layer.weight_bytes(idx.reshape(-1).tolist())
    counts = np.bincount(idx.reshape(-1), minlength=MOE_E)
    log(f"prefill {tokens} tokens top-{k}: {ms * 1e3:.1f} us, {2 * macs / (ms * 1e-3) / 1e12:.1f} int8 TOP/s")
    counters = {}
    f = profile_summary("moe_prefill_2048_pmc", PREFILL_SOURCES)
    if f:
        for key in ("MfmaUtil_pct", "VALUBusy_pct", "gateup_read_bytes", "down_read_bytes", "traffic_bytes_per_layer"):
            if key in f:
                counters[key] = float(f[key].split()[0])
    return {"counters": counters or None, "us": round(ms * 1e3, 1), "tokens": tokens, "k": k,
            "tokens_per_s": round(tokens / (ms * 1e-3), 1),
            "int8_ops": 2 * macs, "int8_TOPs": round(2 * macs / (ms * 1e-3) / 1e12, 2),
            "frac_int8_mfma_peak": round(2 * macs / (ms * 1e-3) / 5.0e15, 4),
            "weight_bytes": int(wbytes), "weight_GBps": round(wbytes / (ms * 1e-3) / 1e9, 1),
            "tokens_per_expert": {"min": int(counts.min()), "mean": round(float(counts.mean()), 1),
                                  "max": int(counts.max())},
            "timing": "HIP graph replay of route + FFN"}


GEMV_SOURCES = ("rfx_decode.h", "rfx_gemv.hip", "rfx_internal.h", "rfx_mx4.h", "rfx_xtile.h")


def kernel_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for name in sorted(GEMV_SOURCES):
        with open(os.path.join(ROOT, "bit_block_quantized_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of a GEMV kernel ("grouped", or "fp4_q4" and the
    like) from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or
    None when there is none for it or the kernel sources changed since it
    was taken."""
    path = os.path.join(ROOT, "profiles", f"gemv_{kernel}_{N}_pmc.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def hbm_reference(torch):
    """Device-to-device copy of 2 GiB: (read + write) bytes / time."""
    n = 1 << 31
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    ms = time_eager(torch, lambda i: b.copy_(a), 10)
    del a, b
    return 2 * n / (ms * 1e-3) / 1e9


def hbm_read_reference(torch, R):
    """A 4 GiB streaming read with the GEMV kernels' load form
    (rfx_read_reference, 32768 workgroups of 256 threads, the best of a
    1024..32768 sweep): bytes read / time."""
    n = 1 << 30
    a = torch.ones(n, dtype=torch.int32, device="cuda")
    out = torch.empty(32768, dtype=torch.int32, device="cuda")
    for _ in range(3):
        R.read_reference(a, out)
    ms = time_eager(torch, lambda i: R.read_reference(a, out), 10)
    del a, out
    return 4 * n / (ms * 1e-3) / 1e9


def bench_config1(torch, R, inputgen, reps):
    """FP4 1024 x 1024, q = 1 (W seed 0, x seed 1): microseconds per call
    (0.56 MB stays in L2, so the time is launch and latency), and the same
    call over 1024 distinct copies (570 MB) back to back for a rate."""
    n = 1024
    W = inputgen.dense_weight(n, n, seed=0)
    tiled = R.quantize_matrix(4, W)
    nbytes = tiled.nbytes
    copies = 1024
    base = torch.empty(copies * nbytes, dtype=torch.uint8, device="cuda")
    one = torch.from_numpy(tiled).cuda()
    for c in range(copies):
        base[c * nbytes:(c + 1) * nbytes].copy_(one)
    mats = [R.DeviceQMat(4, n, n, base[c * nbytes:(c + 1) * nbytes]) for c in range(copies)]
    x = torch.from_numpy(inputgen.activations(1, n, seed=1)).cuda()
    xq = torch.empty((1, n), dtype=torch.int8, device="cuda")
    xs = torch.empty((1, n // 32), dtype=torch.float32, device="cuda")
    xsum = torch.empty((1, n // 32), dtype=torch.int32, device="cuda")
    R.quantize_act(x, xq, xs, xsum)
    y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(R.gemv_workspace_bytes(mats[0], 1), 256), dtype=torch.uint8, device="cuda")
    g = graph_of(torch, lambda i: R.gemv(mats[0], xq, xs, xsum, 1, y, ws), 32)
    us_one = time_graph(torch, g, reps) * 1e3 / 32
    del g
    g = graph_of(torch, lambda i: R.gemv(mats[i], xq, xs, xsum, 1, y, ws), copies)
    us_rot = time_graph(torch, g, 3) * 1e3 / copies
    del g, base, mats
    w, a, _ = algorithmic_bytes(R, 4, 1, n=n, k=n)
    return {"workload": "FP4 1024x1024 q=1, W seed 0, x seed 1", "us_per_call": round(us_one, 3),
            "rotated_1024_copies": {"us_per_call": round(us_rot, 3),
                                    "GBps": round((w + a) / (us_rot * 1e-6) / 1e9, 1)},
            "bytes_per_call": w + a}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(R, work, rows=N, repeats=4):
    """The CPU oracle as it stands on a bounded sample: every row of each
    7168 x 7168 matrix, all six (format, q) products, `repeats` times; once
    on one thread and once over all host threads (the rows split into one
    contiguous chunk per thread, each chunk one call of the unchanged oracle
    GEMV; ctypes releases the GIL). Reported in GB/s of the same algorithmic
    bytes as the GPU step."""
    from concurrent.futures import ThreadPoolExecutor

    import inputgen
    import oracle as O
    blocks = {fmt: O.quantize_matrix(fmt, work[fmt]["W"][:rows]) for fmt in FORMATS}
    xq = {q: O.quantize_act(inputgen.activations(q, K, seed=1)) for q in (1, 4)}
    nbytes = repeats * sum(sum(algorithmic_bytes(R, fmt, q, n=rows)[:2]) for fmt in FORMATS for q in (1, 4))

    def run(threads):
        chunks = [(r * rows // threads, (r + 1) * rows // threads) for r in range(threads)]
        t0 = time.perf_counter()
        with ThreadPoolExecutor(threads) as ex:
            for _ in range(repeats):
                for fmt in FORMATS:
                    for q in (1, 4):
                        list(ex.map(lambda c: O.gemv(fmt, blocks[fmt][c[0]:c[1]], xq[q][0], xq[q][1]), chunks))
        return time.perf_counter() - t0

    dt1 = run(1)
    nth = host_threads()
    dtn = run(nth)
    return {"value": round(nbytes / dtn / 1e9, 4), "unit": "GB/s", "cores": nth, "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of each 7168x7168 matrix, FP2/FP3/FP4 x q=1,4, {repeats} repeats, "
                      f"{nth} threads over row chunks, {dtn:.1f} s",
            "single_thread": {"value": round(nbytes / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "seconds": round(dt1, 1)},
            "cpu_model": cpu_model()}


def cpu_moe_layer(R, inputgen, layer=0, q=4, k=6):
    """The oracle's MoE layer (routing, every pair's and the shared expert's
    FFN in fp64, combine) for the q = 4, top-6 decode workload of `layer`,
    on one thread and over all host threads (one task per (token, expert)
    pair). The experts the tokens pick are encoded by the oracle first,
    outside the timed region."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle as O
    x = inputgen.tokens(layer, 7, q, MOE_H)
    wr = inputgen.router_weight(layer, MOE_E, MOE_H)
    ref = O.route(x, wr, None, k)
    idx, w = ref["idx"], ref["w"]
    experts = sorted(set(idx.reshape(-1).tolist())) + [MOE_E]
    nth = host_threads()
    mats = {}

    def enc(em):
        e, m = em
        rows, cols = (MOE_I, MOE_H) if m < 2 else (MOE_H, MOE_I)
        fmt = 4 if e == MOE_E else (2 if m < 2 else 3)
        return em, (fmt, O.quantize_matrix(fmt, inputgen.expert_weight(layer, e, m, rows, cols)))

    with ThreadPoolExecutor(nth) as ex:
        mats.update(ex.map(enc, [(e, m) for e in experts for m in range(3)]))
    xq, xs = O.quantize_act(x)
    jobs = [(t, int(idx[t][j])) for t in range(q) for j in range(k)] + [(t, MOE_E) for t in range(q)]

    def ffn(job):
        t, e = job
        (fg, gb), (fu, ub), (fd, db) = mats[(e, 0)], mats[(e, 1)], mats[(e, 2)]
        return O.ffn(fg, gb, fu, ub, fd, db, xq[t:t + 1], xs[t:t + 1])["o"][0]

    def layer_once(threads):
        t0 = time.perf_counter()
        O.route(x, wr, None, k)
        with ThreadPoolExecutor(threads) as ex:
            o = list(ex.map(ffn, jobs))
        o_pairs = np.array(o[:q * k]).reshape(q, k, MOE_H)
        O.combine(np.array(o[q * k:]), o_pairs, w)
        return time.perf_counter() - t0

    t1 = layer_once(1)
    tn = layer_once(nth)
    wbytes = sum(R.qmat_bytes(mats[(e, m)][0], *((MOE_I, MOE_H) if m < 2 else (MOE_H, MOE_I)))
                 for e in experts for m in range(3)) + MOE_E * MOE_H * 4
    return {"workload": f"one MoE decode layer, q={q}, top-{k}, 256 experts (layer {layer}), "
                        f"{len(experts) - 1} distinct experts + shared",
            "seconds_1_thread": round(t1, 3), "seconds_all_threads": round(tn, 3), "threads": nth,
            "GBps_all_threads": round(wbytes / tn / 1e9, 4)}


def profile_summary(name, sources):
    """Fields of a committed rocprofv3 summary (profiles/<name>.txt), or
    None when it is missing or the listed kernel sources changed since it
    was taken (its kernel_sources_sha256 no longer matches)."""
    path = os.path.join(ROOT, "profiles", name + ".txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_sources_sha256") != sources_sha256(sources):
        return None
    return fields


def sources_sha256(names):
    import hashlib
    h = hashlib.sha256()
    for name in sorted(names):
        with open(os.path.join(ROOT, "bit_block_quantized_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


MOE_SOURCES = ("rfx_decode.h", "rfx_gemv.hip", "rfx_internal.h", "rfx_moe.hip", "rfx_moe_dev.h", "rfx_moe_ws.h",
               "rfx_mx4.h", "rfx_xtile.h")
PREFILL_SOURCES = ("rfx_decode.h", "rfx_internal.h", "rfx_moe.hip", "rfx_moe_dev.h", "rfx_moe_ws.h", "rfx_prefill.hip")


def profile_only(args, torch, R, inputgen):
    """--only moe / prefill: the workload launched eagerly a few times, for
    a profiler (no graphs, no timing of record)."""
    if args.only == "prefill":
        layers = build_moe_layers(torch, R, inputgen, 1)
        layer = layers[0][0]
        buf = R.MoeBuffers(layer, 2048, 6)
        x = torch.from_numpy(inputgen.tokens(0, 1000, 2048, MOE_H)).cuda()
        n = max(1, args.steps)
        ms = time_eager(torch, lambda i: buf.run(layer, x), n)
        out = {"only": "prefill", "layers_run": n + 10, "us": round(ms * 1e3, 1)}
    else:
        layers = build_moe_layers(torch, R, inputgen, max(1, args.moe_layers))
        q, k = 4, 6
        bufs = [R.MoeBuffers(lay[0], q, k) for lay in layers]
        xs = [torch.from_numpy(inputgen.tokens(l, 7, q, MOE_H)).cuda() for l in range(len(layers))]
        n = max(1, args.steps) * len(layers)
        ms4 = time_eager(torch, lambda i: bufs[i % len(layers)].forward(layers[i % len(layers)][0],
                                                                         xs[i % len(layers)]), n)
        sb = [R.MoeBuffers(lay[1], 1, 4) for lay in layers]
        x0 = torch.from_numpy(inputgen.tokens(100, 0, 1, MOE_H)).cuda()
        xbuf = [x0] + [torch.empty((1, MOE_H), dtype=torch.float32, device="cuda") for _ in layers]

        def step(i):
            for l, lay in enumerate(layers):
                sb[l].forward(lay[1], xbuf[l], resid=xbuf[l], out=xbuf[l + 1])

        ms1 = time_eager(torch, step, max(1, args.steps))
        out = {"only": "moe", "layer_q4_top6_us": round(ms4 * 1e3, 1), "stack_q1_us_per_step": round(ms1 * 1e3, 1),
               "layers": len(layers)}
    if args.copy_ref_mib:
        nb = args.copy_ref_mib << 20
        src = torch.ones(nb, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_ref_bytes"] = nb
    print(json.dumps(out), flush=True)


def per_config(out):
    """Each workload's fraction of the 8 TB/s peak, gathered in one place:
    the dense GEMV (per launch and grouped), the MoE layer, the stacks and
    prefill."""
    pc = {}
    if "config1" in out:
        c1 = out["config1"]
        pc["config1_fp4_1024_q1"] = {"us_per_call": c1["us_per_call"],
                                     "rotated_GBps": c1["rotated_1024_copies"]["GBps"],
                                     "note": "0.56 MB stays in L2: launch-latency-bound"}
    pk = {f"{p['fmt']}_q{p['q']}": p["frac_hbm"] for p in out.get("per_kernel", []) if p["fmt"] in ("FP2", "FP3", "FP4")}
    pc["config2_gemv_7168"] = {"grouped_step_frac": out["frac_hbm_peak"], "single_launch_frac": pk}
    if "moe" in out:
        m = out["moe"]
        pc["config3_moe_layer_q4_top6_frac"] = m["layer_q4_top6"]["frac_hbm"]
        pc["config4_stack8_frac"] = {"q1": m["stack8_q1_top4_zipf"]["frac_hbm"],
                                     "q4": m["stack8_q4_top4_zipf"]["frac_hbm"]}
    if "prefill" in out:
        p = out["prefill"]
        pc["config5_prefill"] = {"us": p["us"], "frac_hbm": round(p["weight_GBps"] / HBM_PEAK_GBPS, 4),
                                 "mfma_util_pct": (p.get("counters") or {}).get("MfmaUtil_pct")}
    return pc


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--kernel-reps", type=int, default=20, help="graph replays per kernel timing")
    ap.add_argument("--moe-layers", type=int, default=8, help="0 skips the MoE sections")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--moe-only", action="store_true", help="skip the GEMV step (profiling the MoE path)")
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="with --only: then run 3 plain device copies of this many MiB (counter scaling)")
    ap.add_argument("--only", default=None,
                    help="fmt,q | grouped | moe | prefill: launch only this, eagerly, for a profiler")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this benchmark measures one GPU only (the decode path has no multi-GPU part); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        print("bench.py: --steps must be at least 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_block_quantized_amd as R
    import inputgen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    R.lib()
    if args.only in ("moe", "prefill"):
        profile_only(args, torch, R, inputgen)
        return
    if args.moe_only:
        layers = build_moe_layers(torch, R, inputgen, max(1, args.moe_layers))
        print(json.dumps({"moe": bench_moe(torch, R, inputgen, layers, reps=max(5, args.steps // 5)),
                          "prefill": bench_prefill(torch, R, inputgen, layers[0][0], reps=5)}), flush=True)
        return
    work, acts, ws = build_gemv(torch, R, inputgen)
    log(f"gemv workload ready: copies {[len(work[f]['mats']) for f in FORMATS]}")

    garrs, gws, _ = grouped_step_jobs(torch, R, work, acts)
    step_bytes = sum(sum(algorithmic_bytes(R, f, q)[:2]) for f in FORMATS for q in (1, 4))
    if args.only:
        if args.only == "grouped":
            n = args.steps * len(garrs)
            ms = time_eager(torch, lambda i: R.gemv_grouped(garrs[i % len(garrs)], gws), n)
            out = {"only": "grouped", "launches": n, "us": round(ms * 1e3, 3),
                   "GBps": round(step_bytes / (ms * 1e-3) / 1e9, 1)}
        else:
            fmt, q = (int(v) for v in args.only.split(","))
            n = args.steps * len(work[fmt]["mats"])
            ms = time_eager(torch, lambda i: gemv_launch(R, work, acts, ws, fmt, q, i), n)
            w, a, _ = algorithmic_bytes(R, fmt, q)
            out = {"only": [fmt, q], "launches": n, "us": round(ms * 1e3, 3),
                   "GBps": round((w + a) / (ms * 1e-3) / 1e9, 1)}
        if args.copy_ref_mib:
            # a plain device copy of known size, so that byte counters read
            # in the same run can be scaled to bytes
            nb = args.copy_ref_mib << 20
            src = torch.ones(nb, dtype=torch.uint8, device="cuda")
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            out["copy_ref_bytes"] = nb
        print(json.dumps(out), flush=True)
        return

    per = []
    for fmt in FORMATS + VARIANTS:
        for q in (1, 4):
            copies = len(work[fmt]["mats"])
            g = graph_of(torch, lambda i: gemv_launch(R, work, acts, ws, fmt, q, i), copies)
            us = time_graph(torch, g, args.kernel_reps) * 1e3 / copies
            us_eager = time_eager(torch, lambda i: gemv_launch(R, work, acts, ws, fmt, q, i), 4 * copies) * 1e3
            w, a, wr = algorithmic_bytes(R, fmt, q)
            per.append({"fmt": FMT_NAME[fmt], "q": q, "us": round(us, 3), "eager_us": round(us_eager, 3),
                        "weight_bytes": w, "act_bytes": a, "write_bytes": wr,
                        "GBps": round((w + a) / us / 1e3, 1),
                        "frac_hbm": round((w + a) / us / 1e3 / HBM_PEAK_GBPS, 4)})
            log(f"{FMT_NAME[fmt]} q={q}: {us:.2f} us (eager {us_eager:.2f})  {(w + a) / us / 1e3:.0f} GB/s")
            del g

    # whole step: the six GEMVs as one grouped launch (the headline) and,
    # for comparison, as six launches back to back
    assert step_bytes == sum(p["weight_bytes"] + p["act_bytes"] for p in per if p["fmt"] in ("FP2", "FP3", "FP4"))
    rot = len(garrs)

    def step_six(i):
        for fmt in FORMATS:
            for q in (1, 4):
                gemv_launch(R, work, acts, ws, fmt, q, copy_index(q, i))

    g = graph_of(torch, step_six, rot)
    ms_six = time_graph(torch, g, max(1, -(-args.steps // rot))) / rot
    del g
    # the timed region: exactly --steps steps (step i: rotation i mod R),
    # one graph of that many grouped launches, replayed --warmup times
    # untimed first
    g = graph_of(torch, lambda i: R.gemv_grouped(garrs[i % rot], gws), args.steps)
    # untimed pre-warm: the same steps for at least PREWARM_S of wall clock,
    # so the timed steps run at the GPU's sustained clocks whatever --steps
    # and --warmup are (measured on MI355X: a fresh process reads ~1 us more
    # per step over the first few milliseconds of back-to-back launches)
    prewarm = prewarm_graph(torch, g)
    for _ in range(args.warmup):
        g.replay()
    ms = time_graph(torch, g, 1, prewarm=False) / args.steps
    value = step_bytes / (ms * 1e-3) / 1e9
    del g
    log(f"step: grouped {ms * 1e3:.2f} us ({value:.0f} GB/s), six launches {ms_six * 1e3:.2f} us")

    ach = value  # one launch per step: the step is the dominant kernel
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
        "config": {"workload": "dense GEMV 7168x7168: six independent GEMVs (FP2/FP3/FP4 x q=1,4) in one grouped "
                               "launch per step, rotated weight copies",
                   "rows": N, "cols": K, "formats": ["FP2", "FP3", "FP4"], "q": [1, 4],
                   "copies": {FMT_NAME[f]: len(work[f]["mats"]) for f in FORMATS},
                   "timing": "one HIP graph of --steps grouped launches after an untimed pre-warm of the same "
                             "graph (prewarm_replays, at least 0.2 s) and --warmup untimed replays",
                   "prewarm_replays": prewarm},
        "frac_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": "gemv_grouped_kernel (FP2/FP3/FP4 x q=1,4, 7168x7168)",
                     "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic("grouped"),
                     "traffic_note": "FETCH_SIZE+WRITE_SIZE per launch, scaled by a 256 MiB copy: "
                                     "profiles/gemv_grouped_7168_pmc.txt (null when the kernel sources changed "
                                     "since the counters were taken)",
                     "bytes_per_launch": step_bytes,
                     "avg_launch_us": round(ms * 1e3, 3)},
        "step_six_launches": {"us": round(ms_six * 1e3, 3),
                              "GBps": round(step_bytes / (ms_six * 1e-3) / 1e9, 1),
                              "frac_hbm": round(step_bytes / (ms_six * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "per_kernel": per,
    }
    del work
    torch.cuda.empty_cache()
    out["config1"] = bench_config1(torch, R, inputgen, args.kernel_reps)
    log(f"config 1: {out['config1']}")
    torch.cuda.empty_cache()
    props = torch.cuda.get_device_properties(0)
    out["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                     "cus": props.multi_processor_count, "hip": torch.version.hip}
    if args.moe_layers > 0:
        layers = build_moe_layers(torch, R, inputgen, args.moe_layers)
        out["moe"] = bench_moe(torch, R, inputgen, layers, reps=max(5, args.steps // 5))
        out["moe"]["placement"] = bench_placement(torch, R, inputgen, layers)
        out["prefill"] = bench_prefill(torch, R, inputgen, layers[0][0], reps=5)
        del layers
        torch.cuda.empty_cache()
    try:
        out["hbm_copy_GBps"] = round(hbm_reference(torch), 1)
        out["hbm_read_GBps"] = round(hbm_read_reference(torch, R), 1)
    except Exception as e:  # pragma: no cover
        out["hbm_copy_GBps"] = f"failed: {e}"
    out["per_config"] = per_config(out)
    if not args.no_cpu_baseline:
        import inputgen as ig
        wk = {f: {"W": ig.dense_weight(N, K, seed=SEEDS[f], outliers=True)} for f in FORMATS}
        out["cpu_baseline"] = cpu_baseline(R, wk)
        if args.moe_layers > 0:
            out["cpu_baseline"]["moe_layer"] = cpu_moe_layer(R, ig)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
