#!/usr/bin/env python3
"""Benchmark of the routed MoE FFN layer on one MI355X.

Headline: MoE-layer prefill throughput (tokens/s) on the 6144-token chunk
(T=6144, H=2048, I=512, E=512, top-10, int4 g=64).  One step = one layer
invocation = route + permute + ffn (fused weighted combine) on inputs already
resident in HBM, the weight codes in the tiled layout (STRATA_L_TILED,
converted once when the weights are loaded; --layout rows for row-major).
Also reported on the same JSON line:

* roofline of the dominant kernel, timed with HIP events the library records
  around its own launches (on the launch stream), over a second timed region
  of the same length;
* decode: microseconds per step on the T=4 draft-verify layer (E=512, top-10),
  cycling through 64 pre-drawn steps so each step touches a fresh expert
  subset, with its HBM roofline;
* the fp64 CPU oracle timed on this host on a bounded sample of the prefill
  workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer prefill tokens/s @6144-tok chunk; decode µs/step; % roofline"
PEAK_MFMA_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
_CSRC = "quantized_expert_ffn_histogram_amd/csrc/"
KERNEL_SOURCES = {
    "gemm_gateup": [_CSRC + "ffn_gemm.hip"],
    "gemm_down": [_CSRC + "ffn_gemm.hip"],
    "gemv_gateup": [_CSRC + "ffn_gemv.hip", _CSRC + "gemv_dev.h"],
    "gemv_down": [_CSRC + "ffn_gemv.hip", _CSRC + "gemv_dev.h"],
    "decode_route_gateup": [_CSRC + f for f in ("decode.hip", "gemv_dev.h", "route_dev.h", "permute_dev.h")],
    "decode_down_combine": [_CSRC + f for f in ("decode.hip", "gemv_dev.h", "route_dev.h", "permute_dev.h")],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(kernel: str) -> str | None:
    rels = KERNEL_SOURCES.get(kernel)
    if rels is None:
        return None
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counted_traffic(kernel: str, workload: str, layout: str = "tiled"):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current source of the kernel with weight codes in `layout`;
    otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get(f"{kernel}@{workload}")
    if not rec or rec.get("source_sha") != source_sha(kernel) or rec.get("layout") != layout:
        return None
    return rec.get("bytes_per_launch")


# rocprofv3 kernel names -> library kernel names (and the workload bench.py runs them on)
COUNTED_KERNELS = {
    "moe_gemm_wide<0, ": ("gemm_gateup", "prefill"),
    "moe_gemm_wide<1, ": ("gemm_down", "prefill"),
    "moe_gemm_general<0, ": ("gemm_gateup", "prefill"),
    "moe_gemm_general<1, ": ("gemm_down", "prefill"),
    "gemv_gateup_kernel": ("gemv_gateup", "decode"),
    "gemv_down_kernel": ("gemv_down", "decode"),
    "decode_route_gateup_kernel": ("decode_route_gateup", "decode"),
    "decode_down_combine_kernel": ("decode_down_combine", "decode"),
}


def record_traffic(fetch_csv: str, write_csv: str, prefill_workload: str, decode_workload: str = "decode",
                   layout: str = "tiled") -> dict:
    """HBM bytes per launch from two rocprofv3 --pmc runs of this script with
    --calibrate-copy (FETCH_SIZE, then WRITE_SIZE; both in KiB per dispatch).
    Each counter is scaled by what it reads for the 1 GiB device copy that
    --calibrate-copy makes (the largest copy dispatch in the run)."""
    import csv
    import collections

    def per_kernel(path, counter):
        vals = collections.defaultdict(list)
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return vals

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    gib = float(1 << 30)
    copy_f = max(max(v) for k, v in fetch.items() if "copyBuffer" in k or "copy_kernel" in k)
    copy_w = max(max(v) for k, v in write.items() if "copyBuffer" in k or "copy_kernel" in k)
    f_scale, w_scale = gib / (copy_f * 1024), gib / (copy_w * 1024)
    out = {"_calibration": {"copy_bytes": int(gib), "fetch_kib": copy_f, "write_kib": copy_w,
                            "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)}}
    for pattern, (kernel, kind) in COUNTED_KERNELS.items():
        fk = [v for k, vs in fetch.items() if pattern in k for v in vs]
        wk = [v for k, vs in write.items() if pattern in k for v in vs]
        if not fk or not wk:
            continue
        fb = float(np.mean(fk)) * 1024 * f_scale
        wb = float(np.mean(wk)) * 1024 * w_scale
        workload = prefill_workload if kind == "prefill" else decode_workload
        out[f"{kernel}@{workload}"] = {
            "fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb),
            "dispatches": min(len(fk), len(wk)), "source_sha": source_sha(kernel), "layout": layout}
    return out


def expert_weight_bytes(cfg, matrices: int = 3) -> int:
    """Packed codes + fp16 scales (+ zero points or fifth bits) of `matrices`
    H x I matrices of one expert."""
    n = matrices * cfg.H * cfg.I
    extra = {"int4": 0, "int4_asym": n // cfg.g // 2, "int5": n // 8}[getattr(cfg, "fmt", "int4")]
    return n // 2 + 2 * (n // cfg.g) + extra


def kernel_work(kernel: str, cfg, pairs: int, distinct: int):
    """Algorithmic work of one launch: (amount, unit, bound)."""
    P, H, I = pairs, cfg.H, cfg.I
    if kernel == "gemm_gateup":
        return 4.0 * P * H * I, "flop", "mfma"
    if kernel == "gemm_down":
        return 2.0 * P * H * I, "flop", "mfma"
    if kernel == "gemv_gateup":  # gate + up weights of the selected experts, plus x
        return float(distinct * expert_weight_bytes(cfg, 2) + cfg.T * H * 2), "byte", "hbm"
    if kernel == "gemv_down":  # down weights of the selected experts, plus out
        return float(distinct * expert_weight_bytes(cfg, 1) + cfg.T * H * 4), "byte", "hbm"
    if kernel == "decode_route_gateup":  # gate + up weights of the selected experts, x and logits
        return float(distinct * expert_weight_bytes(cfg, 2) + cfg.T * (H * 2 + cfg.E * 4)), "byte", "hbm"
    if kernel == "decode_down_combine":  # down weights of the selected experts, plus out
        return float(distinct * expert_weight_bytes(cfg, 1) + cfg.T * H * 4), "byte", "hbm"
    return None, None, None


def time_region(fn, steps: int):
    import torch

    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / 1e3  # seconds


def warm_up(fn, min_steps: int, min_secs: float = 0.2, max_steps: int = 2000) -> int:
    """Untimed steps until at least min_steps ran and min_secs of device work
    passed (the clock ramps up after the idle of a host-to-device upload);
    returns the number of steps."""
    import torch

    n = 0
    t0 = time.perf_counter()
    while n < min_steps or (time.perf_counter() - t0 < min_secs and n < max_steps):
        for _ in range(4):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    return n


def step_percentiles(fn, steps: int, total: bool = False) -> dict:
    """Per-step device time (HIP events around each step): p10 / p50 / p90 in
    us; with total, also the number of steps and the region's wall time."""
    import torch

    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    out = {"p10_us": round(float(np.percentile(t, 10)), 2), "p50_us": round(float(np.percentile(t, 50)), 2),
           "p90_us": round(float(np.percentile(t, 90)), 2)}
    if total:
        out.update(steps=steps, seconds=round(wall, 3), mean_us=round(float(t.mean()), 2))
    return out


def kernel_table(qe):
    rows = {}
    for name in qe.timing_kernels():
        n, ms = qe.timing_query(name)
        if n:
            rows[name] = dict(launches=n, avg_us=1e3 * ms / n, total_ms=ms)
    return rows


def roofline_of(kernel: str, avg_us: float, cfg, pairs: int, distinct: int, workload: str, layout: str = "tiled"):
    work, unit, bound = kernel_work(kernel, cfg, pairs, distinct)
    if work is None:
        return None
    if unit == "flop":
        achieved = work / (avg_us * 1e-6) / 1e12
        peak, u = PEAK_MFMA_TFLOPS, "TFLOP/s"
    else:
        achieved = work / (avg_us * 1e-6) / 1e9
        peak, u = PEAK_HBM_GBS, "GB/s"
    return {
        "kernel": kernel,
        "bound": bound,
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": u,
        "frac": round(achieved / peak, 4),
        "traffic": counted_traffic(kernel, workload, layout),
        "avg_us": round(avg_us, 2),
        "work_per_launch": work,
        "work_unit": unit,
    }


def bench_prefill(qe, args):
    import torch

    import synth

    cfg = synth.config(args.workload)
    t0 = time.time()
    inp = synth.make_inputs(cfg)
    log(f"[bench] inputs for {cfg.name} drawn in {time.time() - t0:.1f}s")
    dev = torch.device("cuda:0")
    logits = torch.from_numpy(inp.logits).to(dev)
    x = torch.from_numpy(inp.x_bf16.view(np.int16)).to(dev).view(torch.bfloat16)
    experts = qe.QuantizedExperts.from_numpy(inp.weights, cfg.g, dev, layout=args.layout)
    # The step is one strata_moe_layer call (fused mode); with --fused 0 the
    # four calls of the deterministic unfused mode.  The four separate calls of
    # the fused mode are timed beside it: each is a host call of its own, and
    # at this size the GPU waits for the host between them.
    run = qe.LayerRunner(experts, cfg.T, cfg.E, cfg.k, fused=bool(args.fused), device=dev, single_call=True)
    run4 = qe.LayerRunner(experts, cfg.T, cfg.E, cfg.k, fused=bool(args.fused), device=dev)

    # The four separate calls are timed first (context); then W warmup steps
    # and exactly args.steps layer calls in one region bracketed by
    # synchronizations: the headline.  After it, a steady-state region of at
    # least 200 steps and --steady-secs seconds with events around every
    # step: median and p10/p90 under sustained load, as the clock settles.
    for _ in range(args.warmup):
        run4(logits, x)
    secs4 = time_region(lambda i: run4(logits, x), args.steps)
    for _ in range(args.warmup):
        run(logits, x)
    secs = time_region(lambda i: run(logits, x), args.steps)
    log(f"[bench] {cfg.name}: {args.steps} steps in {secs * 1e3:.2f} ms "
        f"(four separate calls: {secs4 * 1e3:.2f} ms)")
    # The output of the timed steps, kept for the parity gate.
    timed = {k_: getattr(run, k_).detach().cpu().numpy() for k_ in ("ids", "counts", "offsets", "perm", "inv", "out")}
    timed["w"] = run.w.detach().cpu().numpy()
    steady = None
    if args.steady_secs > 0:
        n_ss = max(200, int(np.ceil(args.steady_secs / (secs / args.steps))))
        steady = step_percentiles(lambda i: run(logits, x), n_ss, total=True)
        steady["tokens_per_s_p50"] = round(cfg.T / (steady["p50_us"] * 1e-6), 1)
        log(f"[bench] {cfg.name}: steady state over {n_ss} steps: {steady}")

    qe.timing_enable(True)
    secs_timed = time_region(lambda i: run(logits, x), args.steps)
    table = kernel_table(qe)
    qe.timing_enable(False)
    for k_, v in table.items():
        log(f"[bench]   {k_:16s} launches={v['launches']:5d} avg={v['avg_us']:9.2f} us")

    distinct = int((run.counts > 0).sum().item())  # experts this layer call touches
    dominant = max(table, key=lambda n: table[n]["total_ms"])
    roof = roofline_of(dominant, table[dominant]["avg_us"], cfg, cfg.T * cfg.k, distinct, cfg.name, args.layout)
    kernels = {n: round(v["avg_us"], 2) for n, v in table.items()}
    return cfg, inp, secs, secs_timed, roof, kernels, secs4, steady, timed


def bench_decode(qe, args, name: str = "decode", layout: str | None = None):
    import torch

    import synth

    cfg = synth.config(name)
    inp = synth.make_inputs(cfg)
    steps = synth.decode_steps(cfg, 64)
    dev = torch.device("cuda:0")
    layout = layout or args.layout
    experts = qe.QuantizedExperts.from_numpy(inp.weights, cfg.g, dev, layout=layout)
    L = [torch.from_numpy(lg).to(dev) for lg, _ in steps]
    X = [torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16) for _, xb in steps]
    # The step is one strata_moe_layer call (two kernels at this size); the
    # four separate calls are timed beside it for reference.
    run = qe.LayerRunner(experts, cfg.T, cfg.E, cfg.k, fused=True, device=dev, single_call=True)
    run4 = qe.LayerRunner(experts, cfg.T, cfg.E, cfg.k, fused=True, device=dev)
    n = len(steps)
    distinct = []
    for i in range(n):  # also counts the experts each pre-drawn step touches
        run(L[i], X[i])
        distinct.append(int((run.counts > 0).sum().item()))
    for i in range(args.warmup):
        run(L[i % n], X[i % n])
    K = args.decode_steps
    secs = time_region(lambda i: run(L[i % n], X[i % n]), K)
    qe.timing_enable(True)
    time_region(lambda i: run(L[i % n], X[i % n]), K)
    table = kernel_table(qe)
    qe.timing_enable(False)
    avg_distinct = float(np.mean([distinct[i % n] for i in range(K)]))
    step_bytes = avg_distinct * expert_weight_bytes(cfg) + cfg.T * (cfg.H * 2 + cfg.E * 4 + cfg.k * 8 + cfg.H * 4)
    us = secs / K * 1e6
    kern = {}
    for name in ("decode_route_gateup", "decode_down_combine"):
        if name in table:
            r = roofline_of(name, table[name]["avg_us"], cfg, cfg.T * cfg.k, avg_distinct, cfg.name, layout)
            kern[name] = {k_: r[k_] for k_ in ("avg_us", "achieved", "frac", "traffic")}
    device_us = sum(v["total_ms"] for v in table.values()) * 1e3 / K
    pct = step_percentiles(lambda i: run(L[i % n], X[i % n]), min(K, 500))
    for i in range(args.warmup):
        run4(L[i % n], X[i % n])
    secs4 = time_region(lambda i: run4(L[i % n], X[i % n]), K)
    qe.timing_enable(True)
    time_region(lambda i: run4(L[i % n], X[i % n]), min(K, 500))
    table4 = kernel_table(qe)
    qe.timing_enable(False)

    # The same steps replayed from HIP graphs, one captured per pre-drawn step
    # (launch cost off the host); each graph's output is checked against the
    # eager step first.
    graph = None
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(3):
                run(L[i], X[i])
        torch.cuda.current_stream().wait_stream(side)
        graphs = []
        for i in range(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run(L[i], X[i])
            graphs.append(g)
        for i in (0, n // 2, n - 1):
            ref = run(L[i], X[i]).clone()
            graphs[i].replay()
            torch.cuda.synchronize()
            if not torch.equal(run.out, ref):
                raise RuntimeError(f"graph replay of step {i} differs from the eager step")
        for i in range(args.warmup):
            graphs[i % n].replay()
        gsecs = time_region(lambda i: graphs[i % n].replay(), K)
        graph = {"us_per_step": round(gsecs / K * 1e6, 2),
                 "hbm_frac_step": round(step_bytes / gsecs * K / 1e9 / PEAK_HBM_GBS, 4)}
        del graphs
    except Exception as exc:  # reported, not hidden
        graph = {"error": str(exc)}
    shared = "" if cfg.draft_sigma is None else f", drafts' logits = token 0's + {cfg.draft_sigma} N(0,1)"
    return {
        "workload": f"{cfg.name}: T={cfg.T} (1 token + {cfg.T - 1} drafts{shared}) H={cfg.H} I={cfg.I} E={cfg.E} "
                    f"k={cfg.k} g={cfg.g}, 64 rotating steps",
        "weight_layout": layout,
        "distinct_experts_per_step": round(avg_distinct, 2),
        "us_per_step": round(us, 2),
        "device_us_per_step": round(device_us, 2),
        "step_percentiles": pct,
        "graph_replay": graph,
        "steps": K,
        "alg_bytes_per_step": int(step_bytes),
        "hbm_frac_step": round(step_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "kernels_us": {n: round(v["avg_us"], 2) for n, v in table.items()},
        "roofline": kern,
        "four_calls": {"us_per_step": round(secs4 / K * 1e6, 2),
                       "kernels_us": {n: round(v["avg_us"], 2) for n, v in table4.items()}},
    }


def layer_work(cfg, distinct: int):
    """Algorithmic work of one whole layer call: (flops, bytes)."""
    flops = 6.0 * cfg.T * cfg.k * cfg.H * cfg.I
    nbytes = distinct * expert_weight_bytes(cfg) + cfg.T * (cfg.H * 2 + cfg.E * 4 + cfg.k * 8 + cfg.H * 4)
    return flops, nbytes


def bench_secondary(qe, args):
    """The other configurations, each timed the same way as the headline one
    (whole layer, inputs resident, HIP events, after at least 0.2 s of
    untimed steps), against the roofline that
    bounds it: HBM for small-batch prefill, the matrix cores for the skewed
    large-chunk prefill and for the 6144-token chunk with 32- and 128-wide
    scale groups; the tiny case is launch-latency bound."""
    import torch

    import synth

    out = {}
    dev = torch.device("cuda:0")
    # (record, workload, bound, steps, one strata_moe_layer call per step
    # instead of the separate calls, weight layout); then the other weight
    # formats, and the headline prefill chunk with the codes in the other
    # layout.
    other = "rows" if args.layout == "tiled" else "tiled"
    L = args.layout
    for key, name, bound, steps, single, layout in (
            ("tiny", "tiny", None, 200, False, L), ("prefill512", "prefill512", "hbm", 50, False, L),
            ("zipf6144", "zipf6144", "mfma", 10, False, L), ("prefill6144_g32", "prefill6144_g32", "mfma", 50, False, L),
            ("prefill6144_g128", "prefill6144_g128", "mfma", 50, False, L),
            ("prefill6144_asym", "prefill6144_asym", "mfma", 30, True, L),
            ("prefill6144_int5", "prefill6144_int5", "mfma", 30, True, L),
            ("decode_asym", "decode_asym", "hbm", 500, True, L), ("decode_int5", "decode_int5", "hbm", 500, True, L),
            (f"prefill6144_{other}", "prefill6144", "mfma", 30, True, other)):
        cfg = synth.config(name)
        inp = synth.make_inputs(cfg)
        logits = torch.from_numpy(inp.logits).to(dev)
        x = torch.from_numpy(inp.x_bf16.view(np.int16)).to(dev).view(torch.bfloat16)
        experts = qe.QuantizedExperts.from_numpy(inp.weights, cfg.g, dev, layout=layout)
        run = qe.LayerRunner(experts, cfg.T, cfg.E, cfg.k, fused=True, device=dev, single_call=single)
        warm = warm_up(lambda i: run(logits, x), max(args.warmup, 3))
        secs = time_region(lambda i: run(logits, x), steps)
        distinct = int((run.counts > 0).sum().item())
        flops, nbytes = layer_work(cfg, distinct)
        us = secs / steps * 1e6
        rec = {"workload": f"{cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} g={cfg.g}",
               "weights": cfg.fmt, "layout": layout,
               "call": "strata_moe_layer" if single else "route + permute + ffn",
               "us_per_step": round(us, 2), "tokens_per_s": round(cfg.T / (us * 1e-6), 1), "steps": steps,
               "warmup_steps": warm,
               "distinct_experts": distinct, "alg_flops": flops, "alg_bytes": int(nbytes)}
        if bound == "hbm":
            rec["roofline"] = {"bound": "hbm", "frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        elif bound == "mfma":
            rec["roofline"] = {"bound": "mfma", "frac": round(flops / (us * 1e-6) / 1e12 / PEAK_MFMA_TFLOPS, 4)}
        out[key] = rec
        log(f"[bench] {key}: {us:.1f} us/step")
        del experts, run, logits, x, inp
        torch.cuda.empty_cache()
    out["router6144"] = bench_router(qe, args)
    return out


def bench_router(qe, args):
    """The router projection in front of the top-k (strata_moe_router) at the
    prefill chunk's shape: T=6144 tokens, H=2048, E=512 router rows, k=10.
    Work: 2*T*H*E flops of bf16 matmul; bytes: x and W_r read once, fp32
    logits written, ids and weights written."""
    import torch

    import synth

    T, H, E, k = 6144, 2048, 512, 10
    dev = torch.device("cuda:0")
    xb, wb = synth.make_router(T, H, E, seed=61)
    x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(wb.view(np.int16)).to(dev).view(torch.bfloat16)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    lib = qe.load()
    stream = torch.cuda.current_stream().cuda_stream

    def call(_i):
        rc = lib.strata_moe_router(x.data_ptr(), T, H, w.data_ptr(), E, k, logits.data_ptr(), ids.data_ptr(),
                                   wts.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(lib.strata_moe_last_error().decode())

    steps = 50
    for i in range(max(args.warmup, 3)):
        call(i)
    secs = time_region(call, steps)
    qe.timing_enable(True)
    for i in range(10):
        call(i)
    torch.cuda.synchronize()
    kern = {n: round(qe.timing_query(n)[1] / max(qe.timing_query(n)[0], 1) * 1e3, 2) for n in qe.timing_kernels()}
    qe.timing_enable(False)
    us = secs / steps * 1e6
    flops = 2.0 * T * H * E
    nbytes = T * H * 2 + E * H * 2 + T * E * 4 + T * k * 8
    proj_us = kern.get("router_logits")
    log(f"[bench] router6144: {us:.1f} us/call {kern}")
    return {"workload": f"router6144: T={T} H={H} E={E} k={k} (bf16 projection, then top-k)",
            "us_per_call": round(us, 2), "steps": steps, "kernels_us": kern, "alg_flops": flops, "alg_bytes": nbytes,
            "roofline_projection": None if not proj_us else {
                "mfma_frac": round(flops / (proj_us * 1e-6) / 1e12 / PEAK_MFMA_TFLOPS, 4),
                "hbm_frac": round((T * H * 2 + E * H * 2 + T * E * 4) / (proj_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}}


def bench_kv(qe, args):
    """The 4-bit KV cache: encoding a prefill chunk's keys and values
    (T = 6144 tokens x 8 KV heads x 128, bf16 in, codes + scales out), and
    sparse attention of one decode step (1 + 3 draft tokens, 32 query heads
    over 8 KV heads) over 2048 selected positions of a 128k-position cache.
    Both are HBM-bound: algorithmic bytes are the inputs read once and the
    outputs written once (for attention: the selected key and value rows,
    q and out)."""
    import torch

    import synth

    dev = torch.device("cuda:0")
    res = {}
    # Encode: K and V of a 6144-token chunk.
    T, Hkv, D, L = 6144, 8, 128, 131072
    g = torch.Generator(device=dev).manual_seed(97)
    xk = torch.randn((T, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
    xv = torch.randn((T, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
    codes_k = torch.empty((L, Hkv, D // 2), dtype=torch.uint8, device=dev)
    codes_v = torch.empty_like(codes_k)
    sc_k = torch.empty((L, Hkv), dtype=torch.float16, device=dev)
    sc_v = torch.empty_like(sc_k)
    slots = torch.arange(T, dtype=torch.int32, device=dev) + 1000

    def enc(_i):  # keys and values in one strata_kv_quantize_pair launch
        qe.kv_quantize_pair(xk, xv, slots, codes_k, sc_k, codes_v, sc_v)

    def enc2(_i):  # the same as two strata_kv_quantize calls
        qe.kv_quantize(xk, slots, codes_k, sc_k)
        qe.kv_quantize(xv, slots, codes_v, sc_v)

    nbytes = 2 * (T * Hkv * D * 2 + T * Hkv * (D // 2 + 2))
    for name, fn in (("encode", enc), ("encode_two_calls", enc2)):
        for i in range(5):
            fn(i)
        steps = 200
        secs = time_region(fn, steps)
        us = secs / steps * 1e6
        res[name] = {"workload": f"K and V of T={T} tokens x Hkv={Hkv} x D={D} (bf16) into a 4-bit cache"
                                 + (", one strata_kv_quantize_pair call" if fn is enc else ", two calls"),
                     "us_per_step": round(us, 2), "alg_bytes": nbytes,
                     "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    # Sparse attention of a decode step over the 128k cache.
    for name in ("attn_decode128k", "attn_chunk16"):
        inp = synth.make_attn_inputs(name)
        cfg = inp.cfg
        kc = torch.empty((cfg.L, cfg.Hkv, cfg.D // 2), dtype=torch.uint8, device=dev)
        vc = torch.empty_like(kc)
        ks = torch.empty((cfg.L, cfg.Hkv), dtype=torch.float16, device=dev)
        vs = torch.empty_like(ks)
        allpos = torch.arange(cfg.L, dtype=torch.int32, device=dev)
        qe.kv_quantize(torch.from_numpy(inp.k_bf16.view(np.int16)).to(dev).view(torch.bfloat16), allpos, kc, ks)
        qe.kv_quantize(torch.from_numpy(inp.v_bf16.view(np.int16)).to(dev).view(torch.bfloat16), allpos, vc, vs)
        q = torch.from_numpy(inp.q_bf16.view(np.int16)).to(dev).view(torch.bfloat16)
        sel = torch.from_numpy(inp.sel).to(dev)
        out = torch.empty((cfg.Tq, cfg.Hq, cfg.D), dtype=torch.float32, device=dev)
        ws = torch.empty(qe.load().strata_sparse_attention_workspace_size(cfg.Tq, cfg.Hq, cfg.n_sel),
                         dtype=torch.uint8, device=dev)

        def attn(_i):
            qe.sparse_attention(q, kc, ks, vc, vs, sel, cfg.sm_scale, out=out, workspace=ws)

        for i in range(10):
            attn(i)
        steps = 2000
        secs = time_region(attn, steps)
        us = secs / steps * 1e6
        qe.timing_enable(True)
        time_region(attn, 200)
        kern = {n: round(qe.timing_query(n)[1] / max(qe.timing_query(n)[0], 1) * 1e3, 2) for n in qe.timing_kernels()}
        qe.timing_enable(False)
        pct = step_percentiles(attn, 500)
        rows = cfg.Tq * cfg.n_sel * cfg.Hkv * 2 * (cfg.D // 2 + 2)
        nbytes = rows + cfg.Tq * cfg.n_sel * 4 + cfg.Tq * cfg.Hq * cfg.D * (2 + 4)
        res[name] = {"workload": f"{name}: Tq={cfg.Tq} Hq={cfg.Hq} Hkv={cfg.Hkv} D={cfg.D} L={cfg.L} "
                                 f"n_sel={cfg.n_sel} (4-bit cache, selected rows only)",
                     "us_per_call": round(us, 2), "step_percentiles": pct, "kernels_us": kern,
                     "alg_bytes": int(nbytes), "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        log(f"[bench] {name}: {us:.2f} us/call {kern}")
        del kc, vc, ks, vs, q, sel, out, ws, inp
        torch.cuda.empty_cache()
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, repeats: int = 3):
    """The fp64 oracle on this host over the whole prefill layer (route, grouping,
    per-expert dequant + SwiGLU, combine): median wall time of `repeats` runs.
    Returns the record and the oracle's output (for the parity gate)."""
    import oracle

    try:
        import threadpoolctl

        info = threadpoolctl.threadpool_info()
        threads = max(p.get("num_threads", 1) for p in info) or 1
        blas = ", ".join(sorted({f"{p.get('internal_api')} {p.get('num_threads')} threads" for p in info}))
    except Exception:  # pragma: no cover
        threads, blas = 1, "unknown"
    times, ref = [], None
    for _ in range(repeats):
        t0 = time.perf_counter()
        ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
        times.append(time.perf_counter() - t0)
    secs = float(np.median(times))
    rec = {
        "value": round(cfg.T / secs, 2),
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"the whole {cfg.name} layer ({cfg.T} tokens), median of {repeats} runs, fp64 NumPy with "
                  "BLAS threads",
        "seconds": round(secs, 2),
        "runs_s": [round(t, 2) for t in times],
        "affinity_cores": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
        "blas": blas,
    }
    return rec, ref


def parity_gate(timed: dict, ref: dict) -> dict:
    """Compare the output of the timed steps with the oracle: routing ids and
    grouping bit-exact, routing weights within 1e-6, out within max |err| <=
    2e-2 RMS(out) and sum |err| / sum |ref| <= 5e-3 over every element."""
    res = {}
    for key, rkey in (("ids", "ids"), ("counts", "counts"), ("offsets", "offsets"), ("perm", "perm"),
                      ("inv", "inv_perm")):
        res[f"{rkey}_bitexact"] = bool(np.array_equal(timed[key].reshape(-1), ref[rkey].reshape(-1)))
    res["w_max_abs_err"] = float(np.abs(timed["w"].astype(np.float64) - ref["w"]).max())
    out = timed["out"].astype(np.float64)
    err = np.abs(out - ref["out"])
    rms = float(np.sqrt(np.mean(ref["out"] ** 2)))
    res["max_err_over_rms"] = float(err.max() / rms)
    res["l1_rel"] = float(err.sum() / np.abs(ref["out"]).sum())
    res["elements"] = int(out.size)
    ok = (all(v for k_, v in res.items() if k_.endswith("_bitexact")) and res["w_max_abs_err"] <= 1e-6
          and res["max_err_over_rms"] <= 2e-2 and res["l1_rel"] <= 5e-3 and bool(np.all(np.isfinite(out))))
    res["status"] = "ok" if ok else "FAIL"
    return res


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=2000)
    ap.add_argument("--workload", default="prefill6144")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the tiny / prefill512 / zipf6144 lines")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true",
                    help="with --no-cpu-baseline: skip the oracle comparison of the headline output (profiling)")
    ap.add_argument("--steady-secs", type=float, default=3.0,
                    help="length of the steady-state prefill region with per-step percentiles (0: skip)")
    ap.add_argument("--fused", type=int, default=1, help="1: fused weighted scatter-add; 0: y rows + combine")
    ap.add_argument("--layout", choices=("tiled", "rows"), default="tiled",
                    help="byte layout of the packed weight codes (strata_weight_layout)")
    ap.add_argument("--router-only", action="store_true",
                    help="time only the router projection + top-k call (router6144) and print its record")
    ap.add_argument("--decode-only", metavar="WORKLOAD",
                    help="time only the decode record of WORKLOAD (decode or decode_shared) and print it")
    ap.add_argument("--kv-only", action="store_true",
                    help="time only the 4-bit KV cache encode and sparse attention and print their record")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_counters.json from two rocprofv3 --pmc runs and exit")
    args = ap.parse_args(argv)

    if args.record_traffic:
        # Records of other workloads already in the file are kept.
        rec = record_traffic(*args.record_traffic, prefill_workload=args.workload,
                             decode_workload=args.decode_only or "decode", layout=args.layout)
        try:
            with open(TRAFFIC_FILE) as f:
                merged = json.load(f)
        except (OSError, ValueError):
            merged = {}
        merged.update(rec)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(merged, f, indent=1, sort_keys=True)
            f.write("\n")
        print(json.dumps(rec, indent=1, sort_keys=True))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the MoE layer here is single-GPU (no sharding or collectives); "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    import quantized_expert_ffn_histogram_amd as qe

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    qe.load()
    if args.router_only:
        print(json.dumps(bench_router(qe, args)), flush=True)
        return 0
    if args.kv_only:
        print(json.dumps(bench_kv(qe, args)), flush=True)
        return 0
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration: 3 copies of 1 GiB (read 1 GiB + write 1 GiB each)")
        del src, dst
    if args.decode_only:
        print(json.dumps(bench_decode(qe, args, args.decode_only)), flush=True)
        return 0

    cfg, inp, secs, secs_timed, roof, kernels, secs4, steady, timed = bench_prefill(qe, args)
    flops, _ = layer_work(cfg, int((timed["counts"] > 0).sum()))
    result = {
        "metric": METRIC,
        "value": round(cfg.T * args.steps / secs, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(secs / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} g={cfg.g}",
            "weights": "int4 symmetric, fp16 scale per group",
            "weight_layout": args.layout,
            "activations": "bf16 in, fp32 out",
            "global_batch": cfg.T,
            "parallelism": "single GPU",
        },
        "roofline": roof,
        "layer_mfma_frac": round(flops / (secs / args.steps) / 1e12 / PEAK_MFMA_TFLOPS, 4),
        "prefill_steady_state": steady,
        "kernels_us": kernels,
        "ms_per_step_with_kernel_events": round(secs_timed / args.steps * 1e3, 4),
        "ms_per_step_four_calls": round(secs4 / args.steps * 1e3, 4),
    }
    if not args.no_decode:
        result["decode"] = bench_decode(qe, args)
        # Drafts that route mostly to the first token's experts: the pairs of
        # one expert stream the same weight rows on one XCD at the same time.
        result["decode_shared"] = bench_decode(qe, args, "decode_shared")
        # The same decode step with the codes in the other layout.
        other = "rows" if args.layout == "tiled" else "tiled"
        result[f"decode_{other}"] = bench_decode(qe, args, "decode", layout=other)
    if not args.no_secondary:
        result["secondary"] = bench_secondary(qe, args)
        result["kv_cache"] = bench_kv(qe, args)
    ref = None
    if not args.no_cpu_baseline:
        result["cpu_baseline"], ref = cpu_baseline(cfg, inp)
    elif not args.no_parity:
        import oracle

        ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    # Parity gate: the headline stands only if the output of the timed steps
    # matches the oracle.
    if ref is not None:
        result["parity"] = parity_gate(timed, ref)
        if result["parity"]["status"] != "ok":
            result["value"] = None
            print(json.dumps(result), flush=True)
            log(f"[bench] PARITY FAILURE: {result['parity']}")
            return 1
    else:
        result["parity"] = {"status": "not checked (--no-cpu-baseline --no-parity)"}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
