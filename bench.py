#!/usr/bin/env python3
"""Benchmark of the single-token routed-expert MoE decode layer on one MI355X.

A step is one replay of a hipGraph holding a 36-layer decode stack: 36
independent full-width layers (H=2048, E=256 experts, top-8 renormalised,
I=512, shared expert Is=512, fp16 weights, M=1 token), each running the whole
hot path (shared expert, router GEMV + top-k + softmax, expert-indexed W13 +
SiLU*mul, W2 + weighted combine + shared add).  2.08 GB of weights stream per
replay, far above the 256 MiB last-level cache, so every replay reads cold
from HBM.  Inputs are seeded synthetic tensors resident in HBM before timing.

Reported (one JSON line): expert-byte throughput in GB/s (value), us/layer,
fraction of the 8 TB/s HBM peak, the roofline of the dominant kernel (the
W13 + SiLU kernel, timed with HIP events on its own stream) and the fp64
oracle timed on this host's cores on a bounded sample of the same layers.
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

METRIC = "MoE decode µs/layer and achieved HBM GB/s (% of MI355X peak), M=1"
HBM_PEAK_GBS = 8000.0
LAYERS = 36
COUNTERS = os.path.join(ROOT, "profiles", "w13_counters_full_e256_k8_i512.json")
KERNEL_SRC = os.path.join(ROOT, "routed_expert_gemv_amd", "csrc", "moe_kernels.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_bytes(sh, n_distinct):
    """Algorithmic HBM bytes of one layer: (expert bytes, total bytes)."""
    routed = n_distinct * (2 * 2 * sh.I * sh.H + 2 * sh.H * sh.I)
    shared = 2 * 3 * sh.Is * sh.H
    expert = routed + shared
    total = expert + 2 * sh.E * sh.H + 2 * sh.M * sh.H * 2
    return expert, total


def w13_launch_bytes(sh):
    """Algorithmic bytes of one routed W13 + SiLU launch at M=1: K experts' gate and
    up rows, x, and the fp32 activations written."""
    return sh.K * 2 * sh.I * sh.H * 2 + sh.M * sh.H * 2 + sh.M * sh.K * sh.I * 4


def counters_traffic(n_launch_bytes):
    """HBM traffic of the W13 kernel from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    try:
        c = json.load(open(COUNTERS))
    except (OSError, ValueError):
        return None
    sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    if c.get("kernel_source_sha256") != sha:
        return None
    return c.get("hbm_bytes_per_dispatch")


def cpu_baseline(stack_tensors, sh, budget_s=12.0):
    """The fp64 oracle, as it is, on this host's cores over a bounded sample."""
    import numpy as np
    import torch
    import oracle

    nthreads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    sample = stack_tensors[:4]
    host = []
    for t in sample:  # host fp64 copies of what the oracle reads (not timed)
        h = {k: t[k].detach().to("cpu", torch.float64).numpy()
             for k in ("x", "wr", "wsgu", "wsd")}
        lg = oracle.router_logits(h["x"], h["wr"])
        ids, _, _ = oracle.topk_softmax(lg, sh.K, sh.renormalize)
        idx = torch.as_tensor(ids.reshape(-1).astype(np.int64), device=t["w13"].device)
        w13 = t["w13"].index_select(0, idx).to("cpu", torch.float64).numpy()
        w2 = t["w2"].index_select(0, idx).to("cpu", torch.float64).numpy()
        h["slices"] = (w13, w2)
        host.append(h)
    done = 0
    t0 = time.perf_counter()
    while True:
        h = host[done % len(host)]
        oracle.moe_layer_fetch(h["x"], h["wr"], lambda ids, s=h["slices"]: s, h["wsgu"],
                               h["wsd"], K=sh.K, renormalize=sh.renormalize, nthreads=nthreads)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    expert, _ = layer_bytes(sh, sh.K)
    us = el / done * 1e6
    return {"value": round(expert * done / el / 1e9, 4), "unit": "GB/s",
            "us_per_layer": round(us, 1), "cores": nthreads, "kind": "oracle",
            "sample": "%d layer evaluations cycling over 4 of the 36 layers (fp64 C oracle: "
                      "router, top-k, 8 experts, shared expert), %.1f s wall" % (done, el)}


def time_w13(layers, sh, reps):
    """Average duration of the routed W13 + SiLU kernel, with HIP events recorded
    around each launch on the stream the kernel runs on (cold: layers rotate)."""
    import torch
    import routed_expert_gemv_amd as moe

    stream = torch.cuda.current_stream()
    acts = [torch.empty((sh.M, sh.K, sh.I), dtype=torch.float32, device="cuda") for _ in layers]
    evs = []
    for r in range(reps + 1):
        for layer, act in zip(layers, acts):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            moe.moe_dbg_w13_silu(layer.t["x"], layer.t["w13"], layer.topk_ids, activated=act,
                                 ws=layer.ws, stream=stream)
            b.record(stream)
            if r > 0:
                evs.append((a, b))
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    return sum(ms) / len(ms) * 1e3, len(ms)  # us, launches


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--w13-reps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the decode layer is not sharded across GPUs "
              "here (requested --gpus %d)." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from routed_expert_gemv_amd import synth
    from routed_expert_gemv_amd.stack import DecodeLayer, DecodeStack

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sh = synth.SHAPES["full_e256_k8_i512"]

    log("drawing %d layers (seeds 0..%d) on %s" % (args.layers, args.layers - 1, dev))
    t0 = time.perf_counter()
    tensors = [synth.draw_layer(sh, s, dev) for s in range(args.layers)]
    layers = [DecodeLayer(t, sh) for t in tensors]
    torch.cuda.synchronize()
    log("drawn in %.1f s; capturing the stack graph" % (time.perf_counter() - t0))
    stack = DecodeStack(layers)
    stack.capture()
    for _ in range(args.warmup):
        stack.replay()
    torch.cuda.synchronize()
    log("warm-up done; timing %d replays" % args.steps)

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        stack.replay()
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    us_layer = ms_step * 1e3 / args.layers

    n_distinct = [len(set(l.topk_ids.flatten().tolist())) for l in layers]
    expert_b = sum(layer_bytes(sh, n)[0] for n in n_distinct)
    total_b = sum(layer_bytes(sh, n)[1] for n in n_distinct)
    gbs_expert = expert_b / (ms_step * 1e-3) / 1e9
    gbs_total = total_b / (ms_step * 1e-3) / 1e9
    log("%.3f ms/replay, %.2f us/layer, %.0f GB/s expert bytes" % (ms_step, us_layer, gbs_expert))

    w13_us, n_launch = time_w13(layers, sh, args.w13_reps)
    w13_b = w13_launch_bytes(sh)
    w13_gbs = w13_b / (w13_us * 1e-6) / 1e9
    traffic = counters_traffic(w13_b)
    log("W13 kernel: %.2f us avg over %d launches, %.0f GB/s" % (w13_us, n_launch, w13_gbs))

    out = {
        "metric": METRIC, "value": round(gbs_expert, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "36-layer full-width MoE decode stack as one hipGraph: M=1, "
                               "H=2048, E=256, top-8 renormalised, I=512, shared Is=512, fp16",
                   "layers": args.layers, "layer_seeds": "0..%d" % (args.layers - 1)},
        "us_per_layer": round(us_layer, 3),
        "frac_of_peak": round(gbs_expert / HBM_PEAK_GBS, 4),
        "gbs_total": round(gbs_total, 1),
        "expert_bytes_per_layer": expert_b // args.layers,
        "roofline": {"kernel": "k_w13_silu (routed W13 GEMV + SiLU*mul, M=1)", "bound": "hbm",
                     "achieved": round(w13_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(w13_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "avg_launch_us": round(w13_us, 3), "bytes_per_launch": w13_b},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host (~%.0f s)" % args.cpu_budget)
        out["cpu_baseline"] = cpu_baseline(tensors, sh, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
