#!/usr/bin/env python3
"""Benchmark of the single-token routed-expert MoE decode layer on one MI355X.

A step is one replay of a hipGraph holding a 36-layer decode stack: 36
independent full-width layers (H=2048, E=256 experts, top-8 renormalised,
I=512, shared expert Is=512, fp16 weights, M=1 token), each running the whole
hot path (shared expert, router GEMV + top-k + softmax, expert-indexed W13 +
SiLU*mul, W2 + weighted combine + shared add).  2.08 GB of weights stream per
replay, far above the 256 MiB last-level cache, so every replay reads cold
from HBM.  Inputs are seeded synthetic tensors resident in HBM before timing.

Each layer is one moe_layer_decode call, three launches at M=1 (router +
shared gate/up, expand, reduce); with --path separate the three entry points
run instead (six kernels per layer).  --shape tp4_shard_e256_k8_i128 runs the
TP=4 shard of the same layer instead (I=128, shared Is=128: 15.2 MB touched
per layer, 548 MB per replay, still above the last-level cache); --tokens
2/4/8 the small-batch layers.

Reported (one JSON line): expert-byte throughput in GB/s (value), us/layer,
fraction of the 8 TB/s HBM peak, the roofline of the dominant kernel (the
expand kernel, timed with HIP events over graphs of that kernel alone, next to
the average of the same graphs in the committed rocprofv3 trace when it was
taken on the current sources; with --tokens, the dominant step of the layer's
three, timed the same way) and the fp64 oracle timed on this host's cores
(one core and all of them) on a bounded sample of the same layers.

With --prefill T the workload is the many-token layer instead: a stack of
full-width layers (default 8) with T tokens each, every layer one
moe_layer_prefill call (seven launches); the line reports tokens/s through a
layer, us/layer, weight bytes per second, and the roofline of the gate/up
grouped GEMM.
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
COUNTERS = os.path.join(ROOT, "profiles", "k_expand_counters_full_e256_k8_i512.json")
STAGES = ("k_router1", "k_expand", "k_reduce")
# the three steps of a layer of 2..8 tokens (the selection launch and the
# expand launch count as one step at M = 5..8)
STAGES_M = ("k_route_shared_m", "k_expand_sel_m", "k_w2_staged")
STAGES_M8 = ("k_route_shared_m", "k_select_m+k_expand_m", "k_w2_staged")
KERNEL_SRC = os.path.join(ROOT, "routed_expert_gemv_amd", "csrc", "moe_kernels.hip")
# sources the decode kernels are compiled from (a summary taken on other
# sources no longer describes the kernels that run)
DECODE_SRCS = tuple(os.path.join(ROOT, "routed_expert_gemv_amd", "csrc", f)
                    for f in ("moe_kernels.hip", "moe_device.h", "moe_internal.h"))
DECODE_SHAPES = ("full_e256_k8_i512", "tp4_shard_e256_k8_i128", "batch2_e256_k8_i512",
                 "batch4_e256_k8_i512", "batch8_e256_k8_i512")
PF_METRIC = "MoE prefill tokens/s through one full-width layer (T tokens per layer)"
PF_STAGES = ("k_pf_router", "k_pf_topk", "k_pf_plan", "k_pf_w13", "k_pf_w2", "k_pf_combine")
PF_KERNEL_SRC = os.path.join(ROOT, "routed_expert_gemv_amd", "csrc", "moe_prefill.hip")
MFMA_F16_PEAK_TFLOPS = 2500.0


def pf_counters_path(T):
    return os.path.join(ROOT, "profiles", "k_pf_w13_counters_prefill_t%d_e256_k8_i512.json" % T)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_bytes(sh, n_distinct):
    """Algorithmic HBM bytes of one layer: (expert bytes, total bytes)."""
    routed = n_distinct * (2 * 2 * sh.I * sh.H + 2 * sh.H * sh.I)
    shared = 2 * 3 * sh.Is * sh.H
    expert = routed + shared
    total = expert + 2 * sh.E * sh.H + 2 * sh.M * sh.H * 2
    return expert, total


def stage_bytes(sh):
    """Algorithmic bytes of each of the three launches of one layer at M=1 (K
    distinct experts) with a shared expert as wide as a routed one, or none
    (the benched shapes): the router alone; the routed and shared gate/up rows;
    the routed and shared down rows.  Weights read once, x once, and the small
    tensors each kernel reads or writes (logits, activations, ids/weights, y)."""
    H, E, K, I, Is = sh.H, sh.E, sh.K, sh.I, sh.Is
    assert Is in (0, I), "stage bytes are for the folded shared-expert placement"
    router = 2 * E * H + 2 * H + 4 * E
    expand = 2 * K * 2 * I * H + 2 * 2 * Is * H + 2 * H + 4 * E + 4 * K * I + 4 * Is + 8 * K
    reduce = 2 * K * H * I + 2 * H * Is + 4 * K * I + 4 * Is + 8 * K + 2 * H
    return dict(zip(STAGES, (router, expand, reduce)))


def stage_bytes_m(sh, n_distinct):
    """Algorithmic bytes of the three steps of a layer of M = sh.M > 1 tokens
    with n_distinct distinct experts and a shared expert as wide as a routed
    one, or none: router rows and shared gate/up rows; the distinct experts'
    gate/up rows and the shared down rows; their down rows.  Weights read once,
    x once, and the small tensors each step reads or writes (logits, routing
    ids/weights, routed and shared activations, shared output, y)."""
    M, H, E, K, I, Is = sh.M, sh.H, sh.E, sh.K, sh.I, sh.Is
    assert Is in (0, I), "stage bytes are for the benched shared-expert width"
    route = 2 * E * H + 2 * 2 * Is * H + 2 * M * H + 4 * M * E + 4 * M * Is
    expand = (2 * 2 * n_distinct * I * H + 2 * H * Is + 2 * M * H + 4 * M * E + 8 * M * K
              + 4 * M * K * I + 4 * M * Is + (4 * M * H if Is else 0))
    w2 = (2 * n_distinct * H * I + 4 * M * K * I + 8 * M * K + (4 * M * H if Is else 0)
          + 2 * M * H)
    names = STAGES_M if M <= 4 else STAGES_M8
    return dict(zip(names, (route, expand, w2)))


def prefill_stage_bytes(sh, n_distinct):
    """Algorithmic bytes of each prefill launch (T = sh.M tokens, n_distinct
    experts with at least one token): weights read once, x read once, and the
    tensors each kernel writes or reads (logits, ids/weights, pair lists,
    activations, the fp32 down products, y)."""
    T, H, E, K, I, Is = sh.M, sh.H, sh.E, sh.K, sh.I, sh.Is
    rows = T * K + (T if Is else 0)
    return dict(zip(PF_STAGES, (
        2 * E * H + 2 * T * H + 4 * T * E,
        4 * T * E + 8 * T * K,
        4 * T * K * 2,
        n_distinct * 2 * 2 * I * H + 2 * 2 * Is * H + 2 * T * H + 2 * T * K * I + 2 * T * Is,
        n_distinct * 2 * H * I + 2 * H * Is + 2 * T * K * I + 2 * T * Is + 4 * rows * H,
        4 * rows * H + 4 * T * K + 2 * T * H)))


def prefill_flops(sh):
    """Multiply-add flops of the router, gate/up and down products (x2 per MAC)."""
    T, H, E, K, I, Is = sh.M, sh.H, sh.E, sh.K, sh.I, sh.Is
    return {"k_pf_router": 2 * T * E * H, "k_pf_w13": 2 * T * (K * 2 * I + 2 * Is) * H,
            "k_pf_w2": 2 * T * (K * I + Is) * H}


def sources_sha(srcs):
    h = hashlib.sha256()
    for f in srcs:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def counters_path(shape):
    return os.path.join(ROOT, "profiles", "k_expand_counters_%s.json" % shape)


def trace_path(shape):
    return os.path.join(ROOT, "profiles", "layer_kernels_trace_%s.md" % shape)


def counters_traffic(path=COUNTERS, srcs=DECODE_SRCS):
    """HBM traffic per launch of the summarised kernel from a committed rocprofv3
    counter summary, if it was taken on the current kernel sources; else None."""
    try:
        c = json.load(open(path))
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256") != sources_sha(srcs):
        return None
    return c.get("hbm_bytes_per_dispatch")


def rocprof_stage_us(shape):
    """Per-kernel average duration inside the stage graphs from the committed
    rocprofv3 kernel-trace summary of this shape (its trailing JSON block), if
    that trace was taken on the current kernel sources; else None."""
    try:
        text = open(trace_path(shape)).read()
        blob = json.loads(text.rsplit("```json", 1)[1].split("```", 1)[0])
    except (OSError, ValueError, IndexError):
        return None
    if blob.get("kernel_source_sha256") != sources_sha(DECODE_SRCS):
        return None
    return blob.get("stage_avg_us")


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or the platform string."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def cpu_baseline(stack_tensors, sh, budget_s=12.0):
    """The fp64 oracle, as it is, on this host: the same layers timed on one
    core and on every core the process may use (half the budget each)."""
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

    def run(threads, budget):
        done = 0
        t0 = time.perf_counter()
        while True:
            h = host[done % len(host)]
            oracle.moe_layer_fetch(h["x"], h["wr"], lambda ids, s=h["slices"]: s, h["wsgu"],
                                   h["wsd"], K=sh.K, renormalize=sh.renormalize,
                                   nthreads=threads)
            done += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return done, el

    d1, e1 = run(1, budget_s / 2)
    dn, en = run(nthreads, budget_s / 2)
    expert, _ = layer_bytes(sh, sh.K)
    return {"value": round(expert * dn / en / 1e9, 4), "unit": "GB/s",
            "us_per_layer": round(en / dn * 1e6, 1), "cores": nthreads, "kind": "oracle",
            "value_1core": round(expert * d1 / e1 / 1e9, 4),
            "us_per_layer_1core": round(e1 / d1 * 1e6, 1),
            "cpu_model": cpu_model(),
            "sample": "fp64 C oracle (router, top-k, 8 experts, shared expert) cycling over 4 "
                      "of the 36 layers: %d layer evaluations on %d threads in %.1f s, %d on 1 "
                      "thread in %.1f s" % (dn, nthreads, en, d1, e1)}


def replay_percentiles(stack, n, layers):
    """p10 / p50 / p90 of the per-layer time over n replays, each bracketed by
    its own pair of HIP events (after the timed loop, so it does not perturb it)."""
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for a, b in ev:
        a.record()
        stack.replay()
        b.record()
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 / layers for a, b in ev)
    pick = lambda q: round(us[min(len(us) - 1, int(q * (len(us) - 1) + 0.5))], 3)
    return [pick(0.1), pick(0.5), pick(0.9)]


def time_stages(layers, reps, names=STAGES):
    """Average duration of each of the three steps of a layer (at M = 1 one
    kernel each): for each step, a hipGraph of that step alone for every layer
    of the stack (inputs left by the full calls before it; the layers rotate,
    so weights stream cold), replayed `reps` times between two HIP events on
    the replay stream."""
    import torch
    import routed_expert_gemv_amd as moe

    def stage_call(layer, stage):
        t, sh = layer.t, layer.shape
        moe.moe_dbg_layer_stage(stage, t["x"], t["wr"], t["w13"], t["w2"], t["wsgu"], t["wsd"],
                                sh.K, sh.renormalize, layer.topk_ids, layer.topk_w, layer.logits,
                                layer.y, layer.ws)

    for layer in layers:  # every stage's inputs in place
        layer.forward()
    torch.cuda.synchronize()
    us = {}
    for i, name in enumerate(names):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for layer in layers:
                stage_call(layer, i + 1)
        g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        us[name] = a.elapsed_time(b) * 1e3 / (reps * len(layers))
        del g
    return us, reps * len(layers)


def prefill_cpu_baseline(t, sh, budget_s=12.0):
    """The fp64 oracle, as it is, on this host's cores: router, top-K, the K
    experts and the shared expert of sampled tokens of one prefill layer.  The
    layer's tensors are widened to fp64 on the host once, before timing; only
    the oracle's own calls are timed (the gather of each token's expert slices
    between them is not)."""
    import numpy as np
    import torch
    import oracle

    nthreads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    h = {k: t[k].detach().to("cpu", torch.float64).numpy()
         for k in ("x", "wr", "wsgu", "wsd", "w13", "w2")}
    order = np.random.default_rng(0).permutation(sh.M)
    done, el = 0, 0.0
    while el < budget_s and done < sh.M:
        m = int(order[done])
        t0 = time.perf_counter()
        lg = oracle.router_logits(h["x"][m], h["wr"], nthreads)
        ids, w, _ = oracle.topk_softmax(lg, sh.K, sh.renormalize)
        el += time.perf_counter() - t0
        w13sel, w2sel = h["w13"][ids], h["w2"][ids]
        t0 = time.perf_counter()
        oracle.token_output(h["x"][m], w13sel, w2sel, w, h["wsgu"], h["wsd"], nthreads)
        el += time.perf_counter() - t0
        done += 1
    return {"value": round(done / el, 3), "unit": "tokens/s", "cores": nthreads,
            "kind": "oracle", "us_per_token": round(el / done * 1e6, 1),
            "sample": "%d tokens of layer 0 (fp64 C oracle per token: router, top-k, 8 experts, "
                      "shared expert), %.1f s of oracle time" % (done, el)}


def time_prefill_stages(layers, reps):
    """Average duration of each of the six prefill stages: per stage, a
    hipGraph of that launch alone for every layer (inputs left by full calls),
    replayed `reps` times between two HIP events on the replay stream."""
    import torch

    for layer in layers:
        layer.forward()
    torch.cuda.synchronize()
    us = {}
    for i, name in enumerate(PF_STAGES):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for layer in layers:
                layer.stage(i + 1)
        g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        us[name] = a.elapsed_time(b) * 1e3 / (reps * len(layers))
        del g
    return us, reps * len(layers)


def prefill_main(args, dev):
    import torch
    from routed_expert_gemv_amd import synth
    from routed_expert_gemv_amd.api import prefill_workspace
    from routed_expert_gemv_amd.stack import DecodeStack, PrefillLayer

    T = args.prefill
    n_layers = args.layers if args.layers_given else 8
    sh = synth.LayerShape(M=T, H=2048, E=256, K=8, I=512, Is=512)
    log("drawing %d prefill layers of %d tokens (seeds 0..%d) on %s" % (n_layers, T, n_layers - 1, dev))
    tensors = [synth.draw_layer(sh, s, dev) for s in range(n_layers)]
    ws = prefill_workspace(T, sh.H, sh.E, sh.I, sh.K, sh.Is, dev)
    layers = [PrefillLayer(t, sh, ws) for t in tensors]
    stack = DecodeStack(layers)
    stack.capture()
    for _ in range(args.warmup):
        stack.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        stack.replay()
    b.record()
    torch.cuda.synchronize()
    ms_step = a.elapsed_time(b) / args.steps
    us_layer = ms_step * 1e3 / n_layers
    pct = replay_percentiles(stack, args.steps, n_layers)
    n_distinct = [len(set(l.topk_ids.flatten().tolist())) for l in layers]
    nd = sum(n_distinct) / len(n_distinct)
    w_bytes = nd * 3 * 2 * sh.I * sh.H + 3 * 2 * sh.Is * sh.H + 2 * sh.E * sh.H
    log("%.3f ms/replay, %.1f us/layer, %.0f tokens/s, %.0f GB/s of weights"
        % (ms_step, us_layer, T / (us_layer * 1e-6), w_bytes / (us_layer * 1e-6) / 1e9))
    st_us, n_launch = time_prefill_stages(layers, args.launch_reps)
    st_b = prefill_stage_bytes(sh, round(nd))
    fl = prefill_flops(sh)
    log("kernels: " + ", ".join("%s %.1f us %.0f GB/s" % (k, st_us[k], st_b[k] / (st_us[k] * 1e-6) / 1e9)
                                 for k in PF_STAGES))
    dom = "k_pf_w13"
    k_gbs = st_b[dom] / (st_us[dom] * 1e-6) / 1e9
    roof = {"kernel": dom, "bound": "hbm", "achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(k_gbs / HBM_PEAK_GBS, 4),
            "traffic": counters_traffic(pf_counters_path(T), (PF_KERNEL_SRC,)),
            "avg_launch_us": round(st_us[dom], 3), "bytes_per_launch": st_b[dom],
            "launches_timed": n_launch,
            "mfma_tflops": round(fl[dom] / (st_us[dom] * 1e-6) / 1e12, 1),
            "mfma_frac": round(fl[dom] / (st_us[dom] * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "per_kernel_us": {k: round(v, 3) for k, v in st_us.items()},
            "per_kernel_bytes": st_b}
    out = {
        "metric": PF_METRIC, "value": round(T / (us_layer * 1e-6), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "%d-layer full-width MoE prefill stack as one hipGraph: T=%d "
                               "tokens per layer, H=2048, E=256, top-8 renormalised, I=512, "
                               "shared Is=512, fp16" % (n_layers, T),
                   "tokens": T, "layers": n_layers, "layer_seeds": "0..%d" % (n_layers - 1),
                   "distinct_experts_per_layer": round(nd, 2)},
        "us_per_layer": round(us_layer, 3),
        "us_per_layer_p10_p50_p90": pct,
        "weight_gbs": round(w_bytes / (us_layer * 1e-6) / 1e9, 1),
        "frac_of_peak": round(w_bytes / (us_layer * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host (~%.0f s)" % args.cpu_budget)
        out["cpu_baseline"] = prefill_cpu_baseline(tensors[0], sh, args.cpu_budget)
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------- rocprofv3 helpers
COPY_BYTES = 1 << 30


def counters_pass(args):
    """Workload for `rocprofv3 --pmc`: the library's plain copy kernel over 1 GiB
    (calibrates what FETCH_SIZE / WRITE_SIZE read for a known byte count), then
    every layer of the stack through moe_layer_decode, twice (cold: layers
    rotate)."""
    import torch
    import routed_expert_gemv_amd as moe
    from routed_expert_gemv_amd import synth
    from routed_expert_gemv_amd.stack import DecodeLayer

    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 2, dtype=torch.float16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        moe.moe_probe_copy(src, dst)
    torch.cuda.synchronize()
    del src, dst
    if args.prefill:
        from routed_expert_gemv_amd.stack import PrefillLayer
        sh = synth.LayerShape(M=args.prefill, H=2048, E=256, K=8, I=512, Is=512)
        layers = [PrefillLayer(synth.draw_layer(sh, s, dev), sh) for s in range(args.layers)]
    else:
        sh = synth.SHAPES[args.shape]
        layers = [DecodeLayer(synth.draw_layer(sh, s, dev), sh) for s in range(args.layers)]
    for _ in range(2):
        for l in layers:
            l.forward()
    torch.cuda.synchronize()
    log("counters pass done: 3 copies of %d bytes, %d layer launches" % (COPY_BYTES, 2 * len(layers)))


def _read_csv_rows(d, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def summarize_counters(fetch_dir, write_dir, out_path, cmds, prefill=0, shape="full_e256_k8_i512"):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE of the expand kernel (and, for
    context, the other two), scaled by what the same counters read for the
    1 GiB copy, into a JSON summary."""
    def per_kernel(d, counter, kernel="k_expand"):
        rows = _read_csv_rows(d, "counter_collection.csv")
        mine, copy = [], []
        for r in rows:
            if r.get("Counter_Name") != counter:
                continue
            v = float(r["Counter_Value"])
            name = r.get("Kernel_Name", "")
            if kernel in name:
                mine.append(v)
            elif "k_probe_copy" in name:
                copy.append(v)
        return mine, copy

    kern = "k_pf_w13" if prefill else "k_expand"
    fw, fc = per_kernel(fetch_dir, "FETCH_SIZE", kern)
    ww, wc = per_kernel(write_dir, "WRITE_SIZE", kern)
    if not fw or not fc or not ww or not wc:
        raise SystemExit("counter rows missing: fetch %d/%d write %d/%d" % (len(fw), len(fc), len(ww), len(wc)))
    kib = 1024.0
    fetch_scale = (sum(fc) / len(fc)) * kib / COPY_BYTES
    write_scale = (sum(wc) / len(wc)) * kib / COPY_BYTES
    fetch_b = (sum(fw) / len(fw)) * kib / fetch_scale
    write_b = (sum(ww) / len(ww)) * kib / write_scale
    from routed_expert_gemv_amd import synth
    if prefill:
        sh = synth.LayerShape(M=prefill, H=2048, E=256, K=8, I=512, Is=512)
        algo = prefill_stage_bytes(sh, sh.E)  # every expert receives tokens at this size
        other_names = ("k_pf_router", "k_pf_w2", "k_pf_combine")
    else:
        sh = synth.SHAPES[shape]
        algo = stage_bytes(sh)
        other_names = ("k_router1", "k_reduce")
    others = {}
    for k in other_names:
        f, _ = per_kernel(fetch_dir, "FETCH_SIZE", k)
        w, _ = per_kernel(write_dir, "WRITE_SIZE", k)
        if f and w:
            others[k] = {"hbm_bytes_per_dispatch": int(round((sum(f) / len(f)) * kib / fetch_scale
                                                             + (sum(w) / len(w)) * kib / write_scale)),
                         "algorithmic_bytes_per_dispatch": algo[k]}
    res = {
        "kernel": ("k_pf_w13 (grouped gate/up GEMM + SiLU*mul, routed and shared experts), T=%d"
                   % prefill) if prefill else
                  "k_expand (routed and shared gate/up + SiLU*mul), M=1",
        "workload": ("full-width prefill layer H=2048 E=256 K=8 I=512 Is=512, T=%d tokens"
                     % prefill) if prefill else
                    "%s: H=%d E=%d K=%d I=%d Is=%d, M=1, 36 layers rotating"
                    % (shape, sh.H, sh.E, sh.K, sh.I, sh.Is),
        "commands": cmds,
        "fetch_size_kib_per_dispatch": sum(fw) / len(fw),
        "write_size_kib_per_dispatch": sum(ww) / len(ww),
        "copy_fetch_kib": sum(fc) / len(fc), "copy_write_kib": sum(wc) / len(wc),
        "copy_bytes": COPY_BYTES, "fetch_scale": fetch_scale, "write_scale": write_scale,
        "hbm_bytes_per_dispatch": int(round(fetch_b + write_b)),
        "algorithmic_bytes_per_dispatch": algo[kern],
        "dispatches": len(fw),
        "other_kernels": others,
        "kernel_source_sha256": sources_sha((PF_KERNEL_SRC,) if prefill else DECODE_SRCS),
    }
    with open(out_path, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res, indent=1))


def summarize_pmc(out_path, dirs, cmds, title):
    """Average per dispatch of every counter collected in the given rocprofv3
    --pmc output folders, for each of the library's kernels (one row per
    kernel and instance), as a markdown table."""
    vals = {}
    for d in dirs:
        for r in _read_csv_rows(d, "counter_collection.csv"):
            name = r.get("Kernel_Name", "")
            if not ("_ZN3moe" in name or "moe::" in name):
                continue
            key = (kernel_key(name), name)
            vals.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    counters = sorted({c for v in vals.values() for c in v})
    # GRBM_GUI_ACTIVE sums the GPU-busy cycles of the 8 XCDs (the 1 GiB copy
    # kernel reads 8x the cycles of its run); TA busy cycles over the cycles of
    # one XCD give the share of the run the memory units were busy
    derived = "TA_BUSY_avr" in counters and "GRBM_GUI_ACTIVE" in counters
    head = counters + (["MemUnitBusy % (TA_BUSY_avr / (GRBM_GUI_ACTIVE/8))"] if derived else [])
    lines = ["# rocprofv3 counters: " + title, ""] + ["Command: `%s`" % c for c in cmds] + [
        "", "Average per dispatch (dispatches in parentheses).  The counters are taken "
            "with each dispatch serialised by the profiler, so kernel times here run "
            "longer than in the graph.", "",
        "| kernel | " + " | ".join(head) + " |", "|---" * (len(head) + 1) + "|"]
    for (k, n), v in sorted(vals.items()):
        tmpl = n[n.find("I", n.find(k) + len(k)):][:40] if "_ZN3moe" in n else ""
        cells = []
        for c in counters:
            x = v.get(c)
            cells.append("%.4g (%d)" % (sum(x) / len(x), len(x)) if x else "-")
        if derived:
            ta, gr = v.get("TA_BUSY_avr"), v.get("GRBM_GUI_ACTIVE")
            cells.append("%.1f" % (100.0 * (sum(ta) / len(ta)) / (sum(gr) / len(gr) / 8))
                         if ta and gr else "-")
        lines.append("| `%s` %s | %s |" % (k, ("`" + tmpl + "`") if tmpl else "", " | ".join(cells)))
    lines += ["", "kernel_source_sha256 (decode sources): " + sources_sha(DECODE_SRCS)]
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def kernel_key(name):
    """The kernel's own name (k_expand, ...) from a mangled or demangled name."""
    import re
    m = re.search(r"_ZN3moe(\d+)", name)
    if m:
        n = int(m.group(1))
        return name[m.end():m.end() + n]
    m = re.search(r"moe::(k_\w+)", name)
    return m.group(1) if m else name.replace("(anonymous namespace)::", "").split("(")[0][:90]


def summarize_trace(trace_dir, out_path, cmd, bench_line=None):
    """Kernel-trace summary: per-kernel count / average duration, the averages
    inside the per-kernel stage graphs bench.py times (next to bench.py's own
    HIP-event figures from the same run, when its output line is given), and the
    idle gap between consecutive kernels; a trailing JSON block holds the
    stage-graph averages and the hash of the kernel sources."""
    rows = _read_csv_rows(trace_dir, "kernel_trace.csv")
    if not rows:
        raise SystemExit("no kernel_trace.csv under " + trace_dir)
    ev = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]) for r in rows)
    by = {}
    for s0, e0, n in ev:
        by.setdefault(n, []).append(e0 - s0)
    ours = [e for e in ev if "moe::" in e[2] or "_ZN3moe" in e[2]]
    gaps = [b[0] - a[1] for a, b in zip(ours, ours[1:]) if 0 <= b[0] - a[1] < 20000]
    lines = ["# rocprofv3 kernel trace: " + os.path.basename(out_path), "",
             "Command: `%s`" % cmd, "",
             "| kernel | dispatches | avg us | min us | max us |", "|---|---|---|---|---|"]
    def short_name(n):
        return n.replace("(anonymous namespace)::", "").split("(")[0][:90]

    for n, d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        lines.append("| `%s` | %d | %.3f | %.3f | %.3f |" % (short_name(n), len(d), sum(d) / len(d) / 1e3,
                                                          min(d) / 1e3, max(d) / 1e3))
    # dispatches inside the per-kernel stage graphs that bench times (each
    # neighbour is the same kernel), next to the average over every dispatch
    runs = {}
    for i in range(1, len(ours) - 1):
        if ours[i - 1][2] == ours[i][2] == ours[i + 1][2]:
            runs.setdefault(ours[i][2], []).append(ours[i][1] - ours[i][0])
    line = None
    if bench_line:
        for ln in open(bench_line):
            if ln.startswith("{"):
                line = json.loads(ln)
    ev_us = ((line or {}).get("roofline") or {}).get("per_kernel_us", {})
    stage_avg = {}
    if runs:
        lines += ["", "Inside the stage graphs (dispatches whose neighbours are the same kernel), "
                      "with bench.py's HIP-event average per launch over the same graphs:", "",
                  "| kernel | dispatches | avg us | min us | max us | HIP events us |",
                  "|---|---|---|---|---|---|"]
        for n, d in sorted(runs.items(), key=lambda kv: -sum(kv[1])):
            k = kernel_key(n)
            stage_avg[k] = round(sum(d) / len(d) / 1e3, 4)
            lines.append("| `%s` | %d | %.3f | %.3f | %.3f | %s |" % (
                short_name(n), len(d), sum(d) / len(d) / 1e3, min(d) / 1e3, max(d) / 1e3,
                "%.3f" % ev_us[k] if k in ev_us else "-"))
    if gaps:
        gaps.sort()
        lines += ["", "Gap between consecutive library kernels (end -> next start, < 20 us): "
                  "n=%d, median %.3f us, mean %.3f us" % (len(gaps), gaps[len(gaps) // 2] / 1e3,
                                                       sum(gaps) / len(gaps) / 1e3)]
    if line:
        lines += ["", "bench.py line of the profiled run: %.3f us/layer, %.1f GB/s (under the "
                      "profiler)" % (line.get("us_per_layer", 0.0), line.get("value", 0.0))]
    blob = {"stage_avg_us": stage_avg, "kernel_source_sha256": sources_sha(DECODE_SRCS)}
    lines += ["", "```json", json.dumps(blob), "```"]
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# Launch structures whose floor probes() measures: the bytes each launch of a
# full-width layer reads (router rows; gate/up rows with the shared ones; down
# rows with the shared ones), and the same bytes with the down rows moved into
# the gate/up launch (split-K partial sums), with and without a launch that
# sums the partials.
FLOOR_STRUCTURES = {
    "router+expand+reduce": (1053696, 37772352, 18896960),
    "router+expand_with_down+partial_sum": (1053696, 37772352 + 18896960, 1048576),
    "router+expand_with_down": (1053696, 37772352 + 18896960),
}


def probes(dev):
    """Empty-kernel launch latency, hipGraph kernel-node gap, the read
    bandwidth of a 2 GiB stream (the practical HBM ceiling), and the floor per
    layer of the launch structures above: pure streams of each launch's bytes,
    36 layers on distinct buffers in one graph."""
    import torch
    import routed_expert_gemv_amd as moe

    res = {}
    for _ in range(20):
        moe.moe_probe_empty()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(200):
        moe.moe_probe_empty()
    b.record()
    torch.cuda.synchronize()
    res["empty_launch_us"] = round(a.elapsed_time(b) * 1e3 / 200, 3)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.moe_probe_empty()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(100):
            moe.moe_probe_empty()
    g.replay()
    torch.cuda.synchronize()
    a.record()
    for _ in range(10):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    res["graph_node_us"] = round(a.elapsed_time(b) * 1e3 / 1000, 3)

    buf = torch.zeros((2 << 30) // 2, dtype=torch.float16, device=dev)
    out = torch.zeros(1, dtype=torch.float32, device=dev)
    moe.moe_probe_read(buf, out)
    torch.cuda.synchronize()
    a.record()
    for _ in range(10):
        moe.moe_probe_read(buf, out)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 10
    res["read_2GiB_GBs"] = round(buf.numel() * 2 / (ms * 1e-3) / 1e9, 1)

    flat = buf.view(torch.uint8)
    floors = {}
    for name, sizes in FLOOR_STRUCTURES.items():
        padded = [(n + 4095) // 4096 * 4096 for n in sizes]
        stride = sum(padded)
        assert stride * LAYERS <= flat.numel()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for layer in range(LAYERS):
                off = layer * stride
                for n, p in zip(sizes, padded):
                    moe.moe_probe_read(flat[off:off + n], out)
                    off += p
        g.replay()
        torch.cuda.synchronize()
        a.record()
        for _ in range(10):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        floors[name] = round(a.elapsed_time(b) * 1e3 / (10 * LAYERS), 3)
        del g
    res["layer_floor_us"] = floors
    del flat, buf
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=None,
                    help="layers in the stack (decode default %d, prefill default 8)" % LAYERS)
    ap.add_argument("--prefill", type=int, default=0, metavar="T",
                    help="bench the many-token layer with T tokens per layer instead of decode")
    ap.add_argument("--shape", choices=DECODE_SHAPES, default=None,
                    help="decode layer shape (default full_e256_k8_i512, or the batch shape "
                         "--tokens names); tp4_shard_e256_k8_i128 is the TP=4 shard")
    ap.add_argument("--tokens", type=int, default=1, choices=(1, 2, 4, 8),
                    help="tokens per layer: 1 (the default workload) or a small decode batch "
                         "(each token routed on its own; distinct experts read once)")
    ap.add_argument("--launch-reps", type=int, default=10)
    ap.add_argument("--path", choices=("fused", "separate", "single"), default="fused",
                    help="fused: moe_layer_decode (three launches per layer); separate: the "
                         "three entry points; single: the single-launch layer (M = 1)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--counters-pass", action="store_true",
                    help="run the rocprofv3 --pmc workload (copy calibration + layer launches)")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"))
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "OUT"))
    ap.add_argument("--bench-line", default=None,
                    help="file holding the bench.py output of the profiled run (for --summarize-trace)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="OUT_THEN_DIRS",
                    help="markdown summary OUT of the --pmc output folders that follow")
    ap.add_argument("--title", default="", help="title of a --summarize-pmc summary")
    ap.add_argument("--cmd", action="append", default=[],
                    help="command line(s) recorded in a summary")
    args = ap.parse_args()
    args.layers_given = args.layers is not None
    if args.layers is None:
        args.layers = LAYERS

    if args.shape is None:
        args.shape = "full_e256_k8_i512" if args.tokens == 1 else "batch%d_e256_k8_i512" % args.tokens
    elif args.tokens != 1:
        ap.error("--tokens and --shape name the workload twice: give one")

    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, cmds=args.cmd, prefill=args.prefill,
                           shape=args.shape)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, cmd=" && ".join(args.cmd), bench_line=args.bench_line)
        return
    if args.summarize_pmc:
        if len(args.summarize_pmc) < 2:
            ap.error("--summarize-pmc OUT DIR [DIR ...]")
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1:], args.cmd, args.title)
        return

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
    if args.counters_pass:
        counters_pass(args)
        return
    if args.prefill:
        prefill_main(args, dev)
        return
    sh = synth.SHAPES[args.shape]

    log("drawing %d layers (seeds 0..%d) on %s" % (args.layers, args.layers - 1, dev))
    t0 = time.perf_counter()
    tensors = [synth.draw_layer(sh, s, dev) for s in range(args.layers)]
    if args.path == "single" and sh.M != 1:
        ap.error("--path single runs one token per layer")
    layers = [DecodeLayer(t, sh, fused=args.path != "separate", single=args.path == "single")
              for t in tensors]
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
    pct = replay_percentiles(stack, args.steps, args.layers)

    n_distinct = [len(set(l.topk_ids.flatten().tolist())) for l in layers]
    expert_b = sum(layer_bytes(sh, n)[0] for n in n_distinct)
    total_b = sum(layer_bytes(sh, n)[1] for n in n_distinct)
    gbs_expert = expert_b / (ms_step * 1e-3) / 1e9
    gbs_total = total_b / (ms_step * 1e-3) / 1e9
    log("%.3f ms/replay, %.2f us/layer, %.0f GB/s expert bytes" % (ms_step, us_layer, gbs_expert))

    roof = None
    if args.path == "single":
        # one kernel per layer: its launch is the layer
        k_gbs = total_b / (ms_step * 1e-3) / 1e9
        roof = {"kernel": "k_layer1", "bound": "hbm", "achieved": round(k_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(k_gbs / HBM_PEAK_GBS, 4),
                "traffic": None, "avg_launch_us": round(us_layer, 3),
                "bytes_per_launch": total_b // args.layers, "launches_timed": args.steps * args.layers,
                "frac_method": "HIP events around the stack replays; one launch per layer"}
        # waits that ran out over the whole run (the state block's counter,
        # 32-bit word 1024 of each layer's workspace): 0 when every hand-off
        # arrived in time
        out_gave_up = sum(int(l.ws[4096:4100].view(torch.int32).item()) for l in layers)
        roof["waits_gave_up"] = out_gave_up
    elif args.path == "fused" and sh.M == 1:
        st_us, n_launch = time_stages(layers, args.launch_reps)
        st_b = stage_bytes(sh)
        dom = max(STAGES, key=lambda k: st_us[k])
        k_gbs = st_b[dom] / (st_us[dom] * 1e-6) / 1e9
        log("kernels (HIP events over stage graphs, %d launches each): %s" % (n_launch, ", ".join(
            "%s %.2f us %.0f GB/s" % (k, st_us[k], st_b[k] / (st_us[k] * 1e-6) / 1e9)
            for k in STAGES)))
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(k_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(k_gbs / HBM_PEAK_GBS, 4),
                "traffic": counters_traffic(counters_path(args.shape)) if dom == "k_expand" else None,
                "avg_launch_us": round(st_us[dom], 3), "bytes_per_launch": st_b[dom],
                "launches_timed": n_launch,
                "frac_method": "HIP events around %d replays of a graph of the kernel alone for "
                               "every layer, divided by the launches" % args.launch_reps,
                "per_kernel_us": {k: round(v, 3) for k, v in st_us.items()},
                "per_kernel_bytes": st_b}
        rp = rocprof_stage_us(args.shape)
        if rp and dom in rp:
            # the same stage graphs in the committed rocprofv3 kernel trace
            roof["rocprof_avg_launch_us"] = rp[dom]
            roof["rocprof_frac"] = round(st_b[dom] / (rp[dom] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
            roof["rocprof_summary"] = os.path.relpath(trace_path(args.shape), ROOT)

    elif args.path == "fused":
        names = STAGES_M if sh.M <= 4 else STAGES_M8
        st_us, n_launch = time_stages(layers, args.launch_reps, names)
        nd_avg = sum(n_distinct) / len(n_distinct)
        st_b = {k: int(round(v)) for k, v in stage_bytes_m(sh, nd_avg).items()}
        dom = max(names, key=lambda k: st_us[k])
        k_gbs = st_b[dom] / (st_us[dom] * 1e-6) / 1e9
        log("steps (HIP events over stage graphs, %d each): %s" % (n_launch, ", ".join(
            "%s %.2f us %.0f GB/s" % (k, st_us[k], st_b[k] / (st_us[k] * 1e-6) / 1e9)
            for k in names)))
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(k_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(k_gbs / HBM_PEAK_GBS, 4),
                "traffic": None, "avg_launch_us": round(st_us[dom], 3),
                "bytes_per_launch": st_b[dom], "launches_timed": n_launch,
                "frac_method": "HIP events around %d replays of a graph of the step alone for "
                               "every layer, divided by the launches; bytes at the stack's mean "
                               "distinct experts per layer" % args.launch_reps,
                "per_kernel_us": {k: round(v, 3) for k, v in st_us.items()},
                "per_kernel_bytes": st_b}

    out = {
        # the headline metric is quoted at one token per layer; other token
        # counts name theirs
        "metric": METRIC if sh.M == 1 else METRIC.replace("M=1", "M=%d" % sh.M),
        "value": round(gbs_expert, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "%d-layer %s MoE decode stack as one hipGraph: M=%d, H=%d, E=%d, "
                               "top-%d renormalised, I=%d, shared Is=%d, fp16"
                               % (args.layers, "TP=4-shard" if args.shape.startswith("tp4")
                                  else "full-width", sh.M, sh.H, sh.E, sh.K, sh.I, sh.Is),
                   "shape": args.shape,
                   "tokens": sh.M,
                   "distinct_experts_per_layer": round(sum(n_distinct) / len(n_distinct), 2),
                   "layers": args.layers, "layer_seeds": "0..%d" % (args.layers - 1),
                   "path": args.path},
        "us_per_layer": round(us_layer, 3),
        "us_per_layer_p10_p50_p90": pct,
        "frac_of_peak": round(gbs_expert / HBM_PEAK_GBS, 4),
        "gbs_total": round(gbs_total, 1),
        "expert_bytes_per_layer": expert_b // args.layers,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_probes:
        del stack
        out["probes"] = probes(dev)
        log("probes: %s" % out["probes"])
        out["frac_of_read_probe"] = round(gbs_expert / out["probes"]["read_2GiB_GBs"], 4)
    if not args.no_cpu_baseline and sh.M == 1:
        log("timing the fp64 oracle on the host (~%.0f s)" % args.cpu_budget)
        out["cpu_baseline"] = cpu_baseline(tensors, sh, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
