"""Host-side checks of bench.py's byte accounting (no GPU): the per-launch
algorithmic bytes cover the layer's weights once, and the committed counter
summary was taken against the same accounting."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from routed_expert_gemv_amd import synth  # noqa: E402


def test_stage_bytes_cover_the_layer_once():
    for name in ("full_e256_k8_i512", "tp4_shard_e256_k8_i128", "tiny_e16_k4_i128"):
        sh = synth.SHAPES[name]
        st = bench.stage_bytes(sh)
        expert, total = bench.layer_bytes(sh, sh.K)
        # the launches' weights (router, K experts' W13 and W2, the shared
        # expert) are the layer's; what remains is the small hand-off tensors
        # (logits, activations, ids and weights), each written once and read once
        extra = sum(st.values()) - total
        assert 0 <= extra < 0.01 * total, (name, extra, total)
        assert st["k_router1"] >= 2 * sh.E * sh.H
        assert st["k_expand"] >= 2 * sh.K * 2 * sh.I * sh.H + 2 * 2 * sh.Is * sh.H
        assert st["k_reduce"] >= 2 * sh.K * sh.H * sh.I + 2 * sh.H * sh.Is


def test_small_batch_step_bytes_cover_the_layer_once():
    # the three steps of an M-token layer read the router, each distinct
    # expert's W13 and W2 and the shared expert once, plus small hand-off
    # tensors (logits, routing outputs, activations, shared output, x, y)
    for name in ("batch2_e256_k8_i512", "batch4_e256_k8_i512", "batch8_e256_k8_i512"):
        sh = synth.SHAPES[name]
        for nd in (sh.K, 16.5, min(sh.M * sh.K, sh.E)):
            st = bench.stage_bytes_m(sh, nd)
            assert list(st) == list(bench.STAGES_M if sh.M <= 4 else bench.STAGES_M8)
            expert, total = bench.layer_bytes(sh, nd)
            extra = sum(st.values()) - total
            assert 0 <= extra < 0.03 * total, (name, nd, extra, total)
            route, expand, w2 = st.values()
            assert route >= 2 * sh.E * sh.H + 2 * 2 * sh.Is * sh.H
            assert expand >= 2 * 2 * nd * sh.I * sh.H + 2 * sh.H * sh.Is
            assert w2 >= 2 * nd * sh.H * sh.I


def test_committed_counters_use_the_same_accounting():
    c = json.load(open(bench.COUNTERS))
    st = bench.stage_bytes(synth.SHAPES["full_e256_k8_i512"])
    assert c["algorithmic_bytes_per_dispatch"] == st["k_expand"]
    for k, v in c["other_kernels"].items():
        assert v["algorithmic_bytes_per_dispatch"] == st[k]
    # calibrated HBM bytes within a few percent of the algorithmic bytes: no re-reads
    assert abs(c["hbm_bytes_per_dispatch"] / st["k_expand"] - 1) < 0.03


def test_committed_traces_and_counters_of_both_single_token_shapes():
    """The committed kernel-trace summaries carry the stage-graph averages that
    bench.py reads, for the kernels it times, and the C2 counter summary uses
    the same byte accounting as the bench."""
    for shape in ("full_e256_k8_i512", "tp4_shard_e256_k8_i128"):
        text = open(bench.trace_path(shape)).read()
        blob = json.loads(text.rsplit("```json", 1)[1].split("```", 1)[0])
        assert set(blob["stage_avg_us"]) == set(bench.STAGES), shape
        assert all(0 < v < 100 for v in blob["stage_avg_us"].values())
        assert len(blob["kernel_source_sha256"]) == 64
        c = json.load(open(bench.counters_path(shape)))
        st = bench.stage_bytes(synth.SHAPES[shape])
        assert c["algorithmic_bytes_per_dispatch"] == st["k_expand"], shape
        assert abs(c["hbm_bytes_per_dispatch"] / st["k_expand"] - 1) < 0.03, shape


def _write_csv(path, header, rows):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_trace_summary_finds_stage_graph_dispatches(tmp_path):
    """Dispatches whose neighbours are the same kernel are the stage graphs'."""
    d = tmp_path / "tr"
    names = ["_ZN3moe9k_router1ILi4EEEvPKDF16_S2_Pf", "_ZN3moe8k_expandILi4E", "_ZN3moe8k_reduceIN"]
    rows, t = [], 0
    for n in names * 2:                    # two full layers
        rows.append([t, t + 1000, n]); t += 2000
    for n, dur in zip(names, (2000, 7000, 4000)):   # a stage graph of 4 launches each
        for _ in range(4):
            rows.append([t, t + dur, n]); t += dur + 100
    _write_csv(str(d / "x" / "tr_kernel_trace.csv"), ["Start_Timestamp", "End_Timestamp", "Kernel_Name"], rows)
    out = tmp_path / "s.md"
    bench.summarize_trace(str(d), str(out), "cmd")
    blob = json.loads(out.read_text().rsplit("```json", 1)[1].split("```", 1)[0])
    assert blob["stage_avg_us"] == {"k_router1": 2.0, "k_expand": 7.0, "k_reduce": 4.0}


def test_pmc_summary_derives_memory_unit_busy(tmp_path):
    d = tmp_path / "p"
    rows = [["_ZN3moe8k_expandILi4E", "TA_BUSY_avr", 100.0], ["_ZN3moe8k_expandILi4E", "GRBM_GUI_ACTIVE", 8000.0],
            ["_ZN3moe8k_expandILi4E", "TA_BUSY_avr", 300.0], ["_ZN3moe8k_expandILi4E", "GRBM_GUI_ACTIVE", 8000.0],
            ["at::native::other", "TA_BUSY_avr", 5.0]]
    _write_csv(str(d / "x" / "pmc_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    out = tmp_path / "c.md"
    bench.summarize_pmc(str(out), [str(d)], ["cmd"], "t")
    line = [l for l in out.read_text().splitlines() if l.startswith("| `k_expand`")][0]
    # TA busy 200 cycles on average over one XCD's 1000 cycles
    assert line.rstrip(" |").endswith("20.0")
    assert "at::native" not in out.read_text()


def test_floor_probe_streams_the_layer_bytes():
    """The launch-structure floors that bench.py's probes measure read the
    full-width layer's bytes launch by launch: the router, expand and reduce
    launches' algorithmic bytes, and the same bytes with the down rows moved
    into the gate/up launch (plus a 1 MiB partial-sum read where a third
    launch remains)."""
    st = bench.stage_bytes(synth.SHAPES["full_e256_k8_i512"])
    router, expand, reduce = st["k_router1"], st["k_expand"], st["k_reduce"]
    fs = bench.FLOOR_STRUCTURES
    assert fs["router+expand+reduce"] == (router, expand, reduce)
    assert fs["router+expand_with_down"] == (router, expand + reduce)
    assert fs["router+expand_with_down+partial_sum"][:2] == (router, expand + reduce)
    assert fs["router+expand_with_down+partial_sum"][2] == 1 << 20
    for sizes in fs.values():
        assert all(n % 16 == 0 for n in sizes)
        # 36 layers on distinct 4 KiB-aligned buffers fit the 2 GiB probe buffer
        assert bench.LAYERS * sum((n + 4095) // 4096 * 4096 for n in sizes) <= 2 << 30
