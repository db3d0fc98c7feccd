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


def test_committed_counters_use_the_same_accounting():
    c = json.load(open(bench.COUNTERS))
    st = bench.stage_bytes(synth.SHAPES["full_e256_k8_i512"])
    assert c["algorithmic_bytes_per_dispatch"] == st["k_expand"]
    for k, v in c["other_kernels"].items():
        assert v["algorithmic_bytes_per_dispatch"] == st[k]
    # calibrated HBM bytes within a few percent of the algorithmic bytes: no re-reads
    assert abs(c["hbm_bytes_per_dispatch"] / st["k_expand"] - 1) < 0.03
