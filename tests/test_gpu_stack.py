"""The 36-layer decode stack at full size, in the launch configuration the
benchmark times (one hipGraph of 36 independent full-width layers): every
layer against the fp64 oracle, and every layer's graph output against eager
execution bitwise."""
import sys

import pytest
import torch

from routed_expert_gemv_amd import synth
from routed_expert_gemv_amd.stack import DecodeLayer, DecodeStack
from tests import cases

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_stack36_graph_parity_every_layer():
    sh = synth.SHAPES["full_e256_k8_i512"]
    print("drawing 36 layers", flush=True)
    tensors = [cases.draw_case(sh, s, DEV) for s in range(36)]
    layers = [DecodeLayer(t, sh) for t in tensors]
    st = DecodeStack(layers)
    st.capture()
    for l in layers:
        l.y.zero_()
    st.replay()
    torch.cuda.synchronize()
    graph_y = [l.y.clone() for l in layers]
    for i in range(36):
        print("oracle layer", i, flush=True)
        ref = cases.oracle_reference(tensors[i], sh, nthreads=8)
        l = layers[i]
        cases.check_route(l.topk_ids, l.topk_w, l.logits, ref, tensors[i], sh, "layer %d" % i)
        rel, mx = cases.check_y(l.y, ref["y"], "layer %d" % i)
        print("  rel-L2 %.3g max-abs %.3g" % (rel, mx), flush=True)
    st.forward_eager()
    torch.cuda.synchronize()
    for i, (l, g) in enumerate(zip(layers, graph_y)):
        assert torch.equal(l.y, g), "layer %d: graph and eager differ" % i
    del layers, tensors, st
    torch.cuda.empty_cache()
