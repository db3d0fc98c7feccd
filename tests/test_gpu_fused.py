"""moe_layer_decode (one fused launch where the sizes allow, else the separate
kernels) against the three entry points issued one after another: routing,
logits and y must agree bit for bit, and no bounded wait may give up."""
import pytest
import torch

import routed_expert_gemv_amd as moe
from routed_expert_gemv_amd import synth
from routed_expert_gemv_amd.stack import DecodeLayer, DecodeStack

pytestmark = pytest.mark.gpu
DEV = "cuda"

SHAPES = [
    synth.SHAPES["tiny_e16_k4_i128"],
    synth.SHAPES["tp4_shard_e256_k8_i128"],
    synth.SHAPES["full_e256_k8_i512"],
    synth.LayerShape(M=1, H=2048, E=256, K=16, I=512, Is=512),      # K*I at the LDS limit
    synth.LayerShape(M=1, H=2048, E=128, K=8, I=1024, Is=1024),     # two chunks per lane
    synth.LayerShape(M=1, H=1024, E=1024, K=16, I=64, Is=64),       # largest E
    synth.LayerShape(M=1, H=4096, E=64, K=4, I=256, Is=0),
    synth.LayerShape(M=1, H=2048, E=64, K=1, I=512, Is=512),        # K = 1
    synth.LayerShape(M=1, H=2048, E=64, K=8, I=512, Is=0, renormalize=False),
    # not fusable: the same entry point runs the separate kernels
    synth.LayerShape(M=1, H=2048, E=64, K=8, I=512, Is=128),
    synth.LayerShape(M=4, H=2048, E=256, K=8, I=512, Is=512),
    synth.LayerShape(M=1, H=512, E=16, K=4, I=128, Is=128),
]


def _id(s):
    return "M%d_H%d_E%d_K%d_I%d_Is%d_r%d" % (s.M, s.H, s.E, s.K, s.I, s.Is, s.renormalize)


@pytest.mark.parametrize("shape", SHAPES, ids=_id)
def test_layer_decode_equals_separate_calls_bitwise(shape):
    print("fused vs separate", shape, flush=True)
    t = synth.draw_layer(shape, 11, DEV)
    a = DecodeLayer(t, shape, fused=False)
    b = DecodeLayer(t, shape, fused=True)
    a.forward()
    for rep in range(3):  # the fused kernel re-arms its counters for the next call
        b.y.zero_()
        b.forward()
        torch.cuda.synchronize()
        assert torch.equal(a.topk_ids, b.topk_ids), rep
        assert torch.equal(a.topk_w, b.topk_w), rep
        assert torch.equal(a.logits, b.logits), rep
        assert torch.equal(a.y, b.y), rep
    assert moe.moe_dbg_layer_timeouts(b.ws) == 0


def test_fused_stack_graph_replays_match_eager():
    sh = synth.SHAPES["full_e256_k8_i512"]
    layers = [DecodeLayer(synth.draw_layer(sh, s, DEV), sh) for s in range(6)]
    ref = [DecodeLayer(l.t, sh, fused=False) for l in layers]
    for r in ref:
        r.forward()
    torch.cuda.synchronize()
    st = DecodeStack(layers)
    st.capture()
    for rep in range(10):
        for l in layers:
            l.y.zero_()
        st.replay()
        torch.cuda.synchronize()
        for i, (l, r) in enumerate(zip(layers, ref)):
            assert torch.equal(l.y, r.y), "replay %d layer %d" % (rep, i)
            assert torch.equal(l.topk_ids, r.topk_ids)
        if rep % 3 == 0:
            for r in ref:
                r.forward()
    for l in layers:
        assert moe.moe_dbg_layer_timeouts(l.ws) == 0
