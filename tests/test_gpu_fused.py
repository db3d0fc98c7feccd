"""moe_layer_decode against the three entry points issued one after another.

Every way of running the layer (three launches at M = 1, three or four for
small batches, else the separate kernels) must agree with the three calls
bit for bit: routing outputs (ids, weights, logits) and y.  The results must also be reproducible call after
call on the same workspace, equal under graph replay, and within the oracle
tolerance.
"""
import pytest
import torch

import routed_expert_gemv_amd as moe
from routed_expert_gemv_amd import synth
from routed_expert_gemv_amd.stack import DecodeLayer, DecodeStack
from tests import cases

pytestmark = pytest.mark.gpu
DEV = "cuda"

SHAPES = [
    synth.SHAPES["tiny_e16_k4_i128"],
    synth.SHAPES["tp4_shard_e256_k8_i128"],
    synth.SHAPES["full_e256_k8_i512"],
    synth.LayerShape(M=1, H=2048, E=256, K=16, I=512, Is=512),
    synth.LayerShape(M=1, H=2048, E=128, K=8, I=1024, Is=1024),
    synth.LayerShape(M=1, H=1024, E=1024, K=16, I=64, Is=64),       # largest E
    synth.LayerShape(M=1, H=4096, E=64, K=4, I=256, Is=0),
    synth.LayerShape(M=1, H=2048, E=64, K=1, I=512, Is=512),        # K = 1
    synth.LayerShape(M=1, H=2048, E=64, K=8, I=512, Is=0, renormalize=False),
    synth.LayerShape(M=1, H=2048, E=64, K=8, I=512, Is=128),
    synth.LayerShape(M=1, H=2048, E=64, K=3, I=256, Is=64),         # odd K, Is < I
    synth.LayerShape(M=1, H=512, E=16, K=4, I=128, Is=128),
    synth.LayerShape(M=1, H=512, E=8, K=2, I=2048, Is=2048),        # longest rows
    # several tokens: three launches up to 4 tokens, four above
    synth.LayerShape(M=4, H=2048, E=256, K=8, I=512, Is=512),
    synth.LayerShape(M=2, H=4096, E=64, K=4, I=256, Is=256),
    synth.LayerShape(M=8, H=1024, E=32, K=4, I=128, Is=0),
    synth.LayerShape(M=3, H=2048, E=1024, K=16, I=64, Is=64),
    # the selection launch with 4, 16 and 1 logits per lane
    synth.LayerShape(M=6, H=2048, E=256, K=8, I=256, Is=256),
    synth.LayerShape(M=7, H=1024, E=1024, K=16, I=64, Is=64),
    synth.LayerShape(M=5, H=512, E=64, K=6, I=128, Is=0, renormalize=False),
    # the same entry point runs the separate kernels
    synth.LayerShape(M=1, H=2048, E=16, K=16, I=2048, Is=0),        # K*I above the LDS stage
] + cases.WIDE_SHAPES


def _id(s):
    return "M%d_H%d_E%d_K%d_I%d_Is%d_r%d" % (s.M, s.H, s.E, s.K, s.I, s.Is, s.renormalize)


@pytest.mark.parametrize("shape", SHAPES, ids=_id)
def test_layer_decode_against_separate_calls(shape):
    print("fused vs separate", shape, flush=True)
    t = cases.draw_case(shape, 11, DEV)
    a = DecodeLayer(t, shape, fused=False)
    b = DecodeLayer(t, shape, fused=True)
    a.forward()
    launches = moe.moe_layer_launches(shape.M, shape.H, shape.E, shape.I, shape.K, shape.Is)
    if shape.M > 1:
        # 3; 4 with the selection launch (M = 5..8) or with a shared down
        # launch of its own (M <= 4, when token 0's workgroups are too few
        # for the shared down blocks)
        assert launches in ((3, 4) if shape.M <= 4 else (4,))
    else:
        assert launches == (3 if shape.K * shape.I <= 16384 else 4 + (2 if shape.Is else 0))
    first = None
    for rep in range(3):  # the workspace keeps its launch count between calls
        b.y.zero_()
        b.forward()
        torch.cuda.synchronize()
        assert torch.equal(a.topk_ids, b.topk_ids), rep
        assert torch.equal(a.topk_w, b.topk_w), rep
        assert torch.equal(a.logits, b.logits), rep
        if first is None:
            first = b.y.clone()
        assert torch.equal(b.y, first), "not reproducible, call %d" % rep
    assert torch.equal(a.y, b.y)
    if launches == 3:
        ref = cases.oracle_reference(t, shape, nthreads=8)
        cases.check_y(b.y, ref["y"], "three launches")


def test_full_width_layer_runs_as_three_launches():
    sh = synth.SHAPES["full_e256_k8_i512"]
    assert moe.moe_layer_launches(sh.M, sh.H, sh.E, sh.I, sh.K, sh.Is) == 3
    assert moe.moe_layer_launches(2, sh.H, sh.E, sh.I, sh.K, sh.Is) == 3
    assert moe.moe_layer_launches(8, sh.H, sh.E, sh.I, sh.K, sh.Is) == 4


def test_fused_stack_graph_replays_match_eager():
    sh = synth.SHAPES["full_e256_k8_i512"]
    layers = [DecodeLayer(synth.draw_layer(sh, s, DEV), sh) for s in range(6)]
    for l in layers:
        l.forward()
    torch.cuda.synchronize()
    eager = [l.y.clone() for l in layers]
    ids = [l.topk_ids.clone() for l in layers]
    st = DecodeStack(layers)
    st.capture()
    for rep in range(10):
        for l in layers:
            l.y.zero_()
        st.replay()
        torch.cuda.synchronize()
        for i, l in enumerate(layers):
            assert torch.equal(l.y, eager[i]), "replay %d layer %d" % (rep, i)
            assert torch.equal(l.topk_ids, ids[i])
        if rep % 3 == 0:
            st.forward_eager()  # eager work between replays
            torch.cuda.synchronize()


@pytest.mark.parametrize("shape", [
    synth.SHAPES["full_e256_k8_i512"],                         # shared as wide as a routed expert
    synth.LayerShape(M=1, H=2048, E=64, K=8, I=512, Is=0),     # no shared expert
    synth.LayerShape(M=1, H=2048, E=64, K=8, I=512, Is=128),   # narrower shared expert
    synth.SHAPES["batch2_e256_k8_i512"],                       # selection in the expand launch
    synth.SHAPES["batch4_e256_k8_i512"],
    synth.SHAPES["batch8_e256_k8_i512"],                       # a selection launch of its own
    synth.LayerShape(M=3, H=1024, E=96, K=6, I=192, Is=0),     # odd sizes, no shared expert
], ids=_id)
def test_layer_stages_in_order_equal_the_full_call(shape):
    """The layer's three steps run one at a time through moe_dbg_layer_stage
    (how bench times each step) give the full call's outputs bit for bit."""
    print("stages vs full call", shape, flush=True)
    t = cases.draw_case(shape, 5, DEV)
    full = DecodeLayer(t, shape)
    full.forward()
    staged = DecodeLayer(t, shape)
    for stage in (1, 2, 3):
        moe.moe_dbg_layer_stage(stage, t["x"], t["wr"], t["w13"], t["w2"], t["wsgu"], t["wsd"],
                                shape.K, shape.renormalize, staged.topk_ids, staged.topk_w,
                                staged.logits, staged.y, staged.ws)
    torch.cuda.synchronize()
    assert torch.equal(full.logits, staged.logits)
    assert torch.equal(full.topk_ids, staged.topk_ids)
    assert torch.equal(full.topk_w, staged.topk_w)
    assert torch.equal(full.y, staged.y)


@pytest.mark.parametrize("name", ["batch2_e256_k8_i512", "batch8_e256_k8_i512"])
def test_small_batch_stack_graph_replays_match_eager(name):
    """Small-batch layers (the selection folded into the expand launch at
    M <= 4, a launch of its own at M = 8) under hipGraph replay: every replay
    equals the eager results bit for bit, with eager work between replays."""
    sh = synth.SHAPES[name]
    print("small-batch stack graph", name, flush=True)
    layers = [DecodeLayer(synth.draw_layer(sh, s, DEV), sh) for s in range(4)]
    for l in layers:
        l.forward()
    torch.cuda.synchronize()
    eager = [(l.y.clone(), l.topk_ids.clone(), l.topk_w.clone()) for l in layers]
    st = DecodeStack(layers)
    st.capture()
    for rep in range(6):
        for l in layers:
            l.y.zero_()
            l.topk_ids.zero_()
        st.replay()
        torch.cuda.synchronize()
        for i, l in enumerate(layers):
            assert torch.equal(l.y, eager[i][0]), "replay %d layer %d" % (rep, i)
            assert torch.equal(l.topk_ids, eager[i][1])
            assert torch.equal(l.topk_w, eager[i][2])
        if rep % 2 == 0:
            st.forward_eager()
            torch.cuda.synchronize()


@pytest.mark.parametrize("M", [2, 3, 4])
def test_tied_logits_shared_experts_layer_equals_separate_calls(M):
    """Router rows in identical pairs (experts 2j and 2j+1 always tie) and
    tokens that are small perturbations of one another, so the tokens share
    most of their experts and break ties by id: the layer (which finds each
    shared expert's tokens and slots from every token's own order) equals
    the separate calls (which read them from the group table) bit for bit,
    and every token's ids are the top-K of its own logits under (logit
    descending, id ascending)."""
    sh = synth.LayerShape(M=M, H=2048, E=128, K=8, I=256, Is=256)
    print("tied pairs", sh, flush=True)
    t = synth.draw_layer(sh, 21, DEV)
    t["wr"] = t["wr"][0::2].repeat_interleave(2, dim=0).contiguous()
    g = torch.Generator(device=DEV).manual_seed(77)
    x0 = t["x"][:1].float()
    noise = torch.randn((M, sh.H), generator=g, device=DEV) * 0.05
    noise[0] = 0
    t["x"] = (x0 + noise).half().contiguous()
    a = DecodeLayer(t, sh, fused=False)
    b = DecodeLayer(t, sh, fused=True)
    a.forward()
    b.forward()
    torch.cuda.synchronize()
    assert torch.equal(a.topk_ids, b.topk_ids)
    assert torch.equal(a.topk_w, b.topk_w)
    assert torch.equal(a.y, b.y)
    lg = b.logits.cpu()
    ids = b.topk_ids.cpu()
    shared = 0
    for m in range(M):
        order = sorted(range(sh.E), key=lambda e: (-lg[m, e].item(), e))
        assert ids[m].tolist() == order[:sh.K], m
        if m:
            shared += len(set(ids[m].tolist()) & set(ids[0].tolist()))
    assert shared > 0  # the tokens do share experts
