"""The single-launch layer (moe_dbg_layer_stage stage 5, M = 1 on an MI355X)
against the three-launch path and the oracle.

The single launch hands the router logits over inside each XCD and the
activations across the XCDs through flags in the workspace's state block; a
wait that runs out computes the awaited data itself.  Every way must give the
same bits: the three-launch path (stage 4), the single launch (stage 5) and the
single launch with every wait giving up at once (stage 6) -- routing outputs
and y -- within the oracle tolerance, call after call on one workspace (the
per-workgroup call counters advance), and under hipGraph replay.
"""
import numpy as np
import pytest
import torch

import routed_expert_gemv_amd as moe
from routed_expert_gemv_amd import synth
from routed_expert_gemv_amd.stack import DecodeLayer, DecodeStack
from tests import cases

pytestmark = pytest.mark.gpu
DEV = "cuda"
GAVE_UP_WORD = 1024  # word of the state block that counts waits that ran out

SHAPES = [
    synth.SHAPES["tiny_e16_k4_i128"],
    synth.SHAPES["tp4_shard_e256_k8_i128"],
    synth.SHAPES["full_e256_k8_i512"],
    synth.LayerShape(M=1, H=1024, E=256, K=8, I=256, Is=256),
    synth.LayerShape(M=1, H=2048, E=128, K=4, I=1024, Is=1024),
    synth.LayerShape(M=1, H=2048, E=200, K=8, I=64, Is=64),          # ragged E
    synth.LayerShape(M=1, H=2048, E=64, K=1, I=512, Is=512),         # K = 1
    synth.LayerShape(M=1, H=2048, E=64, K=8, I=512, Is=0, renormalize=False),
    synth.LayerShape(M=1, H=2048, E=37, K=5, I=128, Is=0),           # odd K, ragged E
    synth.LayerShape(M=1, H=2048, E=8, K=8, I=64, Is=64),            # K = E
]


def _id(s):
    return "H%d_E%d_K%d_I%d_Is%d_r%d" % (s.H, s.E, s.K, s.I, s.Is, s.renormalize)


def gave_up(ws):
    return int(ws[GAVE_UP_WORD * 4:GAVE_UP_WORD * 4 + 4].view(torch.int32).item())


def run_stage(stage, layer):
    t, sh = layer.t, layer.shape
    moe.moe_dbg_layer_stage(stage, t["x"], t["wr"], t["w13"], t["w2"], t["wsgu"], t["wsd"], sh.K,
                            sh.renormalize, layer.topk_ids, layer.topk_w, layer.logits, layer.y,
                            layer.ws)


def outputs(layer):
    return [layer.topk_ids.clone(), layer.topk_w.clone(), layer.logits.clone(), layer.y.clone()]


def assert_same(a, b, where):
    for name, x, y in zip(("ids", "weights", "logits", "y"), a, b):
        assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x,
                           y.view(torch.int32) if y.dtype == torch.float32 else y), \
            "%s differ: %s" % (name, where)


def test_shapes_take_the_single_launch():
    for sh in SHAPES:
        assert cases.single_launch(sh), sh
    # a shape outside its bounds is refused (E > 256)
    sh = synth.LayerShape(M=1, H=2048, E=512, K=8, I=512, Is=512)
    t = synth.draw_layer(sh, 0, DEV)
    with pytest.raises(moe.MoeError):
        run_stage(5, DecodeLayer(t, sh))


@pytest.mark.parametrize("shape", SHAPES, ids=_id)
def test_single_launch_equals_three_launches_and_oracle(shape):
    print("single launch", shape, flush=True)
    t = cases.draw_case(shape, 3, DEV)
    three = DecodeLayer(t, shape)
    run_stage(4, three)
    one = DecodeLayer(t, shape)
    for rep in range(4):  # the call counters advance; results stay the same bits
        one.y.zero_()
        one.topk_ids.zero_()
        run_stage(5, one)
        torch.cuda.synchronize()
        assert_same(outputs(three), outputs(one), "single launch, call %d" % rep)
    assert gave_up(one.ws) == 0
    ref = cases.oracle_reference(t, shape, nthreads=8)
    cases.check_route(one.topk_ids, one.topk_w, one.logits, ref, t, shape, "single launch")
    cases.check_y(one.y, ref["y"], "single launch")


@pytest.mark.parametrize("shape", [synth.SHAPES["tp4_shard_e256_k8_i128"],
                                   synth.SHAPES["full_e256_k8_i512"],
                                   synth.LayerShape(M=1, H=2048, E=37, K=5, I=128, Is=0)],
                         ids=_id)
def test_waits_that_give_up_compute_the_same_bits(shape):
    """Stage 6 gives every wait a limit of zero: each workgroup computes the
    logits and every activation itself, with the same device functions."""
    print("gave-up path", shape, flush=True)
    t = cases.draw_case(shape, 9, DEV)
    normal = DecodeLayer(t, shape)
    run_stage(5, normal)
    forced = DecodeLayer(t, shape)
    run_stage(6, forced)
    run_stage(5, forced)  # and the normal path again on the same workspace
    torch.cuda.synchronize()
    assert gave_up(forced.ws) >= 256
    before = gave_up(forced.ws)
    run_stage(6, forced)
    torch.cuda.synchronize()
    assert gave_up(forced.ws) > before
    assert_same(outputs(normal), outputs(forced), "gave-up path")
    assert gave_up(normal.ws) == 0


def test_layers_sharing_one_workspace():
    """Layers of different sizes issued in turn on one workspace (as a stack
    that reuses it would) give what each gives on a workspace of its own."""
    shapes = [synth.SHAPES["full_e256_k8_i512"], synth.SHAPES["tp4_shard_e256_k8_i128"],
              synth.SHAPES["tiny_e16_k4_i128"]]
    own = [DecodeLayer(cases.draw_case(sh, 20 + i, DEV), sh) for i, sh in enumerate(shapes)]
    ws = moe.workspace(1, 2048, 256, 512, 8, 512, DEV)
    shared = [DecodeLayer(l.t, l.shape) for l in own]
    for l in shared:
        l.ws = ws
    for l in own:
        run_stage(5, l)
    for rep in range(3):
        for l in shared:
            run_stage(5, l)
    torch.cuda.synchronize()
    for a, b in zip(own, shared):
        assert_same(outputs(a), outputs(b), "shared workspace %s" % (a.shape,))
    assert gave_up(ws) == 0


def test_workspace_init_clears_the_state_block():
    sh = synth.SHAPES["full_e256_k8_i512"]
    t = cases.draw_case(sh, 4, DEV)
    ref = DecodeLayer(t, sh)
    run_stage(5, ref)
    layer = DecodeLayer(t, sh)
    layer.ws.fill_(0x5A)           # a workspace that did not come zero-filled
    moe.moe_workspace_init(layer.ws)
    for _ in range(2):
        run_stage(5, layer)
    torch.cuda.synchronize()
    assert_same(outputs(ref), outputs(layer), "after moe_workspace_init")
    assert gave_up(layer.ws) == 0


def test_stack_graph_of_single_launches_matches_eager():
    """36-layer style stack (here 8 layers of the TP=4 shard shape) as one hipGraph:
    every replay equals the eager results, with eager work between replays."""
    sh = synth.SHAPES["tp4_shard_e256_k8_i128"]
    layers = [DecodeLayer(synth.draw_layer(sh, s, DEV), sh) for s in range(8)]
    for l in layers:
        run_stage(5, l)
    torch.cuda.synchronize()
    eager = [outputs(l) for l in layers]
    st = DecodeStack(layers)

    def single_launches(stream=None):
        for l in layers:
            run_stage(5, l)

    st.forward_eager = single_launches
    st.capture()
    for rep in range(8):
        for l in layers:
            l.y.zero_()
        st.replay()
        torch.cuda.synchronize()
        for i, l in enumerate(layers):
            assert_same(eager[i], outputs(l), "replay %d layer %d" % (rep, i))
        if rep % 3 == 1:
            st.forward_eager()
            torch.cuda.synchronize()
    assert all(gave_up(l.ws) == 0 for l in layers)
