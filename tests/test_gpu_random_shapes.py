"""96 seeded random layer sizes across the accepted range (CPU-drawn sizes,
fixed seed, so the list is the same in every run): for each, moe_layer_decode
against the three entry points bit for bit (routing outputs and y), the
layer's steps run one at a time against the full call bit for bit, and the
routing and y against the fp64 oracle.  Sizes: M 1..8, H a multiple of 512 up
to 4096 (M <= 4 above 2048), E up to 512, K up to min(E, 16), I and Is
multiples of 64 up to 1024 (Is also 0), renormalised or not."""
import random

import pytest
import torch

import routed_expert_gemv_amd as moe
from routed_expert_gemv_amd import synth
from routed_expert_gemv_amd.stack import DecodeLayer
from tests import cases

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _shapes(n=96, seed=20261203):
    rng = random.Random(seed)
    out = []
    while len(out) < n:
        M = rng.randint(1, 8)
        H = 512 * rng.randint(1, 8 if M <= 4 else 4)
        E = rng.choice([8, 16, 24, 40, 64, 96, 128, 200, 256, 320, 512])
        K = rng.randint(1, min(E, 16))
        I = 64 * rng.randint(1, 16)
        Is = rng.choice([0, 64 * rng.randint(1, 16), I])
        out.append(synth.LayerShape(M=M, H=H, E=E, K=K, I=I, Is=Is,
                                    renormalize=rng.random() < 0.8))
    return out


SHAPES = _shapes()


def _id(s):
    return "M%d_H%d_E%d_K%d_I%d_Is%d_r%d" % (s.M, s.H, s.E, s.K, s.I, s.Is, s.renormalize)


@pytest.mark.parametrize("i", range(len(SHAPES)), ids=[_id(s) for s in SHAPES])
def test_random_shape(i):
    sh = SHAPES[i]
    print("random shape", i, sh, flush=True)
    t = cases.draw_case(sh, 100 + i, DEV)
    sep = DecodeLayer(t, sh, fused=False)
    lay = DecodeLayer(t, sh, fused=True)
    sep.forward()
    lay.forward()
    torch.cuda.synchronize()
    assert torch.equal(sep.topk_ids, lay.topk_ids)
    assert torch.equal(sep.topk_w, lay.topk_w)
    assert torch.equal(sep.logits, lay.logits)
    assert torch.equal(sep.y, lay.y)
    if moe.moe_layer_launches(sh.M, sh.H, sh.E, sh.I, sh.K, sh.Is) in (3, 4):
        staged = DecodeLayer(t, sh)
        for stage in (1, 2, 3):
            moe.moe_dbg_layer_stage(stage, t["x"], t["wr"], t["w13"], t["w2"], t["wsgu"],
                                    t["wsd"], sh.K, sh.renormalize, staged.topk_ids,
                                    staged.topk_w, staged.logits, staged.y, staged.ws)
        torch.cuda.synchronize()
        assert torch.equal(staged.y, lay.y)
        assert torch.equal(staged.topk_ids, lay.topk_ids)
    ref = cases.oracle_reference(t, sh, nthreads=8)
    cases.check_route(lay.topk_ids, lay.topk_w, lay.logits, ref, t, sh, "random %d" % i)
    cases.check_y(lay.y, ref["y"], "random %d" % i)
