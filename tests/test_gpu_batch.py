"""Small-batch decode (2..8 tokens) against the same tokens run one at a time.

Each token is routed on its own, so a batch must give every token the routing
of its one-token call: the same logits, expert ids and weights, bit for bit.
The combine at M > 1 streams each distinct expert's down rows once, in order
of first appearance over the batch (token 0's slots, then token 1's new
experts, ...), and adds every token's weighted term as its expert comes by.
So a token's fp32 sum runs in its own routing order exactly when its experts
first appear in the batch in that order; then its y equals the one-token y
bit for bit (token 0 always qualifies).  Every other token sums the same
terms in another order: its y is checked against the one-token y within the
rounding of that reordering (relative L2 <= 1e-3), and against the oracle by
the parity tests.
"""
import dataclasses

import numpy as np
import pytest
import torch

from routed_expert_gemv_amd import synth
from routed_expert_gemv_amd.stack import DecodeLayer
from tests import cases

pytestmark = pytest.mark.gpu
DEV = "cuda"


def first_appearance(ids: np.ndarray) -> dict:
    """Position of each distinct expert in order of first appearance, scanning
    the [M, K] ids row by row."""
    pos = {}
    for e in ids.reshape(-1).tolist():
        pos.setdefault(e, len(pos))
    return pos


@pytest.mark.parametrize("fused", [True, False], ids=["layer", "separate"])
@pytest.mark.parametrize("shape", [
    synth.SHAPES["batch2_e256_k8_i512"],
    synth.SHAPES["batch4_e256_k8_i512"],
    synth.SHAPES["batch8_e256_k8_i512"],
    synth.LayerShape(M=3, H=2048, E=64, K=8, I=256, Is=256),
    synth.LayerShape(M=5, H=1024, E=32, K=6, I=128, Is=0),
], ids=lambda s: "M%d_H%d_E%d_K%d_I%d_Is%d" % (s.M, s.H, s.E, s.K, s.I, s.Is))
def test_batch_token_equals_its_single_token_call(shape, fused):
    print("batch vs single", shape, "fused", fused, flush=True)
    t = cases.draw_case(shape, 5, DEV)
    batch = DecodeLayer(t, shape, fused)
    batch.forward()
    torch.cuda.synchronize()
    ids = batch.topk_ids.cpu().numpy()
    pos = first_appearance(ids)
    one = dataclasses.replace(shape, M=1)
    bitwise = 0
    for m in range(shape.M):
        tm = dict(t)
        tm["x"] = t["x"][m:m + 1].contiguous()
        single = DecodeLayer(tm, one, fused)
        single.forward()
        torch.cuda.synchronize()
        where = "token %d of %d" % (m, shape.M)
        assert torch.equal(single.topk_ids[0], batch.topk_ids[m]), "ids " + where
        assert torch.equal(single.topk_w[0], batch.topk_w[m]), "weights " + where
        assert torch.equal(single.logits[0], batch.logits[m]), "logits " + where
        order = [pos[e] for e in ids[m].tolist()]
        if order == sorted(order):
            assert torch.equal(single.y[0], batch.y[m]), "y " + where
            bitwise += 1
        else:
            a = single.y[0].double().cpu().numpy()
            b = batch.y[m].double().cpu().numpy()
            rel = np.linalg.norm(a - b) / max(np.linalg.norm(a), 1e-300)
            assert rel <= 1e-3, "y %s: rel-L2 %g to the single call" % (where, rel)
    print("  %d of %d tokens bitwise equal to their single-token call" % (bitwise, shape.M),
          flush=True)
    assert bitwise >= 1
