"""Test-side helpers: margin-guarded seeded cases, oracle references and the
comparison rules of the parity tests.

Tolerances:
  * expert ids: identical, element by element, in order;
  * logits: |L_gpu - L| <= gamma * sum_h |Wr[e,h] x[h]| with
    gamma = (H/64 + 6) * 2^-24 * 1.01: each lane runs a serial chain of H/128
    v_dot2 ops (at most two roundings each) and the wave tree adds 6 levels;
  * routing weights: |dw_k| <= sum_j |dw_k/dL_j| |dL_j| <= dLmax / 2 for
    renormalised weights (dLmax for the unnormalised ones), plus 2e-6 for the
    fp32 exp / sum / divide;
  * y (fp16): relative L2 <= 2e-3 and max-abs <= 2e-2 against the fp64 oracle.
A drawn x is replaced (synth.redraw_x) until, for every token, neighbouring
logits among the top-(K+1) are more than GUARD_FACTOR x that token's largest
logit bound apart.  Any factor above 2 makes the GPU's fp32 order provably the
oracle's fp64 order (each logit moves by at most its bound); 4 leaves slack.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from routed_expert_gemv_amd import synth

GUARD_FACTOR = 4.0
Y_REL_L2 = 2e-3
Y_MAX_ABS = 2e-2
MAX_ATTEMPTS = 64


# Widths away from the powers of two: H = 512*HC for HC = 3, 5, 6, 7, and
# down-projection rows with an exact three-chunk lane mapping (I = 192: 8 lanes,
# 384: 16, 768: 32) or a padded one (320, 448, 576, 704, 960, 1088, 1536, 1984).
WIDE_SHAPES = [
    synth.LayerShape(M=1, H=2048, E=128, K=8, I=768, Is=768),
    synth.LayerShape(M=1, H=2048, E=128, K=8, I=768, Is=0),
    synth.LayerShape(M=4, H=3072, E=64, K=8, I=192, Is=192),
    synth.LayerShape(M=1, H=1536, E=32, K=4, I=320, Is=448),
    synth.LayerShape(M=2, H=2560, E=64, K=6, I=960, Is=1088),
    synth.LayerShape(M=8, H=1536, E=256, K=8, I=1536, Is=0),
    synth.LayerShape(M=3, H=3584, E=16, K=4, I=384, Is=640),
    synth.LayerShape(M=1, H=4096, E=64, K=8, I=1984, Is=1984),
    synth.LayerShape(M=5, H=1024, E=32, K=5, I=576, Is=576),
    synth.LayerShape(M=1, H=2560, E=256, K=8, I=384, Is=384),
    synth.LayerShape(M=7, H=1536, E=48, K=7, I=704, Is=0),
]


def host64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def required_margin(t: dict, shape: synth.LayerShape) -> np.ndarray:
    """Per-token routing margin that makes the selection provably identical."""
    return GUARD_FACTOR * logit_bound(t, shape).max(axis=-1)


def draw_case(shape: synth.LayerShape, seed: int, device) -> dict:
    """Seeded layer with x redrawn until every token's routing margin is provably safe."""
    t = synth.draw_layer(shape, seed, device)
    wr64 = host64(t["wr"])
    for attempt in range(MAX_ATTEMPTS):
        if attempt > 0:
            t["x"] = synth.redraw_x(shape, seed, attempt, device)
        lg = oracle.router_logits(host64(t["x"]), wr64)
        _, _, margin = oracle.topk_softmax(lg, shape.K, shape.renormalize)
        if np.all(margin > required_margin(t, shape)):
            t["attempt"] = attempt
            t["margin"] = margin
            return t
    raise RuntimeError("no x with a safe routing margin in %d attempts" % MAX_ATTEMPTS)


def oracle_reference(t: dict, shape: synth.LayerShape, nthreads: int = 1) -> dict:
    """fp64 oracle of the layer; only the selected experts' slices are brought to the host."""
    w13, w2 = t["w13"], t["w2"]

    def fetch(ids):
        idx = torch.as_tensor(np.asarray(ids, dtype=np.int64), device=w13.device)
        return host64(w13.index_select(0, idx)), host64(w2.index_select(0, idx))

    return oracle.moe_layer_fetch(host64(t["x"]), host64(t["wr"]), fetch, host64(t["wsgu"]),
                                  host64(t["wsd"]), K=shape.K, renormalize=shape.renormalize,
                                  nthreads=nthreads)


def logit_bound(t: dict, shape: synth.LayerShape) -> np.ndarray:
    gamma = (shape.H / 64 + 6) * 2.0 ** -24 * 1.01
    return gamma * (np.abs(host64(t["x"])) @ np.abs(host64(t["wr"])).T) + 1e-30


def check_route(ids, w, logits, ref, t, shape, where=""):
    ids = ids.cpu().numpy()
    np.testing.assert_array_equal(ids, ref["expert_ids"], err_msg="expert ids " + where)
    bound = logit_bound(t, shape)
    lg = logits.double().cpu().numpy()
    err = np.abs(lg - ref["logits"])
    assert np.all(err <= bound), "logit error %g above bound %g %s" % (
        err.max(), bound[err > bound].min(), where)
    dl = bound.max(axis=-1, keepdims=True)
    tol = (0.5 if shape.renormalize else 1.0) * dl + 2e-6
    werr = np.abs(w.double().cpu().numpy() - ref["weights"])
    assert np.all(werr <= tol), "weight error %g %s" % (werr.max(), where)
    if shape.renormalize:
        assert np.all(np.abs(w.double().cpu().numpy().sum(-1) - 1.0) <= 1e-6)


def y_errors(y, ref_y):
    yg = y.double().cpu().numpy().reshape(ref_y.shape)
    rel = np.linalg.norm(yg - ref_y) / max(np.linalg.norm(ref_y), 1e-300)
    mx = np.abs(yg - ref_y).max()
    return rel, mx


def check_y(y, ref_y, where=""):
    rel, mx = y_errors(y, ref_y)
    assert rel <= Y_REL_L2, "rel-L2 %g > %g %s" % (rel, Y_REL_L2, where)
    assert mx <= Y_MAX_ABS, "max-abs %g > %g %s" % (mx, Y_MAX_ABS, where)
    return rel, mx


def single_launch(shape: synth.LayerShape) -> bool:
    """Whether moe_layer_decode runs these sizes as the single-launch layer on
    an MI355X (256 CUs in 8 XCDs): the bounds moe_decode.h states for it."""
    if shape.M != 1 or shape.H not in (1024, 2048) or not 1 <= shape.E <= 256:
        return False
    if not 1 <= shape.K <= min(8, shape.E) or shape.I not in (64, 128, 256, 512, 1024):
        return False
    if shape.Is not in (0, shape.I) or shape.K * shape.I > 4096:
        return False
    rpl = 64 // (64 if shape.I >= 512 else shape.I // 8)
    rpw = shape.H // 256
    return rpw % rpl == 0 and rpw // rpl <= 8
