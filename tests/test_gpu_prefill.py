"""moe_layer_prefill (T tokens at once, matrix cores) against the fp64 oracle.

With many tokens some have logits closer together than the fp32 router's
rounding error, so more than one top-K order is correct for them.  The checks
therefore take the route apart:
  * logits: |L_gpu - L| <= gamma * sum_h |Wr[e,h] x[t,h]| with gamma = H * 2^-23,
    the bound for fp32 sums of H exact products in any order, with round to
    nearest or toward zero (the matrix-core sums are not in a fixed serial
    order);
  * top-K + weights: the GPU's ids are exactly the oracle's top-K of the GPU's
    own logits (widened to fp64, exact), and its weights match the oracle's
    weights of those logits within 2e-6;
  * every token whose oracle margin exceeds GUARD x its largest logit bound has
    exactly the oracle's ids;
  * y: within the layer tolerance (rel-L2 2e-3, max-abs 2e-2) of the oracle's
    output for the route the GPU took (its ids, with the oracle's fp64 weights
    for those ids).
The routed activations are rounded to fp16 before the down products (the
worklog's pipeline stores `activated` in fp16, part 10); the bound above is
unaffected and y stays well inside its tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_gemv_amd as moe
from routed_expert_gemv_amd import synth
from tests import cases

pytestmark = pytest.mark.gpu
DEV = "cuda"
GUARD = 4.0


def _shape(T, H, E, K, I, Is, renorm=True):
    return synth.LayerShape(M=T, H=H, E=E, K=K, I=I, Is=Is, renormalize=renorm)


SMALL = [
    _shape(200, 512, 16, 4, 128, 64),        # ragged token tail, 50 pairs per expert
    _shape(300, 1024, 8, 2, 256, 128),       # 75 pairs per expert
    _shape(1, 512, 16, 4, 128, 128),         # one token
    _shape(7, 192, 16, 4, 64, 64),           # odd k-step count (3), I = 64: half the waves idle
    _shape(130, 64, 32, 8, 64, 0),           # one k step, no shared expert (combine alone)
    _shape(96, 512, 64, 8, 128, 0, False),   # unnormalised weights, no shared expert
    _shape(64, 256, 1024, 16, 64, 64),       # largest E and K
    _shape(257, 512, 100, 6, 192, 320),      # E, I, Is not powers of two; ragged column tiles
    _shape(520, 512, 8, 2, 128, 64),         # ~130 pairs per expert: some experts span two row tiles
    _shape(1030, 256, 4, 2, 64, 0),          # ~515 pairs per expert: four and five row tiles, ragged
]


def _id(s):
    return "T%d_H%d_E%d_K%d_I%d_Is%d_r%d" % (s.M, s.H, s.E, s.K, s.I, s.Is, s.renormalize)


def _run(t, sh, ws=None):
    out = moe.moe_layer_prefill(t["x"], t["wr"], t["w13"], t["w2"], t["wsgu"], t["wsd"],
                                K=sh.K, renormalize=sh.renormalize, ws=ws)
    torch.cuda.synchronize()
    return out


def _pf_bound(t, sh):
    gamma = sh.H * 2.0 ** -23
    return gamma * (np.abs(cases.host64(t["x"])) @ np.abs(cases.host64(t["wr"])).T) + 1e-30


def _check_route(t, sh, ids, w, logits, ref_logits, where):
    """The route checks of the module docstring; returns the GPU ids (numpy)."""
    bound = _pf_bound(t, sh)
    lg = logits.double().cpu().numpy()
    err = np.abs(lg - ref_logits)
    assert np.all(err <= bound), "logit error %g above its bound %s" % (err.max(), where)
    gi = ids.cpu().numpy()
    gw = w.double().cpu().numpy()
    own_ids, own_w, _ = oracle.topk_softmax(lg, sh.K, sh.renormalize)
    np.testing.assert_array_equal(gi, own_ids, err_msg="top-K of the GPU logits " + where)
    assert np.abs(gw - own_w).max() <= 2e-6, "weights of the GPU logits " + where
    ref_ids, _, margin = oracle.topk_softmax(ref_logits, sh.K, sh.renormalize)
    safe = margin > GUARD * bound.max(axis=-1)
    np.testing.assert_array_equal(gi[safe], ref_ids[safe], err_msg="unambiguous tokens " + where)
    differ = int((gi[~safe] != ref_ids[~safe]).any(axis=-1).sum())
    print("%s: %d of %d tokens unambiguous; %d of the others took a route other than the "
          "oracle's" % (where, int(safe.sum()), len(safe), differ), flush=True)
    return gi


def _oracle_y(t, sh, rows, gi, ref_logits, nthreads=8, whole=False):
    """Oracle y [len(rows), H] for the given tokens under the GPU's route.  With
    whole=True every expert's weights come to the host once (for many tokens);
    otherwise each token's selected slices are fetched on their own."""
    x = cases.host64(t["x"])
    wsgu = cases.host64(t["wsgu"])
    wsd = cases.host64(t["wsd"])
    wts = oracle.route_weights(ref_logits[rows], gi[rows], sh.renormalize)
    if whole:
        w13_all = t["w13"].cpu().numpy().astype(np.float64)
        w2_all = t["w2"].cpu().numpy().astype(np.float64)
    out = np.empty((len(rows), sh.H))
    for n, r in enumerate(rows):
        if whole:
            w13sel, w2sel = w13_all[gi[r]], w2_all[gi[r]]
        else:
            idx = torch.as_tensor(gi[r].astype(np.int64), device=t["w13"].device)
            w13sel = cases.host64(t["w13"].index_select(0, idx))
            w2sel = cases.host64(t["w2"].index_select(0, idx))
        out[n] = oracle.token_output(x[r], w13sel, w2sel, wts[n], wsgu, wsd, nthreads)
    return out


@pytest.mark.parametrize("sh", SMALL, ids=_id)
def test_prefill_matches_oracle(sh):
    print("prefill", sh, flush=True)
    t = synth.draw_layer(sh, 21, DEV)
    y, ids, w, logits = _run(t, sh)
    ref_logits = oracle.router_logits(cases.host64(t["x"]), cases.host64(t["wr"]), 8)
    gi = _check_route(t, sh, ids, w, logits, ref_logits, _id(sh))
    ref_y = _oracle_y(t, sh, np.arange(sh.M), gi, ref_logits)
    rel, mx = cases.check_y(y, ref_y, _id(sh))
    print("  y rel-L2 %.3g max-abs %.3g" % (rel, mx), flush=True)


def test_prefill_full_width_2048_tokens_sampled():
    """2048 tokens at the full-width shape (the prefill bench workload): every
    token's route is checked; y is checked on 256 sampled tokens, including the
    first and last."""
    sh = _shape(2048, 2048, 256, 8, 512, 512)
    print("prefill full width", sh, flush=True)
    t = synth.draw_layer(sh, 0, DEV)
    y, ids, w, logits = _run(t, sh)
    ref_logits = oracle.router_logits(cases.host64(t["x"]), cases.host64(t["wr"]), 16)
    gi = _check_route(t, sh, ids, w, logits, ref_logits, "full width")
    rows = np.unique(np.concatenate([[0, sh.M - 1],
                                     np.random.default_rng(1).choice(sh.M, 254, replace=False)]))
    ref_y = _oracle_y(t, sh, rows, gi, ref_logits, 16, whole=True)
    rel, mx = cases.check_y(y[rows.tolist()], ref_y, "full width sampled")
    print("  y rel-L2 %.3g max-abs %.3g on %d tokens" % (rel, mx, len(rows)), flush=True)
    # every expert received work: the bench's byte count assumes all 256 are read
    assert len(np.unique(gi)) == sh.E


def test_prefill_is_reproducible_and_stages_compose():
    sh = _shape(333, 1024, 64, 8, 256, 256)
    t = synth.draw_layer(sh, 5, DEV)
    ws = moe.prefill_workspace(sh.M, sh.H, sh.E, sh.I, sh.K, sh.Is)
    y0, ids0, w0, l0 = [v.clone() for v in _run(t, sh, ws)]
    for rep in range(3):  # the expert lists may be filled in another order each call
        y, ids, w, lg = _run(t, sh, ws)
        assert torch.equal(y, y0) and torch.equal(ids, ids0), rep
        assert torch.equal(w, w0) and torch.equal(lg, l0), rep
    outs = None
    for stage in range(1, 7):
        outs = moe.moe_dbg_prefill_stage(stage, t["x"], t["wr"], t["w13"], t["w2"], t["wsgu"],
                                         t["wsd"], K=sh.K, renormalize=True, ws=ws,
                                         y=outs[0] if outs else None,
                                         topk_ids=outs[1] if outs else None,
                                         topk_w=outs[2] if outs else None,
                                         logits=outs[3] if outs else None)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], y0) and torch.equal(outs[1], ids0)


def test_prefill_graph_replays_match_eager():
    sh = _shape(512, 2048, 256, 8, 512, 512)
    t = synth.draw_layer(sh, 9, DEV)
    ws = moe.prefill_workspace(sh.M, sh.H, sh.E, sh.I, sh.K, sh.Is)
    y_e, ids_e, _, _ = [v.clone() for v in _run(t, sh, ws)]
    y = torch.empty_like(y_e)
    ids = torch.empty_like(ids_e)
    w = torch.empty((sh.M, sh.K), dtype=torch.float32, device=DEV)
    lg = torch.empty((sh.M, sh.E), dtype=torch.float32, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):  # captures on torch's capture stream (the current one inside)
        moe.moe_layer_prefill(t["x"], t["wr"], t["w13"], t["w2"], t["wsgu"], t["wsd"], K=sh.K,
                              topk_ids=ids, topk_w=w, logits=lg, y=y, ws=ws)
    for rep in range(4):
        y.zero_()
        ids.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_e) and torch.equal(ids, ids_e), rep
        if rep % 2 == 0:
            _run(t, sh, ws)  # eager work between replays
