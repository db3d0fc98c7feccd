"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each test ties one part of the oracle to a library routine, a closed form, a
brute-force enumeration, a value printed on the pages or an invariant of the
mathematics, so that a plausible slip (a dropped term, a wrong sign, a
transposed operand, gate/up swapped, a wrong weight index, a wrong tie rule)
fails at least one of them.  No GPU is needed.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special as sp
import torch
import torch.nn.functional as F

import oracle
from routed_expert_gemv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SILU1 = 0.7310585786300049  # 1 / (1 + e^-1), textbook value of silu(1)


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- router GEMV
def test_router_matches_library_matmul_nonsquare():
    r = _rng(1)
    E, H, M = 24, 64, 3
    wr = r.standard_normal((E, H))
    x = r.standard_normal((M, H))
    got = oracle.router_logits(x, wr)
    want = x @ wr.T
    assert got.shape == (M, E)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


def test_router_one_hot_rows_pick_columns():
    # x = e_j selects column j of the router: a transposed operand fails here
    E, H = 5, 7
    wr = np.arange(E * H, dtype=np.float64).reshape(E, H)
    for j in range(H):
        x = np.zeros(H)
        x[j] = 1.0
        np.testing.assert_array_equal(oracle.router_logits(x, wr), wr[:, j])


# ---------------------------------------------------------------- top-k + softmax
def _selected_by_definition(logits, K):
    """Brute force over all K-subsets: the selected set S is the only one where every
    member outranks every non-member under (logit desc, id asc)."""
    E = len(logits)
    found = []
    for S in itertools.combinations(range(E), K):
        inside = set(S)
        ok = all((logits[a], -a) > (logits[b], -b) for a in S for b in range(E) if b not in inside)
        if ok:
            found.append(S)
    assert len(found) == 1
    S = found[0]
    return sorted(S, key=lambda e: (-logits[e], e))


@pytest.mark.parametrize("seed", range(12))
def test_topk_bruteforce_e16_k4_distinct(seed):
    r = _rng(100 + seed)
    logits = r.standard_normal(16)
    ids, w, margin = oracle.topk_softmax(logits, 4)
    order = _selected_by_definition(list(logits), 4)
    assert list(ids) == order
    # the sum of the selected logits is the largest over all C(16,4) subsets
    best = max(itertools.combinations(range(16), 4), key=lambda S: sum(logits[list(S)]))
    assert set(best) == set(order)
    np.testing.assert_allclose(w, sp.softmax(logits[order]), rtol=1e-14, atol=0)
    top5 = np.sort(logits)[::-1][:5]
    assert margin == pytest.approx(np.min(top5[:-1] - top5[1:]), rel=0, abs=0)


@pytest.mark.parametrize("seed", range(12))
def test_topk_bruteforce_with_ties(seed):
    r = _rng(200 + seed)
    logits = r.integers(0, 4, size=16).astype(np.float64)  # many ties
    ids, w, margin = oracle.topk_softmax(logits, 4)
    assert list(ids) == _selected_by_definition(list(logits), 4)
    np.testing.assert_allclose(w, sp.softmax(logits[ids]), rtol=1e-14)


@pytest.mark.parametrize("E,K", [(16, 4), (256, 8)])
def test_uniform_router_ties_to_lowest_ids(E, K):
    ids, w, margin = oracle.topk_softmax(np.zeros(E), K)
    assert list(ids) == list(range(K))
    np.testing.assert_array_equal(w, np.full(K, 1.0 / K))
    assert margin == 0.0


def test_known_logits_closed_form_weights():
    logits = np.log(np.array([1.0, 2.0, 3.0, 4.0, 0.5]))
    ids, w, _ = oracle.topk_softmax(logits, 4, renormalize=True)
    assert list(ids) == [3, 2, 1, 0]
    np.testing.assert_allclose(w, [0.4, 0.3, 0.2, 0.1], rtol=1e-15)
    ids, w, _ = oracle.topk_softmax(logits, 4, renormalize=False)
    assert list(ids) == [3, 2, 1, 0]
    np.testing.assert_allclose(w, np.array([4.0, 3.0, 2.0, 1.0]) / 10.5, rtol=1e-15)


def test_k_equals_e_is_full_softmax():
    r = _rng(7)
    logits = r.standard_normal(9)
    ids, w, _ = oracle.topk_softmax(logits, 9, renormalize=True)
    assert list(ids) == list(np.argsort(-logits, kind="stable"))
    np.testing.assert_allclose(w, sp.softmax(logits)[ids], rtol=1e-14)
    assert w.sum() == pytest.approx(1.0, abs=1e-15)


def test_unnormalised_weights_are_full_softmax_entries():
    r = _rng(8)
    logits = r.standard_normal(32)
    ids, w, _ = oracle.topk_softmax(logits, 5, renormalize=False)
    np.testing.assert_allclose(w, sp.softmax(logits)[ids], rtol=1e-14)
    assert w.sum() < 1.0


def test_margin_closed_form():
    logits = np.array([5.0, 3.0, 2.5, 1.0, 0.9, -2.0])
    assert oracle.topk_softmax(logits, 2)[2] == pytest.approx(0.5)   # gaps 2, 0.5
    assert oracle.topk_softmax(logits, 4)[2] == pytest.approx(0.1)   # gaps 2, .5, 1.5, .1
    assert oracle.topk_softmax(logits, 1)[2] == pytest.approx(2.0)


# ---------------------------------------------------------------- gate/up + SiLU
def test_activated_worked_example_gate_then_up():
    # x one-hot on column 0: gate_j = column 0 of gate row j, up_j = column 0 of up row j
    H, I = 4, 3
    r = _rng(3)
    w13 = r.standard_normal((2 * I, H))
    w13[:I, 0] = [1.0, -2.0, 0.5]     # gate
    w13[I:, 0] = [2.0, 3.0, -1.0]     # up
    x = np.array([1.0, 0.0, 0.0, 0.0])
    got = oracle.expert_activated(x, w13)
    g = np.array([1.0, -2.0, 0.5])
    u = np.array([2.0, 3.0, -1.0])
    want = g * sp.expit(g) * u
    np.testing.assert_allclose(got, want, rtol=1e-15)
    assert got[0] == pytest.approx(2 * SILU1, rel=1e-15)
    # gate and up swapped would give silu(u) * g instead
    assert not np.allclose(got, u * sp.expit(u) * g)


def test_silu_special_values():
    H, I = 2, 4
    w13 = np.zeros((2 * I, H))
    w13[:I, 0] = [0.0, 40.0, -40.0, -800.0]
    w13[I:, 0] = 1.0
    got = oracle.expert_activated(np.array([1.0, 0.0]), w13)
    assert got[0] == 0.0                      # silu(0) = 0
    assert got[1] == pytest.approx(40.0, rel=1e-15)   # silu(g) -> g for large g
    assert abs(got[2]) < 1e-15                # silu(g) -> 0 for very negative g
    assert got[3] == 0.0 and not math.isnan(got[3])


# ---------------------------------------------------------------- down + combine
def test_page_unit_dot_128_golden():
    fx = json.load(open(os.path.join(GOLDEN, "page_closed_forms.json")))["w2_unit_dot_128"]
    I, H, K = fx["I"], 16, 8
    w2 = [np.full((H, I), fx["w2"]) for _ in range(K)]
    act = np.full((K, I), fx["activated"])
    _, w, _ = oracle.topk_softmax(_rng(5).standard_normal(64), K)
    out = oracle.weighted_down(w2, act, w)
    np.testing.assert_allclose(out, fx["expected"], rtol=1e-14)
    assert not np.allclose(out, fx["wrong_value_seen_on_page"])


def test_combine_known_expert_outputs():
    # expert e: gate = c_e = (e+1)/4, up = 1 -> activated = silu(c_e); its down rows give
    # (e+1)(h+1) silu(c_e).  Router logits chosen so ids and weights are known.
    E, K, H, I = 6, 3, 5, 2
    lg = np.array([0.1, 0.7, -0.3, 0.5, 0.2, 0.6])
    wr = np.zeros((E, H))
    wr[:, 0] = lg
    x = np.zeros((1, H))
    x[0, 0] = 1.0
    c = (np.arange(E) + 1) / 4.0
    w13 = np.zeros((E, 2 * I, H))
    w13[:, :I, 0] = c[:, None]               # gate rows
    w13[:, I:, 0] = 1.0                      # up rows
    w2 = np.zeros((E, H, I))
    for e in range(E):
        w2[e, :, 0] = (e + 1) * (np.arange(H) + 1)
    res = oracle.moe_layer(x, wr, w13, w2, K=K)
    ids = [1, 5, 3]
    assert list(res["expert_ids"][0]) == ids
    sel = np.array([0.7, 0.6, 0.5])
    w = np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum()
    np.testing.assert_allclose(res["weights"][0], w, rtol=1e-15)
    per_expert = [(e + 1) * c[e] * sp.expit(c[e]) for e in ids]
    want = (np.arange(H) + 1) * sum(wk * pe for wk, pe in zip(w, per_expert))
    np.testing.assert_allclose(res["y"][0], want, rtol=1e-14)


# ---------------------------------------------------------------- whole layer
def _layer64(shape, seed):
    t = synth.draw_layer(shape, seed, "cpu")
    return {k: (None if v is None else v.double().numpy()) for k, v in t.items()}


def test_closed_form_unit_layer_is_silu1():
    # x = 1, W13 = 2^-11, W2 = 1/I: g = u = 1 exactly, y = silu(1) * sum(w) = silu(1)
    H, E, K, I, Is = 2048, 16, 4, 128, 128
    r = _rng(11)
    wr = r.standard_normal((E, H)) * 0.02
    x = np.ones((1, H))
    w13 = np.full((E, 2 * I, H), 2.0 ** -11)
    w2 = np.full((E, H, I), 1.0 / I)
    res = oracle.moe_layer(x, wr, w13, w2, K=K)
    np.testing.assert_allclose(res["y"], SILU1, rtol=1e-14)
    wsgu = np.full((2 * Is, H), 2.0 ** -11)
    wsd = np.full((H, Is), 1.0 / Is)
    res = oracle.moe_layer(x, wr, w13, w2, wsgu, wsd, K=K)
    np.testing.assert_allclose(res["y"], 2 * SILU1, rtol=1e-14)


def test_k1_is_dense_swiglu_mlp_torch_library():
    shp = synth.LayerShape(M=2, H=256, E=8, K=1, I=64, Is=32)
    t = _layer64(shp, 21)
    res = oracle.moe_layer(t["x"], t["wr"], t["w13"], t["w2"], t["wsgu"], t["wsd"], K=1)
    X = torch.from_numpy(t["x"])
    for m in range(2):
        e = int(np.argmax(t["x"][m] @ t["wr"].T))
        assert res["expert_ids"][m, 0] == e and res["weights"][m, 0] == 1.0
        W13 = torch.from_numpy(t["w13"][e])
        W2 = torch.from_numpy(t["w2"][e])
        h = F.silu(F.linear(X[m], W13[:64])) * F.linear(X[m], W13[64:])
        y = F.linear(h, W2)
        Wsgu = torch.from_numpy(t["wsgu"])
        hs = F.silu(F.linear(X[m], Wsgu[:32])) * F.linear(X[m], Wsgu[32:])
        y = y + F.linear(hs, torch.from_numpy(t["wsd"]))
        np.testing.assert_allclose(res["y"][m], y.numpy(), rtol=1e-12, atol=1e-14)


def test_shared_expert_alone_is_dense_swiglu():
    r = _rng(31)
    H, Is = 96, 40
    x = r.standard_normal((3, H))
    wsgu = r.standard_normal((2 * Is, H))
    wsd = r.standard_normal((H, Is))
    got = oracle.shared_expert(x, wsgu, wsd)
    X = torch.from_numpy(x)
    hs = F.silu(F.linear(X, torch.from_numpy(wsgu[:Is]))) * F.linear(X, torch.from_numpy(wsgu[Is:]))
    want = F.linear(hs, torch.from_numpy(wsd)).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_expert_relabelling_invariance():
    # the softmax denominator sums all E experts in id order, so relabelling may move
    # the last bit of the weights; selection must be identical
    shp = synth.LayerShape(M=1, H=2048, E=16, K=4, I=128, Is=0)
    t = _layer64(shp, 0)
    res = oracle.moe_layer(t["x"], t["wr"], t["w13"], t["w2"], K=4)
    perm = _rng(9).permutation(16)
    res_p = oracle.moe_layer(t["x"], t["wr"][perm], t["w13"][perm], t["w2"][perm], K=4)
    np.testing.assert_array_equal(perm[res_p["expert_ids"][0]], res["expert_ids"][0])
    np.testing.assert_allclose(res_p["weights"], res["weights"], rtol=1e-14, atol=0)
    np.testing.assert_allclose(res_p["y"], res["y"], rtol=1e-13, atol=1e-16)


def test_scaling_w2_by_two_doubles_output_exactly():
    shp = synth.LayerShape(M=1, H=2048, E=16, K=4, I=128, Is=0)
    t = _layer64(shp, 1)
    a = oracle.moe_layer(t["x"], t["wr"], t["w13"], t["w2"], K=4)
    b = oracle.moe_layer(t["x"], t["wr"], t["w13"], 2.0 * t["w2"], K=4)
    np.testing.assert_array_equal(b["y"], 2.0 * a["y"])


def test_gathered_slices_equal_indexed_tensors_bitwise():
    shp = synth.LayerShape(M=2, H=512, E=12, K=3, I=64, Is=64)
    t = _layer64(shp, 4)
    full = oracle.moe_layer(t["x"], t["wr"], t["w13"], t["w2"], t["wsgu"], t["wsd"], K=3)
    fetched = oracle.moe_layer_fetch(t["x"], t["wr"], lambda ids: (t["w13"][ids], t["w2"][ids]),
                                     t["wsgu"], t["wsd"], K=3)
    np.testing.assert_array_equal(full["expert_ids"], fetched["expert_ids"])
    np.testing.assert_array_equal(full["y"], fetched["y"])


def test_thread_count_does_not_change_bits():
    shp = synth.LayerShape(M=2, H=1024, E=16, K=4, I=128, Is=64)
    t = _layer64(shp, 2)
    a = oracle.moe_layer(t["x"], t["wr"], t["w13"], t["w2"], t["wsgu"], t["wsd"], K=4, nthreads=1)
    b = oracle.moe_layer(t["x"], t["wr"], t["w13"], t["w2"], t["wsgu"], t["wsd"], K=4, nthreads=4)
    for k in ("expert_ids", "weights", "y", "logits", "margin"):
        np.testing.assert_array_equal(a[k], b[k])


def test_tokens_are_routed_independently():
    shp = synth.LayerShape(M=3, H=512, E=16, K=4, I=64, Is=0)
    t = _layer64(shp, 6)
    allm = oracle.moe_layer(t["x"], t["wr"], t["w13"], t["w2"], K=4)
    for m in range(3):
        one = oracle.moe_layer(t["x"][m:m + 1], t["wr"], t["w13"], t["w2"], K=4)
        np.testing.assert_array_equal(one["y"][0], allm["y"][m])
        np.testing.assert_array_equal(one["expert_ids"][0], allm["expert_ids"][m])


# ---- routing weights of a given selection (used where the selection has ties
# within rounding: BI-V100 worklog, part 8 -- the routing step is top-k + softmax)

def test_route_weights_two_experts_are_logistic():
    # renormalised weights of two experts depend only on their logit gap:
    # w_i = 1 / (1 + exp(L_j - L_i))
    lg = np.array([0.25, -1.5, 2.0, 0.75, -0.5])
    w = oracle.route_weights(lg, np.array([3, 1]), True)
    assert w[0] == pytest.approx(1.0 / (1.0 + math.exp(-1.5 - 0.75)), rel=1e-14)
    assert w[1] == pytest.approx(1.0 / (1.0 + math.exp(0.75 + 1.5)), rel=1e-14)


def test_route_weights_uniform_logits():
    E, K = 12, 5
    lg = np.full(E, 0.3)
    ids = np.array([7, 0, 11, 2, 5])
    np.testing.assert_allclose(oracle.route_weights(lg, ids, True), np.full(K, 1.0 / K), rtol=1e-15)
    np.testing.assert_allclose(oracle.route_weights(lg, ids, False), np.full(K, 1.0 / E), rtol=1e-15)


def test_route_weights_follow_the_ids_order():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal(32)
    ids = np.array([4, 17, 9, 30])
    w = oracle.route_weights(lg, ids, False)
    perm = np.array([2, 0, 3, 1])
    np.testing.assert_array_equal(oracle.route_weights(lg, ids[perm], False), w[perm])
    # unnormalised weights of every expert are the full softmax (sum 1, ratios exp(dL))
    full = oracle.route_weights(lg, np.arange(32), False)
    assert full.sum() == pytest.approx(1.0, abs=1e-14)
    assert full[4] / full[17] == pytest.approx(math.exp(lg[4] - lg[17]), rel=1e-13)


def test_route_weights_of_the_top_k_match_topk_softmax():
    rng = np.random.default_rng(6)
    lg = rng.standard_normal((3, 64))
    for renorm in (True, False):
        ids, w, _ = oracle.topk_softmax(lg, 6, renorm)
        np.testing.assert_allclose(oracle.route_weights(lg, ids, renorm), w, rtol=1e-14)


def test_route_weights_reject_bad_ids():
    with pytest.raises(ValueError):
        oracle.route_weights(np.zeros(4), np.array([0, 4]), True)
    with pytest.raises(ValueError):
        oracle.route_weights(np.zeros(4), np.array([-1, 2]), True)
