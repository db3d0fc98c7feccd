"""HIP path vs the fp64 oracle, through the C ABI, on seeded synthetic layers.

Rules (tests/cases.py): expert ids identical and in order; logits and routing
weights within the bounds derived from the fp32 arithmetic; fp16 outputs
within relative L2 2e-3 and max-abs 2e-2.  Bitwise checks cover run-to-run
determinism, direct indexing vs gather-then-GEMV, expert relabelling, W2
scaling and graph replay vs eager execution.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import routed_expert_gemv_amd as moe
from routed_expert_gemv_amd import synth
from routed_expert_gemv_amd.stack import DecodeLayer, DecodeStack
from tests import cases

pytestmark = pytest.mark.gpu
DEV = "cuda"
SILU1_F16 = 0.73095703125        # fp16(silu(1)), silu(1) = 0.7310585786...
TWO_SILU1_F16 = 1.4619140625     # fp16(2 silu(1))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_layer(t, shape, fused=True):
    layer = DecodeLayer(t, shape, fused=fused)
    layer.forward()
    torch.cuda.synchronize()
    return layer


def parity(shape, seed, tag=""):
    """Both paths (three entry points; moe_layer_decode) against the oracle."""
    say("parity", tag, shape, "seed", seed)
    t = cases.draw_case(shape, seed, DEV)
    ref = cases.oracle_reference(t, shape, nthreads=8)
    for fused in (False, True):
        layer = run_layer(t, shape, fused)
        where = "%s seed %d fused=%s" % (tag, seed, fused)
        cases.check_route(layer.topk_ids, layer.topk_w, layer.logits, ref, t, shape, where)
        rel, mx = cases.check_y(layer.y, ref["y"], where)
        say("  ok fused=%s rel-L2 %.3g max-abs %.3g (x attempt %d)" % (fused, rel, mx, t["attempt"]))
    return t, layer, ref


# ------------------------------------------------------------------ closed forms
def test_wave_sum_of_ones_is_64():
    say("wave_sum ones")
    v = torch.ones(64, dtype=torch.float32, device=DEV)
    assert moe.moe_dbg_wave_sum(v).item() == 64.0


def test_wave_sum_integers_exact():
    g = torch.Generator(device="cpu").manual_seed(5)
    v = torch.randint(-1000, 1000, (64,), generator=g).float()
    got = moe.moe_dbg_wave_sum(v.to(DEV)).item()
    assert got == float(v.double().sum())


@pytest.mark.parametrize("I", [128, 512])
def test_w2_unit_dot_is_128_page_value(I):
    # all-ones activations and unit W2 weights over an I-wide dot give I * sum(w)
    say("w2 unit dot I=%d" % I)
    E, K, H = 32, 8, 2048
    g = torch.Generator(device="cpu").manual_seed(1)
    ids = torch.randperm(E, generator=g)[:K].to(torch.int32).reshape(1, K).to(DEV)
    w = torch.softmax(torch.randn(1, K, generator=g), -1).to(DEV)
    act = torch.ones((1, K, I), dtype=torch.float32, device=DEV)
    w2 = torch.ones((E, H, I), dtype=torch.float16, device=DEV)
    y = moe.moe_dbg_w2_combine(act, w2, ids, w)
    torch.cuda.synchronize()
    assert torch.all(y.float() == float(I)), y.float().unique()


@pytest.mark.parametrize("with_shared", [False, True])
def test_closed_form_layer_is_silu1(with_shared):
    say("closed form silu(1) shared=%s" % with_shared)
    sh = synth.LayerShape(M=1, H=2048, E=16, K=4, I=128, Is=128 if with_shared else 0)
    t = synth.draw_layer(sh, 9, DEV)  # random router
    t["x"] = torch.ones_like(t["x"])
    t["w13"] = torch.full_like(t["w13"], 2.0 ** -11)
    t["w2"] = torch.full_like(t["w2"], 1.0 / sh.I)
    if with_shared:
        t["wsgu"] = torch.full_like(t["wsgu"], 2.0 ** -11)
        t["wsd"] = torch.full_like(t["wsd"], 1.0 / sh.Is)
    layer = run_layer(t, sh)
    want = TWO_SILU1_F16 if with_shared else SILU1_F16
    assert torch.all(layer.y.float() == want), layer.y.float().unique()


def test_dot2_keeps_fp16_subnormals_exact():
    # router rows of fp16 subnormals (k * 2^-24) against x = 1: every product and
    # partial sum is exact in fp32, so the logits must equal the fp64 sums exactly
    E, H = 8, 2048
    k = (torch.arange(E * H, dtype=torch.float64).reshape(E, H) % 7) - 3
    wr = (k * 2.0 ** -24).to(torch.float16)
    assert torch.equal(wr.double(), k * 2.0 ** -24)  # representable (subnormal) fp16
    x = torch.ones((1, H), dtype=torch.float16)
    _, _, lg = moe.moe_route(x.to(DEV), wr.to(DEV), 2)
    torch.cuda.synchronize()
    assert torch.equal(lg.double().cpu(), (wr.double() @ x.double().T).T)


# ------------------------------------------------------------------ parity
@pytest.mark.parametrize("name,seeds", [
    ("tiny_e16_k4_i128", [0, 1, 2]),
    ("tp4_shard_e256_k8_i128", [0, 1]),
    ("full_e256_k8_i512", [0, 1]),
    ("batch2_e256_k8_i512", [0, 1, 2]),
    ("batch4_e256_k8_i512", [0, 1, 2]),
    ("batch8_e256_k8_i512", [0, 1, 2]),
])
def test_layer_parity(name, seeds):
    for s in seeds:
        parity(synth.SHAPES[name], s, name)


def test_staged_down_kernel_at_64k_lds():
    """M=4, K=8, I=512: the staged down kernel holds 64 KiB of activations in
    dynamic LDS next to its static arrays, above the default 64 KiB limit; the
    calls must succeed (any failed launch status raises) and match the oracle."""
    parity(synth.SHAPES["batch4_e256_k8_i512"], 7, "staged 64 KiB")


@pytest.mark.parametrize("shape", [
    synth.LayerShape(M=3, H=2048, E=64, K=8, I=256, Is=256),          # ragged token count
    synth.LayerShape(M=5, H=1024, E=32, K=6, I=128, Is=0),            # ragged M and K
    synth.LayerShape(M=7, H=512, E=16, K=3, I=64, Is=64),
    synth.LayerShape(M=1, H=2048, E=16, K=1, I=128, Is=128),          # K = 1: dense SwiGLU
    synth.LayerShape(M=2, H=2048, E=16, K=16, I=128, Is=0),           # K = E: every expert
    synth.LayerShape(M=2, H=2048, E=16, K=1, I=128, Is=128),          # K = 1 at M > 1
    synth.LayerShape(M=4, H=1024, E=8, K=8, I=64, Is=64),             # K = E at M = 4
    synth.LayerShape(M=8, H=512, E=1024, K=16, I=64, Is=0),           # largest E, K, M
    synth.LayerShape(M=2, H=2048, E=8, K=2, I=2048, Is=2048),         # largest I
    synth.LayerShape(M=4, H=4096, E=16, K=4, I=1024, Is=512),         # largest H
    synth.LayerShape(M=4, H=4096, E=256, K=16, I=2048, Is=2048),      # largest H, K, I together
    synth.LayerShape(M=2, H=2048, E=64, K=8, I=512, Is=0, renormalize=False),
], ids=lambda s: "M%d_H%d_E%d_K%d_I%d_Is%d_r%d" % (s.M, s.H, s.E, s.K, s.I, s.Is, s.renormalize))
def test_edge_shapes(shape):
    parity(shape, 3, "edge")


@pytest.mark.parametrize("shape", cases.WIDE_SHAPES,
                         ids=lambda s: "M%d_H%d_E%d_K%d_I%d_Is%d" % (s.M, s.H, s.E, s.K, s.I, s.Is))
def test_widths_off_the_powers_of_two(shape):
    parity(shape, 4, "wide")


def test_shared_expert_alone():
    sh = synth.SHAPES["full_e256_k8_i512"]
    say("shared expert alone", sh)
    t = synth.draw_layer(sh, 2, DEV)
    s = moe.shared_expert(t["x"], t["wsgu"], t["wsd"])
    torch.cuda.synchronize()
    ref = oracle.shared_expert(cases.host64(t["x"]), cases.host64(t["wsgu"]), cases.host64(t["wsd"]))
    err = np.linalg.norm(s.double().cpu().numpy() - ref) / np.linalg.norm(ref)
    assert err < 1e-5, err


def test_w13_stage_matches_oracle():
    sh = synth.SHAPES["full_e256_k8_i512"]
    say("w13 stage", sh)
    t = cases.draw_case(sh, 0, DEV)
    ids, _, _ = moe.moe_route(t["x"], t["wr"], sh.K)
    act = moe.moe_dbg_w13_silu(t["x"], t["w13"], ids)
    torch.cuda.synchronize()
    x64 = cases.host64(t["x"])[0]
    for k, e in enumerate(ids[0].cpu().tolist()):
        ref = oracle.expert_activated(x64, cases.host64(t["w13"][e]), nthreads=8)
        err = np.linalg.norm(act[0, k].double().cpu().numpy() - ref) / np.linalg.norm(ref)
        assert err < 1e-5, (k, e, err)


@pytest.mark.parametrize("M", [2, 4, 8])
def test_uniform_router_ties_to_lowest_ids(M):
    # every logit 0: each token takes experts 0..K-1 in id order; the layer's
    # token masks and slots (found from each token's order at M <= 4) place
    # every activation where the separate calls' group table does
    sh = synth.LayerShape(M=M, H=2048, E=256, K=8, I=128, Is=0)
    t = synth.draw_layer(sh, 1, DEV)
    t["wr"].zero_()
    layer = run_layer(t, sh)
    assert layer.topk_ids.cpu().tolist() == [list(range(8))] * M
    assert torch.all(layer.topk_w == 0.125)
    sep = run_layer(t, sh, fused=False)
    assert torch.equal(layer.y, sep.y)


def test_same_tokens_share_every_expert():
    # identical tokens: |U| = K, every expert's rows read once for all tokens
    sh = synth.LayerShape(M=4, H=2048, E=256, K=8, I=512, Is=512)
    t = cases.draw_case(sh, 4, DEV)
    t["x"] = t["x"][:1].expand(4, -1).contiguous()
    layer = run_layer(t, sh)
    ref = cases.oracle_reference(t, sh, nthreads=8)
    cases.check_route(layer.topk_ids, layer.topk_w, layer.logits, ref, t, sh, "shared tokens")
    cases.check_y(layer.y, ref["y"], "shared tokens")
    assert torch.equal(layer.y[0], layer.y[3])


# ------------------------------------------------------------------ bitwise invariants
def test_run_to_run_bitwise():
    sh = synth.SHAPES["full_e256_k8_i512"]
    t = cases.draw_case(sh, 5, DEV)
    layer = DecodeLayer(t, sh)
    outs = []
    for _ in range(3):
        layer.forward()
        torch.cuda.synchronize()
        outs.append(layer.y.clone())
    assert all(torch.equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("name", ["full_e256_k8_i512", "batch4_e256_k8_i512"])
def test_direct_indexing_equals_gather_then_gemv_bitwise(name):
    sh = synth.SHAPES[name]
    say("gather vs direct", name)
    t = cases.draw_case(sh, 6, DEV)
    ids, w, _ = moe.moe_route(t["x"], t["wr"], sh.K)
    s = moe.shared_expert(t["x"], t["wsgu"], t["wsd"])
    y_direct = moe.moe_decode_fused(t["x"], t["w13"], t["w2"], ids, w, shared_in=s)
    # gathered copies of the distinct experts, in order of first appearance
    flat = ids.flatten().cpu().tolist()
    uniq = list(dict.fromkeys(flat))
    pos = {e: i for i, e in enumerate(uniq)}
    idx = torch.tensor(uniq, device=DEV)
    w13g = t["w13"].index_select(0, idx).contiguous()
    w2g = t["w2"].index_select(0, idx).contiguous()
    ids_g = torch.tensor([pos[e] for e in flat], dtype=torch.int32, device=DEV).reshape(ids.shape)
    y_gather = moe.moe_decode_fused(t["x"], w13g, w2g, ids_g, w, shared_in=s)
    torch.cuda.synchronize()
    assert torch.equal(y_direct, y_gather)


def test_expert_relabelling_bitwise():
    sh = synth.SHAPES["tp4_shard_e256_k8_i128"]
    t = cases.draw_case(sh, 7, DEV)
    a = run_layer(t, sh)
    ya, ida, wa = a.y.clone(), a.topk_ids.clone(), a.topk_w.clone()
    perm = torch.randperm(sh.E, generator=torch.Generator().manual_seed(3)).to(DEV)
    tp = dict(t)
    tp["wr"] = t["wr"][perm].contiguous()
    tp["w13"] = t["w13"][perm].contiguous()
    tp["w2"] = t["w2"][perm].contiguous()
    b = run_layer(tp, sh)
    assert torch.equal(perm[b.topk_ids.long()].int(), ida)
    assert torch.equal(b.topk_w, wa)
    assert torch.equal(b.y, ya)


def test_scaling_w2_doubles_output_bitwise():
    sh = synth.LayerShape(M=1, H=2048, E=256, K=8, I=512, Is=0)
    t = cases.draw_case(sh, 8, DEV)
    y1 = run_layer(t, sh).y.clone()
    t2 = dict(t)
    t2["w2"] = t["w2"] * 2
    y2 = run_layer(t2, sh).y
    # the fp32 sum doubles exactly; rounding to fp16 commutes with doubling only for
    # normal fp16 results (subnormals sit on a fixed 2^-24 grid)
    normal = y1.float().abs() >= 2.0 ** -14
    assert torch.equal(y2[normal], (y1 * 2)[normal])
    assert torch.all((y2.float() - 2 * y1.float()).abs()[~normal] <= 2.0 ** -23)


def test_graph_replay_equals_eager_bitwise():
    sh = synth.SHAPES["full_e256_k8_i512"]
    layers = [DecodeLayer(cases.draw_case(sh, s, DEV), sh) for s in (0, 1)]
    st = DecodeStack(layers)
    st.forward_eager()
    torch.cuda.synchronize()
    eager = [l.y.clone() for l in layers]
    st.capture()
    for rep in range(3):
        for l in layers:
            l.y.zero_()
        torch.cuda.synchronize()
        st.replay()
        torch.cuda.synchronize()
        for l, e in zip(layers, eager):
            assert torch.equal(l.y, e), "replay %d differs" % rep
        st.forward_eager()  # eager work between replays
        torch.cuda.synchronize()


def test_empty_call_and_errors_on_device():
    sh = synth.SHAPES["tiny_e16_k4_i128"]
    t = synth.draw_layer(sh, 0, DEV)
    x0 = t["x"][:0]
    ids, w, lg = moe.moe_route(x0, t["wr"], sh.K)
    assert ids.shape == (0, sh.K)
    with pytest.raises(moe.MoeError):
        moe.moe_route(t["x"], t["wr"], 17)          # K > 16
    with pytest.raises(moe.MoeError):
        moe.moe_decode_fused(t["x"], t["w13"], t["w2"], torch.zeros((1, 4), dtype=torch.int32,
                             device=DEV), torch.zeros((1, 4), device=DEV),
                             ws=torch.empty(16, dtype=torch.uint8, device=DEV))


def test_copy_probe_copies():
    """The counter-calibration copy kernel moves exactly its bytes (ragged tail included)."""
    src = torch.randn(3 * 2048 * 8 + 40, device=DEV).half()
    dst = torch.zeros_like(src)
    moe.moe_probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
