"""The C-ABI library without a GPU: it loads, exports every function that
include/moe_decode.h and include/moe_prefill.h declare, and rejects bad
arguments on the host before anything is enqueued (no call here reaches a
kernel launch)."""
import ctypes as C
import os
import re

import numpy as np
import pytest
import torch

from routed_expert_gemv_amd import _lib, build, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_decode.h")
HEADERS = [HEADER, os.path.join(ROOT, "include", "moe_prefill.h")]

FAKE = 0x10000       # aligned, never dereferenced: validation fails first
FAKE_ODD = 0x10002   # 2-byte aligned only


def declared_functions():
    names = []
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names += re.findall(r"^(?:moe_status|int|size_t|const char \*)\s*(\w+)\s*\(", text,
                            flags=re.M)
    return names


def test_library_builds_and_loads():
    assert os.path.exists(build.LIB) or build.build(force=True)
    L = _lib.lib()
    assert L.moe_abi_version() == 5


def test_library_matches_the_sources():
    L = _lib.lib()
    assert L.moe_build_id().decode() == build.source_id()


def test_stale_library_is_refused(tmp_path, monkeypatch):
    """A library built from other sources than the tree holds is never loaded:
    with one source edited (a copy with an extra comment stands in for it),
    lib() raises instead of handing out the old binary."""
    src = build.SOURCES[0]
    edited = tmp_path / os.path.basename(src)
    edited.write_bytes(open(src, "rb").read() + b"\n// edited after the build\n")
    monkeypatch.setattr(build, "SOURCES", [str(edited)] + build.SOURCES[1:])
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(_lib.StaleLibraryError):
        _lib.lib()


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) >= {"moe_route", "shared_expert", "moe_decode_fused", "moe_workspace_bytes",
                          "moe_layer_prefill", "moe_prefill_workspace_bytes"}
    L = C.CDLL(build.LIB)
    for n in names:
        assert hasattr(L, n), "declared symbol %s is not exported" % n
    assert set(names) == set(_lib.EXPORTED)
    # the Python binding carries the same names
    import routed_expert_gemv_amd as m
    assert [n for n in names if not hasattr(m, n)] == []


def test_abi_version_matches_header():
    m = re.search(r"#define MOE_ABI_VERSION (\d+)", open(HEADER).read())
    assert int(m.group(1)) == _lib.lib().moe_abi_version()


def test_status_strings():
    L = _lib.lib()
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = L.moe_status_str(code).decode()
        assert s and s != "unknown status"
    assert L.moe_status_str(-99).decode() == "unknown status"


def test_workspace_bytes():
    L = _lib.lib()
    n = L.moe_workspace_bytes(1, 2048, 256, 512, 8, 512)
    assert n >= 8 * 512 * 4 and n % 256 == 0
    assert L.moe_workspace_bytes(8, 2048, 256, 512, 8, 512) >= 8 * 8 * 512 * 4
    assert L.moe_workspace_bytes(9, 2048, 256, 512, 8, 512) == 0      # M > 8
    assert L.moe_workspace_bytes(1, 2000, 256, 512, 8, 512) == 0      # H
    assert L.moe_workspace_bytes(1, 2048, 256, 500, 8, 512) == 0      # I
    assert L.moe_workspace_bytes(1, 2048, 4, 512, 8, 0) == 0          # K > E
    assert L.moe_workspace_bytes(8, 4096, 256, 512, 8, 0) == 0        # H = 4096 needs M <= 4


# The decode boundary: H a multiple of 512 up to 4096 (M <= 4 above 2048);
# I and Is multiples of 64 up to 2048.
H_ACCEPT = list(range(512, 4097, 512))
H_REJECT = [0, 256, 768, 1000, 2000, 4608, 8192]
I_ACCEPT = list(range(64, 2049, 64))
I_REJECT = [0, 32, 96, 100, 200, 992, 2112, 4096]


def test_decode_boundary_accept_and_reject_sets():
    """Every decode entry point takes exactly the widths above.  An accepted
    shape passes validation and stops at the null x (-1); a rejected one
    stops at the shape check (-2); neither reaches a launch."""
    L = _lib.lib()

    def route(M=1, H=2048):
        return L.moe_route(None, FAKE, M, H, 256, 8, 1, FAKE, FAKE, FAKE, None)

    def shared(M=1, H=2048, Is=512):
        return L.shared_expert(None, FAKE, FAKE, M, H, Is, FAKE, FAKE, 1 << 30, None)

    def fused(M=1, H=2048, I=512):
        return L.moe_decode_fused(None, FAKE, FAKE, FAKE, FAKE, None, M, H, 256, I, 8, FAKE, FAKE,
                                  1 << 30, None)

    def layer(M=1, H=2048, I=512, Is=512):
        gu = FAKE if Is else None
        return L.moe_layer_decode(None, FAKE, FAKE, FAKE, gu, gu, M, H, 256, I, 8, Is, 1, FAKE,
                                  FAKE, FAKE, FAKE, FAKE, 1 << 30, None)

    def ws(M=1, H=2048, I=512, Is=512):
        return L.moe_workspace_bytes(M, H, 256, I, 8, Is)

    for H in H_ACCEPT:
        for M in (1, 4):
            assert route(M, H) == shared(M, H) == fused(M, H) == layer(M, H) == -1, (M, H)
            assert ws(M, H) > 0
        m5 = -1 if H <= 2048 else -2       # 5..8 tokens only up to H = 2048
        assert route(5, H) == shared(5, H) == fused(5, H) == layer(5, H) == m5, H
        assert (ws(8, H) > 0) == (H <= 2048)
    for H in H_REJECT:
        assert route(1, H) == shared(1, H) == fused(1, H) == layer(1, H) == -2, H
        assert ws(1, H) == 0
    for I in I_ACCEPT:
        assert fused(I=I) == shared(Is=I) == layer(I=I, Is=I) == -1, I
        assert layer(I=I, Is=0) == layer(I=512, Is=I) == layer(M=3, I=I, Is=192) == -1, I
        assert ws(I=I, Is=I) > 0 and ws(M=8, I=I, Is=0) > 0
    for I in I_REJECT:
        assert fused(I=I) == layer(I=I, Is=512) == -2, I
        assert ws(I=I) == 0
        if I:  # Is = 0 means "no shared expert" where the entry point allows it
            assert shared(Is=I) == layer(I=512, Is=I) == -2, I


def test_lane_map_rule():
    """The down-projection lane mapping of every accepted width: exact where
    n/8 = LPR*CPL with LPR in {8, 16, 32, 64} and CPL <= 4 (the largest such
    LPR), else 64 lanes and ceil(n/512) chunks with the steps past the row
    padded; and the widths named in the header."""
    L = _lib.lib()

    def lm(n):
        a, b, c = C.c_int(), C.c_int(), C.c_int()
        st = L.moe_dbg_lane_map(n, C.byref(a), C.byref(b), C.byref(c))
        return st, a.value, b.value, c.value

    for n in I_ACCEPT:
        st, lpr, cpl, pad = lm(n)
        assert st == 0
        chunks = n // 8
        exact = [l for l in (64, 32, 16, 8) if chunks % l == 0 and chunks // l <= 4]
        if exact:
            assert (lpr, cpl, pad) == (exact[0], chunks // exact[0], 0), n
        else:
            assert (lpr, cpl, pad) == (64, -(-chunks // 64), 1), n
        assert lpr * cpl * 8 >= n and lpr * (cpl - 1) * 8 < n   # no wholly empty step
    assert lm(768)[1:] == (32, 3, 0) and lm(192)[1:] == (8, 3, 0) and lm(384)[1:] == (16, 3, 0)
    assert lm(512)[1:] == (64, 1, 0) and lm(2048)[1:] == (64, 4, 0) and lm(128)[1:] == (16, 1, 0)
    assert lm(320)[1:] == (64, 1, 1) and lm(1536)[1:] == (64, 3, 0) and lm(1984)[1:] == (64, 4, 1)
    for n in I_REJECT:
        assert lm(n)[0] == -2
    assert L.moe_dbg_lane_map(512, None, None, None) == -1


def test_route_validation():
    L = _lib.lib()
    ok = dict(M=1, H=2048, E=256, K=8)

    def call(x=FAKE, wr=FAKE, ids=FAKE, w=FAKE, lg=FAKE, **kw):
        a = dict(ok, **kw)
        return L.moe_route(x, wr, a["M"], a["H"], a["E"], a["K"], 1, ids, w, lg, None)

    assert call(x=None) == -1
    assert call(lg=None) == -1
    assert call(H=2000) == -2
    assert call(M=9) == -2
    assert call(M=-1) == -2
    assert call(E=0) == -2
    assert call(K=17, E=256) == -2
    assert call(K=9, E=8) == -2
    assert call(E=1025) == -2
    assert call(x=FAKE_ODD) == -3
    assert call(M=0) == 0          # empty call: nothing enqueued


def test_shared_expert_validation():
    L = _lib.lib()

    def call(x=FAKE, gu=FAKE, d=FAKE, s=FAKE, ws=FAKE, M=1, H=2048, Is=512, n=1 << 20):
        return L.shared_expert(x, gu, d, M, H, Is, s, ws, n, None)

    assert call(d=None) == -1
    assert call(Is=500) == -2
    assert call(H=4096, M=8) == -2
    assert call(gu=FAKE_ODD) == -3
    assert call(ws=FAKE + 16) == -3
    assert call(n=100) == -4
    assert call(M=0) == 0


def test_fused_validation():
    L = _lib.lib()
    need = L.moe_workspace_bytes(2, 2048, 256, 512, 8, 0)

    def call(x=FAKE, w13=FAKE, w2=FAKE, ids=FAKE, tw=FAKE, sh=None, y=FAKE, ws=FAKE,
             M=2, H=2048, E=256, I=512, K=8, n=need):
        return L.moe_decode_fused(x, w13, w2, ids, tw, sh, M, H, E, I, K, y, ws, n, None)

    assert call(w2=None) == -1
    assert call(y=None) == -1
    assert call(I=96) == -2
    assert call(K=0) == -2
    assert call(w13=FAKE_ODD) == -3
    assert call(sh=FAKE + 2) == -3
    assert call(n=need - 1) == -4
    assert call(M=0) == 0


def test_debug_probe_validation():
    L = _lib.lib()
    assert L.moe_probe_copy(None, FAKE, 16, None) == -1
    assert L.moe_probe_copy(FAKE, FAKE + 8, 16, None) == -3
    assert L.moe_probe_copy(FAKE, FAKE, 24, None) == -3
    assert L.moe_dbg_wave_sum(None, FAKE, None) == -1
    assert L.moe_dbg_wave_sum(FAKE + 1, FAKE, None) == -3
    assert L.moe_dbg_w13_silu(FAKE, FAKE, FAKE, 1, 2048, 256, 512, 8, None, FAKE, 1 << 20,
                              None) == -1
    assert L.moe_dbg_w2_combine(FAKE, FAKE, FAKE, FAKE, None, 1, 2048, 256, 512, 8, FAKE, FAKE,
                                16, None) == -4


def test_python_binding_rejects_host_tensors():
    import routed_expert_gemv_amd as m
    x = torch.zeros(1, 2048, dtype=torch.float16)
    with pytest.raises(ValueError):
        m.moe_route(x, torch.zeros(16, 2048, dtype=torch.float16), 4)


def test_generator_is_seeded_and_ordered():
    sh = synth.LayerShape(M=2, H=512, E=4, K=2, I=64, Is=64)
    a = synth.draw_layer(sh, 3, "cpu")
    b = synth.draw_layer(sh, 3, "cpu")
    c = synth.draw_layer(sh, 4, "cpu")
    for k in ("wr", "w13", "w2", "wsgu", "wsd", "x"):
        assert torch.equal(a[k], b[k])
        assert not torch.equal(a[k], c[k])
        assert a[k].dtype == torch.float16 and a[k].is_contiguous()
    assert a["w13"].shape == (4, 128, 512) and a["w2"].shape == (4, 512, 64)
    assert a["wsgu"].shape == (128, 512) and a["wsd"].shape == (512, 64)
    # weights ~ N(0, 0.02), x ~ N(0, 1)
    assert 0.015 < a["w13"].float().std().item() < 0.025
    assert 0.8 < a["x"].float().std().item() < 1.2
    x1 = synth.redraw_x(sh, 3, 1, "cpu")
    assert x1.shape == (2, 512) and not torch.equal(x1, a["x"])
    assert torch.equal(x1, synth.redraw_x(sh, 3, 1, "cpu"))


def test_margin_guard_redraws_until_separated():
    from tests import cases
    sh = synth.SHAPES["tiny_e16_k4_i128"]
    t = cases.draw_case(sh, 0, "cpu")
    import oracle
    lg = oracle.router_logits(cases.host64(t["x"]), cases.host64(t["wr"]))
    _, _, margin = oracle.topk_softmax(lg, sh.K)
    bound = cases.logit_bound(t, sh).max(axis=-1)
    # the accepted margin exceeds twice the worst-case fp32 logit error of every token
    assert np.all(margin > 2 * bound)
    assert np.all(margin > cases.required_margin(t, sh))


def test_layer_launch_counts():
    L = _lib.lib()
    assert L.moe_layer_launches(1, 2048, 256, 512, 8, 512) == 3    # M = 1: three launches
    assert L.moe_layer_launches(1, 2048, 256, 512, 8, 0) == 3
    assert L.moe_layer_launches(2, 2048, 256, 512, 8, 512) == 3    # up to 4 tokens: selection folded
    assert L.moe_layer_launches(4, 2048, 256, 512, 8, 512) == 3
    # K = 1 with narrow experts and a wide shared one: more shared down
    # blocks than token 0's workgroups take, so they get a launch of their own
    assert L.moe_layer_launches(2, 4096, 64, 64, 1, 2048) == 4
    assert L.moe_layer_launches(2, 2048, 16, 128, 1, 128) == 4     # 128 shared blocks, 16 of token 0
    assert L.moe_layer_launches(2, 2048, 16, 128, 4, 128) == 3     # 128 shared blocks, 64 of token 0
    assert L.moe_layer_launches(5, 2048, 256, 512, 8, 512) == 4    # 5..8 tokens: a selection launch
    assert L.moe_layer_launches(8, 2048, 256, 512, 8, 512) == 4
    assert L.moe_layer_launches(1, 2048, 16, 2048, 16, 0) == 4     # K*I above the LDS stage
    assert L.moe_layer_launches(0, 2048, 256, 512, 8, 512) == 0
    assert L.moe_layer_launches(9, 2048, 256, 512, 8, 512) == 0


def test_layer_stage_probe_validation():
    L = _lib.lib()

    def call(stage, M=1, H=2048):
        return L.moe_dbg_layer_stage(stage, FAKE, FAKE, FAKE, FAKE, None, None, M, H, 256, 512, 8,
                                     0, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)

    assert call(0) == -2 and call(7) == -2 and call(-1) == -2
    assert call(2, M=9) == -2          # stages 1..4 take the layer's sizes (M = 1..8)
    assert call(5, M=2) == -2          # not the single-launch path
    assert call(2, H=2000) == -2
    assert L.moe_dbg_layer_stage(2, None, FAKE, FAKE, FAKE, None, None, 1, 2048, 256, 512, 8, 0, 1,
                                 FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == -1


def test_noalloc_validation():
    """The entry point without a workspace refuses bad sizes, and sizes whose
    workspace exceeds its static buffer, before touching the device."""
    L = _lib.lib()

    def call(M=1, H=2048, E=256, I=512, K=8, Is=0, gu=None, d=None):
        return L.moe_layer_decode_noalloc(FAKE, FAKE, FAKE, FAKE, gu, d, M, H, E, I, K, Is, 1,
                                          FAKE, FAKE, FAKE, FAKE, None)

    assert call(H=2000) == -2 and call(M=9) == -2 and call(K=0) == -2
    assert call(M=8, E=1024, I=2048, K=16) == -6          # over 512 KiB of workspace
    assert call(M=8, I=2048, K=16, Is=2048, gu=FAKE, d=FAKE) == -6
    assert L.moe_status_str(-6).decode() != "unknown status"


def test_workspace_init_validation():
    L = _lib.lib()
    assert L.moe_workspace_init(None, 8192, None) == -1
    assert L.moe_workspace_init(FAKE_ODD, 8192, None) == -3
    assert L.moe_workspace_init(FAKE, 8191, None) == -4


def test_prefill_workspace_bytes():
    L = _lib.lib()
    T, H, E, I, K, Is = 2048, 2048, 256, 512, 8, 512
    n = L.moe_prefill_workspace_bytes(T, H, E, I, K, Is)
    # at least the down products [T*K, H] fp32 and both activations (fp16)
    assert n >= T * K * H * 4 + T * K * I * 2 + T * Is * 2 and n % 256 == 0
    assert L.moe_prefill_workspace_bytes(T, H, E, I, K, 0) < n
    assert L.moe_prefill_workspace_bytes(T + 1, H, E, I, K, Is) > n
    assert L.moe_prefill_workspace_bytes(0, H, E, I, K, Is) > 0          # T = 0: valid
    assert L.moe_prefill_workspace_bytes(65537, H, E, I, K, Is) == 0     # T too large
    assert L.moe_prefill_workspace_bytes(T, 2000, E, I, K, Is) == 0      # H % 64
    assert L.moe_prefill_workspace_bytes(T, H, E, 96, K, Is) == 0        # I % 64
    assert L.moe_prefill_workspace_bytes(T, H, E, I, K, 32) == 0         # Is % 64
    assert L.moe_prefill_workspace_bytes(T, H, 1025, I, K, Is) == 0      # E
    assert L.moe_prefill_workspace_bytes(T, H, 4, I, 8, Is) == 0         # K > E
    # routed activations [T*K, I] fp16 must stay under 4 GiB (32-bit row offsets)
    assert L.moe_prefill_workspace_bytes(65536, 1024, 256, 2048, 16, 0) == 0
    assert L.moe_prefill_workspace_bytes(65536, 1024, 256, 1024, 16, 0) > 0
    assert L.moe_prefill_workspace_bytes(T, 64, 16, 64, 4, 64) > 0       # smallest dims


def test_prefill_validation():
    L = _lib.lib()
    shape = dict(T=256, H=2048, E=256, I=512, K=8, Is=512)
    need = L.moe_prefill_workspace_bytes(*shape.values())

    def call(fn=L.moe_layer_prefill, pre=(), x=FAKE, wr=FAKE, w13=FAKE, w2=FAKE, gu=FAKE, d=FAKE,
             ids=FAKE, tw=FAKE, lg=FAKE, y=FAKE, ws=FAKE, n=need, **kw):
        a = dict(shape, **kw)
        return fn(*pre, x, wr, w13, w2, gu, d, a["T"], a["H"], a["E"], a["I"], a["K"], a["Is"], 1,
                  ids, tw, lg, y, ws, n, None)

    assert call(x=None) == -1
    assert call(y=None) == -1
    assert call(gu=None) == -1            # one of the shared pair missing
    assert call(T=-1) == -2
    assert call(T=65537) == -2
    assert call(H=2000) == -2
    assert call(I=96) == -2
    assert call(K=0) == -2
    assert call(E=1025) == -2
    assert call(Is=0) == -2               # shared weights given but Is = 0
    assert call(w13=FAKE_ODD) == -3
    assert call(ws=FAKE + 16) == -3
    assert call(y=FAKE + 4) == -3         # y is written 8 bytes at a time
    assert call(n=need - 1) == -4
    assert call(T=0) == 0                 # empty call: nothing enqueued
    # without a shared expert Is is ignored and the workspace is smaller
    small = L.moe_prefill_workspace_bytes(256, 2048, 256, 512, 8, 0)
    assert call(gu=None, d=None, Is=0, n=small - 1) == -4
    # the stage probe: stage 1..6 only, same validation
    assert call(fn=L.moe_dbg_prefill_stage, pre=(0,)) == -2
    assert call(fn=L.moe_dbg_prefill_stage, pre=(7,)) == -2
    assert call(fn=L.moe_dbg_prefill_stage, pre=(4,), x=None) == -1
