"""moe_layer_decode_noalloc (the library's static device buffer as the
workspace) against moe_layer_decode with a workspace of its own: the same bits
for routing outputs and y, on consecutive calls (the buffer keeps the previous
call's contents), the second smaller than the first; sizes beyond the buffer
are refused."""
import pytest
import torch

import routed_expert_gemv_amd as moe
from routed_expert_gemv_amd import _lib, synth
from tests import cases

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(sh, seed):
    t = cases.draw_case(sh, seed, DEV)
    ref = moe.moe_layer_decode(t["x"], t["wr"], t["w13"], t["w2"], t["wsgu"], t["wsd"], sh.K,
                               sh.renormalize)
    got = moe.moe_layer_decode_noalloc(t["x"], t["wr"], t["w13"], t["w2"], t["wsgu"], t["wsd"],
                                       sh.K, sh.renormalize)
    torch.cuda.synchronize()
    return t, ref, got


def _same(ref, got, where):
    for name, a, b in zip(("y", "ids", "weights", "logits"), ref, got):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b), \
            "%s differs: %s" % (name, where)


@pytest.mark.parametrize("first,second", [
    ("batch8_e256_k8_i512", "full_e256_k8_i512"),      # 8 tokens, then 1
    ("full_e256_k8_i512", "tiny_e16_k4_i128"),         # full width, then the tiny layer
    ("batch4_e256_k8_i512", "tp4_shard_e256_k8_i128"),
])
def test_noalloc_equals_layer_decode(first, second):
    print("no-alloc", first, "then", second, flush=True)
    for name, seed in ((first, 31), (second, 32)):
        sh = synth.SHAPES[name]
        t, ref, got = _both(sh, seed)
        _same(ref, got, name)
        if sh.M == 1:
            oref = cases.oracle_reference(t, sh, nthreads=8)
            cases.check_y(got[0], oref["y"], "no-alloc " + name)


def test_noalloc_refuses_sizes_beyond_its_buffer():
    L = _lib.lib()
    # M = 8, K = 16, I = 2048 needs over 1 MiB of workspace: refused before any launch
    assert L.moe_layer_decode_noalloc(1, 1, 1, 1, None, None, 8, 2048, 1024, 2048, 16, 0, 1,
                                      1, 1, 1, 1, None) == -6
    sh = synth.LayerShape(M=8, H=2048, E=16, K=16, I=2048, Is=0)
    t = synth.draw_layer(sh, 0, DEV)
    with pytest.raises(moe.MoeError) as err:
        moe.moe_layer_decode_noalloc(t["x"], t["wr"], t["w13"], t["w2"], None, None, sh.K)
    assert err.value.status == -6
