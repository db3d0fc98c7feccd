"""fp64 CPU oracle of the single-token routed-expert MoE decode layer.

TEST INFRASTRUCTURE ONLY.  The oracle is the checker that the HIP path is
compared against; only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it.  It shares no code with the HIP path (the
package ``routed_expert_gemv_amd``) and never imports it.

The arithmetic lives in ``moe_oracle.c`` (plain loops, fp64, no BLAS, no
fast-math); this module only marshals numpy arrays into it.  fp16 inputs are
widened to fp64 with numpy, which is exact.

Sources: the BI-V100 inference worklog ("如何在天垓 BI-V100 上优化大模型推理：
一份工作日志"), parts 2, 3, 8 and 10; the decode analysis report of 2026-07-14,
section on code-level profiling (MoE = gate / routing top-k / routed experts /
shared expert).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A prebuilt copy to load instead (used only by the mutation test, which builds
# deliberately broken copies of moe_oracle.c to show the pins catch them).
_LIB_OVERRIDE = os.environ.get("MOE_ORACLE_LIB_OVERRIDE")
_lock = threading.Lock()
_lib = None

_DP = C.POINTER(C.c_double)
_IP = C.POINTER(C.c_int32)


def build(force: bool = False) -> str:
    """Compile moe_oracle.c into liboracle.so (gcc -O2, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
               "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if _LIB_OVERRIDE:
                lib = C.CDLL(_LIB_OVERRIDE)
            else:
                build()
                lib = C.CDLL(_LIB)
            lib.oracle_abi_version.restype = C.c_int
            lib.oracle_max_threads.restype = C.c_int
            lib.oracle_router_logits.argtypes = [_DP, _DP, C.c_int, C.c_int, C.c_int, _DP]
            lib.oracle_topk_softmax.argtypes = [_DP, C.c_int, C.c_int, C.c_int, _IP, _DP, _DP]
            lib.oracle_topk_softmax.restype = C.c_int
            lib.oracle_route_weights.argtypes = [_DP, C.c_int, C.c_int, _IP, C.c_int, _DP]
            lib.oracle_route_weights.restype = C.c_int
            lib.oracle_expert_activated.argtypes = [_DP, _DP, C.c_int, C.c_int, C.c_int, _DP]
            lib.oracle_weighted_down.argtypes = [C.POINTER(_DP), _DP, _DP, C.c_int, C.c_int,
                                                 C.c_int, C.c_int, _DP]
            lib.oracle_shared_expert.argtypes = [_DP, _DP, _DP, C.c_int, C.c_int, C.c_int, _DP, _DP]
            lib.oracle_token_output.argtypes = [_DP, _DP, _DP, _DP, _DP, _DP, C.c_int, C.c_int,
                                                C.c_int, C.c_int, C.c_int, _DP, _DP]
            lib.oracle_moe_layer.argtypes = [_DP, _DP, _DP, _DP, _DP, _DP] + [C.c_int] * 8 + \
                [_IP, _DP, _DP, _DP, _DP]
            lib.oracle_moe_layer.restype = C.c_int
            _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch tensor on the host
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(_DP)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def router_logits(x, wr, nthreads: int = 1) -> np.ndarray:
    """logits[m, e] = sum_h wr[e, h] * x[m, h] (the router GEMV), fp64."""
    lib = _load()
    x = _f64(x)
    wr = _f64(wr)
    x2 = x.reshape(-1, x.shape[-1])
    E, H = wr.shape
    assert x2.shape[1] == H
    out = np.empty((x2.shape[0], E), dtype=np.float64)
    for m in range(x2.shape[0]):
        xm = np.ascontiguousarray(x2[m])
        row = np.empty(E, dtype=np.float64)
        lib.oracle_router_logits(_p(xm), _p(wr), H, E, nthreads, _p(row))
        out[m] = row
    return out.reshape(x.shape[:-1] + (E,))


def topk_softmax(logits, K: int, renormalize: bool = True):
    """Top-K selection (logit descending, lower id first on ties) + routing weights.

    Returns (expert_ids int32 [.., K], weights fp64 [.., K], margin fp64 [..]).
    """
    lib = _load()
    lg = _f64(logits)
    E = lg.shape[-1]
    l2 = lg.reshape(-1, E)
    ids = np.empty((l2.shape[0], K), dtype=np.int32)
    w = np.empty((l2.shape[0], K), dtype=np.float64)
    margin = np.empty(l2.shape[0], dtype=np.float64)
    for m in range(l2.shape[0]):
        row = np.ascontiguousarray(l2[m])
        idr = np.empty(K, dtype=np.int32)
        wr_ = np.empty(K, dtype=np.float64)
        mg = np.empty(1, dtype=np.float64)
        rc = lib.oracle_topk_softmax(_p(row), E, K, int(bool(renormalize)),
                                     idr.ctypes.data_as(_IP), _p(wr_), _p(mg))
        if rc != 0:
            raise ValueError("oracle_topk_softmax: bad sizes E=%d K=%d" % (E, K))
        ids[m], w[m], margin[m] = idr, wr_, mg[0]
    shp = lg.shape[:-1]
    return ids.reshape(shp + (K,)), w.reshape(shp + (K,)), margin.reshape(shp)


def route_weights(logits, ids, renormalize: bool = True) -> np.ndarray:
    """Routing weights of a given selection ids [.., K] under logits [.., E] (fp64)."""
    lib = _load()
    lg = _f64(logits)
    E = lg.shape[-1]
    l2 = lg.reshape(-1, E)
    idv = np.ascontiguousarray(ids, dtype=np.int32)
    K = idv.shape[-1]
    i2 = idv.reshape(-1, K)
    assert i2.shape[0] == l2.shape[0]
    w = np.empty((l2.shape[0], K), dtype=np.float64)
    for m in range(l2.shape[0]):
        row = np.ascontiguousarray(l2[m])
        idr = np.ascontiguousarray(i2[m])
        wr_ = np.empty(K, dtype=np.float64)
        rc = lib.oracle_route_weights(_p(row), E, K, idr.ctypes.data_as(_IP),
                                      int(bool(renormalize)), _p(wr_))
        if rc != 0:
            raise ValueError("oracle_route_weights: bad sizes or ids (E=%d K=%d)" % (E, K))
        w[m] = wr_
    return w.reshape(idv.shape)


def expert_activated(x, w13e, nthreads: int = 1) -> np.ndarray:
    """activated[j] = silu(gate_j) * up_j for one token and one expert's [2I, H] rows."""
    lib = _load()
    x = _f64(x).reshape(-1)
    w13e = _f64(w13e)
    twoI, H = w13e.shape
    I = twoI // 2
    out = np.empty(I, dtype=np.float64)
    lib.oracle_expert_activated(_p(x), _p(w13e), H, I, nthreads, _p(out))
    return out


def weighted_down(w2_list, activated, weights, nthreads: int = 1) -> np.ndarray:
    """out[h] = sum_k weights[k] * sum_j w2_list[k][h, j] * activated[k, j]."""
    lib = _load()
    mats = [_f64(w) for w in w2_list]
    act = _f64(activated)
    wts = _f64(weights).reshape(-1)
    K = len(mats)
    H, I = mats[0].shape
    assert act.shape == (K, I) and wts.shape == (K,)
    arr = (_DP * K)(*[_p(m) for m in mats])
    out = np.empty(H, dtype=np.float64)
    lib.oracle_weighted_down(arr, _p(act), _p(wts), H, I, K, nthreads, _p(out))
    return out


def shared_expert(x, wsgu, wsd, nthreads: int = 1) -> np.ndarray:
    """Shared-expert output s[m, h] (gate_up -> silu*mul -> down), fp64."""
    lib = _load()
    x = _f64(x)
    wsgu = _f64(wsgu)
    wsd = _f64(wsd)
    x2 = x.reshape(-1, x.shape[-1])
    H = x2.shape[1]
    Is = wsgu.shape[0] // 2
    out = np.empty((x2.shape[0], H), dtype=np.float64)
    scr = np.empty(Is, dtype=np.float64)
    for m in range(x2.shape[0]):
        xm = np.ascontiguousarray(x2[m])
        s = np.empty(H, dtype=np.float64)
        lib.oracle_shared_expert(_p(xm), _p(wsgu), _p(wsd), H, Is, nthreads, _p(scr), _p(s))
        out[m] = s
    return out.reshape(x.shape)


def token_output(x, w13sel, w2sel, weights, wsgu=None, wsd=None, nthreads: int = 1) -> np.ndarray:
    """y[h] for one token from the selected experts' slices (routing order) + shared expert."""
    lib = _load()
    x = _f64(x).reshape(-1)
    w13sel = _f64(w13sel)
    w2sel = _f64(w2sel)
    wts = _f64(weights).reshape(-1)
    K, twoI, H = w13sel.shape
    I = twoI // 2
    assert w2sel.shape == (K, H, I) and wts.shape == (K,)
    if wsgu is not None:
        wsgu = _f64(wsgu)
        wsd = _f64(wsd)
        Is = wsgu.shape[0] // 2
    else:
        Is = 0
    scr = np.empty(K * I + Is, dtype=np.float64)
    y = np.empty(H, dtype=np.float64)
    lib.oracle_token_output(_p(x), _p(w13sel), _p(w2sel), _p(wts), _p(wsgu), _p(wsd),
                            H, I, K, Is, nthreads, _p(scr), _p(y))
    return y


def moe_layer(x, wr, w13, w2, wsgu=None, wsd=None, *, K: int, renormalize: bool = True,
              nthreads: int = 1) -> dict:
    """Whole layer for M tokens with full expert tensors on the host (small configs)."""
    lib = _load()
    x = _f64(x)
    x2 = x.reshape(-1, x.shape[-1])
    wr = _f64(wr)
    w13 = _f64(w13)
    w2 = _f64(w2)
    M, H = x2.shape
    E, twoI, H2 = w13.shape
    I = twoI // 2
    assert H2 == H and wr.shape == (E, H) and w2.shape == (E, H, I)
    if wsgu is not None:
        wsgu = _f64(wsgu)
        wsd = _f64(wsd)
        Is = wsgu.shape[0] // 2
        assert wsgu.shape == (2 * Is, H) and wsd.shape == (H, Is)
    else:
        Is = 0
    ids = np.empty((M, K), dtype=np.int32)
    w = np.empty((M, K), dtype=np.float64)
    y = np.empty((M, H), dtype=np.float64)
    lg = np.empty((M, E), dtype=np.float64)
    mg = np.empty(M, dtype=np.float64)
    rc = lib.oracle_moe_layer(_p(x2), _p(wr), _p(w13), _p(w2), _p(wsgu), _p(wsd),
                              M, H, E, I, K, Is, int(bool(renormalize)), nthreads,
                              ids.ctypes.data_as(_IP), _p(w), _p(y), _p(lg), _p(mg))
    if rc != 0:
        raise ValueError("oracle_moe_layer failed (sizes M=%d H=%d E=%d I=%d K=%d)" % (M, H, E, I, K))
    return {"expert_ids": ids, "weights": w, "y": y, "logits": lg, "margin": mg}


def moe_layer_fetch(x, wr, fetch_experts, wsgu=None, wsd=None, *, K: int,
                    renormalize: bool = True, nthreads: int = 1) -> dict:
    """Whole layer when the expert tensors are too large to widen on the host.

    Routing is decided here, from ``x`` and ``wr`` alone; ``fetch_experts(ids)``
    must return the selected slices ``(W13[ids] [K,2I,H], W2[ids] [K,H,I])`` in
    the order given.
    """
    x = _f64(x)
    x2 = x.reshape(-1, x.shape[-1])
    lg = router_logits(x2, wr, nthreads)
    ids, w, mg = topk_softmax(lg, K, renormalize)
    M, H = x2.shape
    y = np.empty((M, H), dtype=np.float64)
    for m in range(M):
        w13sel, w2sel = fetch_experts(ids[m])
        y[m] = token_output(x2[m], w13sel, w2sel, w[m], wsgu, wsd, nthreads)
    return {"expert_ids": ids, "weights": w, "y": y, "logits": lg, "margin": mg}
