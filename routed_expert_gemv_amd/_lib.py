"""ctypes loader of libmoe_decode.so and the prototypes of include/moe_decode.h and
include/moe_prefill.h."""
from __future__ import annotations

import ctypes as C
import os
import threading

from . import build as _build

_lock = threading.Lock()
_lib = None

MOE_OK = 0
STATUS_NAMES = {0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_ALIGN",
                -4: "MOE_ERR_WORKSPACE", -5: "MOE_ERR_HIP", -6: "MOE_ERR_SCRATCH"}
EXPORTED = ["moe_abi_version", "moe_build_id", "moe_status_str", "moe_workspace_bytes", "moe_route",
            "shared_expert", "moe_decode_fused", "moe_dbg_wave_sum", "moe_dbg_w13_silu",
            "moe_dbg_w2_combine", "moe_layer_decode", "moe_layer_launches", "moe_dbg_layer_stage",
            "moe_probe_empty", "moe_probe_read", "moe_probe_copy", "moe_prefill_workspace_bytes",
            "moe_layer_prefill", "moe_dbg_prefill_stage", "moe_workspace_init",
            "moe_layer_decode_noalloc", "moe_dbg_lane_map"]

_vp = C.c_void_p
_i = C.c_int
_sz = C.c_size_t


class StaleLibraryError(RuntimeError):
    """The built library does not come from the sources in the tree."""


def lib() -> C.CDLL:
    """The loaded library; built in-tree first if it is missing.  Raises if it
    cannot be built or loaded, or if it was built from other sources than the
    tree holds (rebuild with routed_expert_gemv_amd.build): there is no other
    implementation to fall back to."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_build.LIB):  # load what is built; build only if nothing is
                _build.build(force=True)
            L = C.CDLL(_build.LIB)
            L.moe_build_id.restype = C.c_char_p
            L.moe_build_id.argtypes = []
            built, want = L.moe_build_id().decode(), _build.source_id()
            if built != want:
                raise StaleLibraryError(
                    "%s was built from other sources (build id %s..., sources %s...); rebuild it "
                    "with `python -m routed_expert_gemv_amd.build`" % (_build.LIB, built[:12],
                                                                      want[:12]))
            L.moe_abi_version.restype = _i
            L.moe_abi_version.argtypes = []
            L.moe_status_str.restype = C.c_char_p
            L.moe_status_str.argtypes = [_i]
            L.moe_workspace_bytes.restype = _sz
            L.moe_workspace_bytes.argtypes = [_i] * 6
            L.moe_route.restype = _i
            L.moe_route.argtypes = [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp]
            L.shared_expert.restype = _i
            L.shared_expert.argtypes = [_vp, _vp, _vp, _i, _i, _i, _vp, _vp, _sz, _vp]
            L.moe_decode_fused.restype = _i
            L.moe_decode_fused.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                           _vp, _vp, _sz, _vp]
            L.moe_dbg_wave_sum.restype = _i
            L.moe_dbg_wave_sum.argtypes = [_vp, _vp, _vp]
            _ip = C.POINTER(C.c_int)
            L.moe_dbg_lane_map.restype = _i
            L.moe_dbg_lane_map.argtypes = [_i, _ip, _ip, _ip]
            L.moe_dbg_w13_silu.restype = _i
            L.moe_dbg_w13_silu.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _sz, _vp]
            L.moe_dbg_w2_combine.restype = _i
            L.moe_dbg_w2_combine.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp,
                                             _vp, _sz, _vp]
            L.moe_layer_decode.restype = _i
            L.moe_layer_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp] + [_i] * 7 + \
                [_vp, _vp, _vp, _vp, _vp, _sz, _vp]
            L.moe_dbg_layer_stage.restype = _i
            L.moe_dbg_layer_stage.argtypes = [_i] + L.moe_layer_decode.argtypes
            L.moe_probe_empty.restype = _i
            L.moe_probe_empty.argtypes = [_vp]
            L.moe_probe_copy.restype = _i
            L.moe_probe_copy.argtypes = [_vp, _vp, _sz, _vp]
            L.moe_probe_read.restype = _i
            L.moe_probe_read.argtypes = [_vp, _sz, _vp, _vp]
            L.moe_layer_launches.restype = _i
            L.moe_layer_launches.argtypes = [_i] * 6
            L.moe_prefill_workspace_bytes.restype = _sz
            L.moe_prefill_workspace_bytes.argtypes = [_i] * 6
            L.moe_layer_prefill.restype = _i
            L.moe_layer_prefill.argtypes = L.moe_layer_decode.argtypes
            L.moe_layer_decode_noalloc.restype = _i
            L.moe_layer_decode_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp] + [_i] * 7 + \
                [_vp, _vp, _vp, _vp, _vp]
            L.moe_workspace_init.restype = _i
            L.moe_workspace_init.argtypes = [_vp, _sz, _vp]
            L.moe_dbg_prefill_stage.restype = _i
            L.moe_dbg_prefill_stage.argtypes = [_i] + L.moe_layer_decode.argtypes
            _lib = L
    return _lib


def path() -> str:
    return _build.LIB
