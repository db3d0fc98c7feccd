"""Python binding of the C ABI in include/moe_decode.h (same names).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe_decode.so.  Tensors are torch tensors on the current HIP device; torch
provides device memory and streams, nothing else.  A non-zero status from the
library raises MoeError.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _lib


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _lib.lib().moe_status_str(int(status)).decode()
        super().__init__("%s: %s (%s)" % (fn, msg, _lib.STATUS_NAMES.get(status, status)))
        self.status = status


def _check(fn, st):
    if st != 0:
        raise MoeError(fn, st)


def _dev_tensor(name, t, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor, got %s" % (name, t.device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    return t


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t):
    return None if t is None else t.data_ptr()


def moe_abi_version() -> int:
    return int(_lib.lib().moe_abi_version())


def moe_status_str(status: int) -> str:
    """The library's name for a status code."""
    return _lib.lib().moe_status_str(int(status)).decode()


def moe_build_id() -> str:
    """SHA-256 of the sources the loaded library was built from."""
    return _lib.lib().moe_build_id().decode()


def moe_workspace_bytes(M: int, H: int, E: int, I: int, K: int, Is: int = 0) -> int:
    return int(_lib.lib().moe_workspace_bytes(M, H, E, I, K, Is))


def workspace(M: int, H: int, E: int, I: int, K: int, Is: int = 0, device=None) -> torch.Tensor:
    """A zero-filled device workspace big enough for every entry point at these sizes."""
    n = moe_workspace_bytes(M, H, E, I, K, Is)
    if n == 0:
        raise MoeError("moe_workspace_bytes", -2)
    return torch.zeros(n, dtype=torch.uint8, device=device or torch.cuda.current_device())


def moe_workspace_init(ws, stream=None) -> None:
    """Zero the state block at the start of a workspace (needed once before a
    workspace that did not come from workspace() is first used)."""
    _dev_tensor("ws", ws, torch.uint8)
    _check("moe_workspace_init", _lib.lib().moe_workspace_init(_ptr(ws), ws.numel(),
                                                               _stream(stream, ws.device)))


def moe_route(x, w_router, K: int, renormalize: bool = True, topk_ids=None, topk_w=None,
              logits=None, stream=None):
    """Router GEMV + top-K + routing weights.  Returns (topk_ids, topk_w, logits)."""
    _dev_tensor("x", x, torch.float16, 2)
    _dev_tensor("w_router", w_router, torch.float16, 2)
    M, H = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != H:
        raise ValueError("w_router must be [E, %d], got %s" % (H, tuple(w_router.shape)))
    dev = x.device
    topk_ids = torch.empty((M, K), dtype=torch.int32, device=dev) if topk_ids is None else topk_ids
    topk_w = torch.empty((M, K), dtype=torch.float32, device=dev) if topk_w is None else topk_w
    logits = torch.empty((M, E), dtype=torch.float32, device=dev) if logits is None else logits
    _dev_tensor("topk_ids", topk_ids, torch.int32)
    _dev_tensor("topk_w", topk_w, torch.float32)
    _dev_tensor("logits", logits, torch.float32)
    if topk_ids.numel() != M * K or topk_w.numel() != M * K or logits.numel() != M * E:
        raise ValueError("output sizes do not match M=%d K=%d E=%d" % (M, K, E))
    st = _lib.lib().moe_route(_ptr(x), _ptr(w_router), M, H, E, K, int(bool(renormalize)),
                              _ptr(topk_ids), _ptr(topk_w), _ptr(logits), _stream(stream, dev))
    _check("moe_route", st)
    return topk_ids, topk_w, logits


def shared_expert(x, w_gate_up, w_down, s_out=None, ws=None, stream=None):
    """Shared expert (gate_up -> SiLU*mul -> down) into fp32 s_out [M, H]."""
    _dev_tensor("x", x, torch.float16, 2)
    _dev_tensor("w_gate_up", w_gate_up, torch.float16, 2)
    _dev_tensor("w_down", w_down, torch.float16, 2)
    M, H = x.shape
    Is = w_gate_up.shape[0] // 2
    if w_gate_up.shape != (2 * Is, H) or w_down.shape != (H, Is):
        raise ValueError("shared expert shapes: gate_up %s, down %s for H=%d"
                         % (tuple(w_gate_up.shape), tuple(w_down.shape), H))
    dev = x.device
    s_out = torch.empty((M, H), dtype=torch.float32, device=dev) if s_out is None else s_out
    _dev_tensor("s_out", s_out, torch.float32)
    if s_out.numel() != M * H:
        raise ValueError("s_out must have M*H elements")
    if ws is None:
        ws = workspace(max(M, 1), H, 1, 64, 1, Is, dev)
    _dev_tensor("ws", ws, torch.uint8)
    st = _lib.lib().shared_expert(_ptr(x), _ptr(w_gate_up), _ptr(w_down), M, H, Is, _ptr(s_out),
                                  _ptr(ws), ws.numel(), _stream(stream, dev))
    _check("shared_expert", st)
    return s_out


def moe_decode_fused(x, w13, w2, topk_ids, topk_w, shared_in=None, y=None, ws=None, stream=None):
    """Expert-indexed W13 + SiLU*mul, W2 + weighted combine (+ shared_in) -> fp16 y [M, H]."""
    _dev_tensor("x", x, torch.float16, 2)
    _dev_tensor("w13", w13, torch.float16, 3)
    _dev_tensor("w2", w2, torch.float16, 3)
    _dev_tensor("topk_ids", topk_ids, torch.int32)
    _dev_tensor("topk_w", topk_w, torch.float32)
    M, H = x.shape
    E, twoI, H2 = w13.shape
    I = twoI // 2
    K = topk_ids.shape[-1]
    if H2 != H or w2.shape != (E, H, I):
        raise ValueError("expert shapes: w13 %s, w2 %s for H=%d"
                         % (tuple(w13.shape), tuple(w2.shape), H))
    if topk_ids.numel() != M * K or topk_w.numel() != M * K:
        raise ValueError("topk_ids / topk_w must be [M, K]")
    dev = x.device
    if shared_in is not None:
        _dev_tensor("shared_in", shared_in, torch.float32)
        if shared_in.numel() != M * H:
            raise ValueError("shared_in must be [M, H]")
    y = torch.empty((M, H), dtype=torch.float16, device=dev) if y is None else y
    _dev_tensor("y", y, torch.float16)
    if y.numel() != M * H:
        raise ValueError("y must be [M, H]")
    if ws is None:
        ws = workspace(max(M, 1), H, E, I, K, 0, dev)
    _dev_tensor("ws", ws, torch.uint8)
    st = _lib.lib().moe_decode_fused(_ptr(x), _ptr(w13), _ptr(w2), _ptr(topk_ids), _ptr(topk_w),
                                     _ptr(shared_in), M, H, E, I, K, _ptr(y), _ptr(ws), ws.numel(),
                                     _stream(stream, dev))
    _check("moe_decode_fused", st)
    return y


def moe_dbg_lane_map(n: int):
    """The lane mapping of down-projection rows n fp16 wide (host query):
    (lanes per row, 16-byte chunks per lane, whether steps past the row are
    padded)."""
    import ctypes as C
    a, b, c = C.c_int(), C.c_int(), C.c_int()
    _check("moe_dbg_lane_map", _lib.lib().moe_dbg_lane_map(int(n), C.byref(a), C.byref(b),
                                                          C.byref(c)))
    return a.value, b.value, bool(c.value)


def moe_dbg_wave_sum(values, out=None, stream=None):
    """Test probe: the 64 fp32 values summed by one wave's cross-lane reduction."""
    _dev_tensor("values", values, torch.float32)
    if values.numel() != 64:
        raise ValueError("values must hold 64 elements")
    out = torch.empty(1, dtype=torch.float32, device=values.device) if out is None else out
    st = _lib.lib().moe_dbg_wave_sum(_ptr(values), _ptr(out), _stream(stream, values.device))
    _check("moe_dbg_wave_sum", st)
    return out


def moe_dbg_w13_silu(x, w13, topk_ids, activated=None, ws=None, stream=None):
    """Test probe: the W13 + SiLU*mul stage alone -> activated [M, K, I] fp32."""
    _dev_tensor("x", x, torch.float16, 2)
    _dev_tensor("w13", w13, torch.float16, 3)
    _dev_tensor("topk_ids", topk_ids, torch.int32)
    M, H = x.shape
    E, twoI, _ = w13.shape
    I = twoI // 2
    K = topk_ids.shape[-1]
    dev = x.device
    activated = (torch.zeros((M, K, I), dtype=torch.float32, device=dev)
                 if activated is None else activated)
    _dev_tensor("activated", activated, torch.float32)
    if ws is None:
        ws = workspace(max(M, 1), H, E, I, K, 0, dev)
    st = _lib.lib().moe_dbg_w13_silu(_ptr(x), _ptr(w13), _ptr(topk_ids), M, H, E, I, K,
                                     _ptr(activated), _ptr(ws), ws.numel(), _stream(stream, dev))
    _check("moe_dbg_w13_silu", st)
    return activated


def moe_dbg_w2_combine(activated, w2, topk_ids, topk_w, shared_in=None, y=None, ws=None,
                       stream=None):
    """Test probe: the W2 + combine stage alone on injected activations [M, K, I] fp32."""
    _dev_tensor("activated", activated, torch.float32, 3)
    _dev_tensor("w2", w2, torch.float16, 3)
    _dev_tensor("topk_ids", topk_ids, torch.int32)
    _dev_tensor("topk_w", topk_w, torch.float32)
    M, K, I = activated.shape
    E, H, I2 = w2.shape
    if I2 != I or topk_ids.numel() != M * K or topk_w.numel() != M * K:
        raise ValueError("shapes do not match activated [M, K, I]")
    dev = activated.device
    if shared_in is not None:
        _dev_tensor("shared_in", shared_in, torch.float32)
    y = torch.empty((M, H), dtype=torch.float16, device=dev) if y is None else y
    _dev_tensor("y", y, torch.float16)
    if ws is None:
        ws = workspace(max(M, 1), H, E, I, K, 0, dev)
    st = _lib.lib().moe_dbg_w2_combine(_ptr(activated), _ptr(w2), _ptr(topk_ids), _ptr(topk_w),
                                       _ptr(shared_in), M, H, E, I, K, _ptr(y), _ptr(ws),
                                       ws.numel(), _stream(stream, dev))
    _check("moe_dbg_w2_combine", st)
    return y


def _layer_call(x, w_router, w13, w2, w_gate_up, w_down, K, renormalize, topk_ids, topk_w,
                logits, y, ws, make_ws=None):
    """Checks and marshals the layer entry points' arguments; returns (outputs, C args)."""
    _dev_tensor("x", x, torch.float16, 2)
    _dev_tensor("w_router", w_router, torch.float16, 2)
    _dev_tensor("w13", w13, torch.float16, 3)
    _dev_tensor("w2", w2, torch.float16, 3)
    M, H = x.shape
    E, twoI, H2 = w13.shape
    I = twoI // 2
    if H2 != H or w2.shape != (E, H, I) or w_router.shape != (E, H):
        raise ValueError("layer shapes: router %s, w13 %s, w2 %s for H=%d"
                         % (tuple(w_router.shape), tuple(w13.shape), tuple(w2.shape), H))
    Is = 0
    if w_gate_up is not None or w_down is not None:
        _dev_tensor("w_gate_up", w_gate_up, torch.float16, 2)
        _dev_tensor("w_down", w_down, torch.float16, 2)
        Is = w_gate_up.shape[0] // 2
        if w_gate_up.shape != (2 * Is, H) or w_down.shape != (H, Is):
            raise ValueError("shared expert shapes: gate_up %s, down %s"
                             % (tuple(w_gate_up.shape), tuple(w_down.shape)))
    dev = x.device
    topk_ids = torch.empty((M, K), dtype=torch.int32, device=dev) if topk_ids is None else topk_ids
    topk_w = torch.empty((M, K), dtype=torch.float32, device=dev) if topk_w is None else topk_w
    logits = torch.empty((M, E), dtype=torch.float32, device=dev) if logits is None else logits
    y = torch.empty((M, H), dtype=torch.float16, device=dev) if y is None else y
    for name, t, dt, n in (("topk_ids", topk_ids, torch.int32, M * K),
                           ("topk_w", topk_w, torch.float32, M * K),
                           ("logits", logits, torch.float32, M * E), ("y", y, torch.float16, M * H)):
        _dev_tensor(name, t, dt)
        if t.numel() != n:
            raise ValueError("%s must have %d elements" % (name, n))
    args = (_ptr(x), _ptr(w_router), _ptr(w13), _ptr(w2), _ptr(w_gate_up), _ptr(w_down), M, H, E,
            I, K, Is, int(bool(renormalize)), _ptr(topk_ids), _ptr(topk_w), _ptr(logits), _ptr(y))
    if ws is False:  # the entry point takes no workspace
        return (y, topk_ids, topk_w, logits), args
    if ws is None:
        ws = (make_ws or workspace)(max(M, 1), H, E, I, K, Is, dev)
    _dev_tensor("ws", ws, torch.uint8)
    return (y, topk_ids, topk_w, logits), args + (_ptr(ws), ws.numel())


def moe_layer_decode(x, w_router, w13, w2, w_gate_up=None, w_down=None, K: int = 8,
                     renormalize: bool = True, topk_ids=None, topk_w=None, logits=None, y=None,
                     ws=None, stream=None):
    """The whole layer (shared expert, routing, routed experts, combine) in as few
    launches as the sizes allow.  Returns (y, topk_ids, topk_w, logits)."""
    out, args = _layer_call(x, w_router, w13, w2, w_gate_up, w_down, K, renormalize, topk_ids,
                            topk_w, logits, y, ws)
    st = _lib.lib().moe_layer_decode(*args, _stream(stream, x.device))
    _check("moe_layer_decode", st)
    return out


def moe_layer_decode_noalloc(x, w_router, w13, w2, w_gate_up=None, w_down=None, K: int = 8,
                             renormalize: bool = True, topk_ids=None, topk_w=None, logits=None,
                             y=None, stream=None):
    """moe_layer_decode without a workspace argument: the library's static
    512 KiB device buffer serves as the workspace (nothing is allocated by the
    call; calls on one GPU must not overlap).  Returns (y, topk_ids, topk_w, logits)."""
    out, args = _layer_call(x, w_router, w13, w2, w_gate_up, w_down, K, renormalize, topk_ids,
                            topk_w, logits, y, False)
    st = _lib.lib().moe_layer_decode_noalloc(*args, _stream(stream, x.device))
    _check("moe_layer_decode_noalloc", st)
    return out


def moe_dbg_layer_stage(stage: int, x, w_router, w13, w2, w_gate_up=None, w_down=None,
                        K: int = 8, renormalize: bool = True, topk_ids=None, topk_w=None,
                        logits=None, y=None, ws=None, stream=None):
    """Test and benchmark probe of moe_layer_decode.  Stage 1, 2, 3: one step
    of the layer's launches (router; selection and gate/up rows; down rows
    and combine -- the shared expert's rows go with them as the layer places
    them; one launch each, except the selection launch of M = 5..8), alone,
    on buffers a full call already filled; 4: the layer's launches whole; 5
    (M = 1): the single-launch path; 6: the single-launch path with every
    wait giving up at once (each workgroup computes what it would have waited
    for).  Returns (y, topk_ids, topk_w, logits)."""
    out, args = _layer_call(x, w_router, w13, w2, w_gate_up, w_down, K, renormalize, topk_ids,
                            topk_w, logits, y, ws)
    st = _lib.lib().moe_dbg_layer_stage(int(stage), *args, _stream(stream, x.device))
    _check("moe_dbg_layer_stage", st)
    return out


def moe_layer_launches(M: int, H: int, E: int, I: int, K: int, Is: int = 0) -> int:
    """Number of kernels moe_layer_decode enqueues for these sizes (0 if unsupported)."""
    return int(_lib.lib().moe_layer_launches(M, H, E, I, K, Is))


def moe_probe_empty(stream=None):
    """Bench probe: launch one empty kernel."""
    dev = torch.device("cuda", torch.cuda.current_device())
    _check("moe_probe_empty", _lib.lib().moe_probe_empty(_stream(stream, dev)))


def moe_probe_copy(src, dst, stream=None) -> None:
    """Test probe: plain device copy of src into dst (same byte size)."""
    _dev_tensor("src", src, torch.float16)
    _dev_tensor("dst", dst, torch.float16)
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst differ in size")
    _check("moe_probe_copy", _lib.lib().moe_probe_copy(_ptr(src), _ptr(dst), n,
                                                        _stream(stream, src.device)))


def moe_probe_read(buf, out=None, stream=None):
    """Bench probe: stream the bytes of a device tensor with 16-byte loads."""
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    out = torch.zeros(1, dtype=torch.float32, device=buf.device) if out is None else out
    n = buf.numel() * buf.element_size()
    _check("moe_probe_read", _lib.lib().moe_probe_read(_ptr(buf), n - n % 16, _ptr(out),
                                                       _stream(stream, buf.device)))
    return out


def moe_prefill_workspace_bytes(T: int, H: int, E: int, I: int, K: int, Is: int = 0) -> int:
    return int(_lib.lib().moe_prefill_workspace_bytes(T, H, E, I, K, Is))


def prefill_workspace(T: int, H: int, E: int, I: int, K: int, Is: int = 0,
                      device=None) -> torch.Tensor:
    """A device workspace big enough for moe_layer_prefill at these sizes."""
    n = moe_prefill_workspace_bytes(T, H, E, I, K, Is)
    if n == 0:
        raise MoeError("moe_prefill_workspace_bytes", -2)
    return torch.zeros(n, dtype=torch.uint8, device=device or torch.cuda.current_device())


def moe_layer_prefill(x, w_router, w13, w2, w_gate_up=None, w_down=None, K: int = 8,
                      renormalize: bool = True, topk_ids=None, topk_w=None, logits=None, y=None,
                      ws=None, stream=None):
    """The layer for T tokens at once (x [T, H]) on the matrix cores.
    Returns (y, topk_ids, topk_w, logits)."""
    out, args = _layer_call(x, w_router, w13, w2, w_gate_up, w_down, K, renormalize, topk_ids,
                            topk_w, logits, y, ws, prefill_workspace)
    _check("moe_layer_prefill", _lib.lib().moe_layer_prefill(*args, _stream(stream, x.device)))
    return out


def moe_dbg_prefill_stage(stage: int, x, w_router, w13, w2, w_gate_up=None, w_down=None,
                          K: int = 8, renormalize: bool = True, topk_ids=None, topk_w=None,
                          logits=None, y=None, ws=None, stream=None):
    """One of moe_layer_prefill's six stages alone (test-only; for timing)."""
    out, args = _layer_call(x, w_router, w13, w2, w_gate_up, w_down, K, renormalize, topk_ids,
                            topk_w, logits, y, ws, prefill_workspace)
    _check("moe_dbg_prefill_stage",
           _lib.lib().moe_dbg_prefill_stage(int(stage), *args, _stream(stream, x.device)))
    return out
