"""Seeded synthetic MoE decode layers (inputs only; none of the layer's arithmetic).

This module is the one place both sides of a parity check take their inputs
from: the HIP path receives the tensors on the device, the fp64 oracle receives
host copies of the same tensors.  It draws random numbers and nothing else.

Recipe (the pages measure on a private checkpoint; seeded synthetic tensors at
the pages' shapes stand in for it):
  draw order per layer seed s:  Wr [E,H], W13 [E,2I,H] (expert by expert),
  W2 [E,H,I] (expert by expert), Wsgu [2Is,H], Wsd [H,Is], x [M,H];
  weights = fp16(N(0,1) * 0.02) drawn in fp32, x = fp16(N(0,1)).
  A redraw of x (attempt a >= 1) uses a fresh generator seeded s + 1000003*a.
"""
from __future__ import annotations

from dataclasses import dataclass, asdict

import torch

X_REDRAW_STRIDE = 1_000_003
WEIGHT_STD = 0.02


@dataclass(frozen=True)
class LayerShape:
    """Shape of one MoE decode layer: M tokens, hidden H, E experts, top-K,
    per-expert intermediate I, shared-expert intermediate Is (0 = none)."""
    M: int
    H: int
    E: int
    K: int
    I: int
    Is: int
    renormalize: bool = True

    def as_dict(self):
        return asdict(self)


# Workloads at the pages' shapes (hidden 2048, 256 experts, top-8) plus a tiny one.
SHAPES = {
    "tiny_e16_k4_i128": LayerShape(M=1, H=2048, E=16, K=4, I=128, Is=0),
    "tp4_shard_e256_k8_i128": LayerShape(M=1, H=2048, E=256, K=8, I=128, Is=128),
    "full_e256_k8_i512": LayerShape(M=1, H=2048, E=256, K=8, I=512, Is=512),
    "batch2_e256_k8_i512": LayerShape(M=2, H=2048, E=256, K=8, I=512, Is=512),
    "batch4_e256_k8_i512": LayerShape(M=4, H=2048, E=256, K=8, I=512, Is=512),
    "batch8_e256_k8_i512": LayerShape(M=8, H=2048, E=256, K=8, I=512, Is=512),
}
STACK_LAYERS = 36  # the 36-layer decode stack is 36 independent full-width layers


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _weights(g, shape, device):
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(WEIGHT_STD).to(torch.float16)


def draw_layer(shape: LayerShape, seed: int, device="cpu") -> dict:
    """Draw one layer's tensors (fp16, row-major, contiguous) on ``device``."""
    dev = torch.device(device)
    g = _gen(dev, seed)
    H, E, I, Is, M = shape.H, shape.E, shape.I, shape.Is, shape.M
    out = {}
    out["wr"] = _weights(g, (E, H), dev)
    w13 = torch.empty((E, 2 * I, H), dtype=torch.float16, device=dev)
    for e in range(E):
        w13[e] = _weights(g, (2 * I, H), dev)
    out["w13"] = w13
    w2 = torch.empty((E, H, I), dtype=torch.float16, device=dev)
    for e in range(E):
        w2[e] = _weights(g, (H, I), dev)
    out["w2"] = w2
    if Is > 0:
        out["wsgu"] = _weights(g, (2 * Is, H), dev)
        out["wsd"] = _weights(g, (H, Is), dev)
    else:
        out["wsgu"] = None
        out["wsd"] = None
    out["x"] = torch.randn((M, H), generator=g, device=dev, dtype=torch.float32).to(torch.float16)
    return out


def redraw_x(shape: LayerShape, seed: int, attempt: int, device="cpu") -> torch.Tensor:
    """A fresh activation x [M,H] for attempt >= 1 (used when a draw must be replaced)."""
    if attempt < 1:
        raise ValueError("attempt 0 is the x drawn by draw_layer")
    dev = torch.device(device)
    g = _gen(dev, seed + X_REDRAW_STRIDE * attempt)
    return torch.randn((shape.M, shape.H), generator=g, device=dev,
                       dtype=torch.float32).to(torch.float16)
