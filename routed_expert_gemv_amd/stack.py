"""One layer's buffers and call sequence (decode, or prefill over many tokens),
and a hipGraph of many layers.

A layer runs either as moe_layer_decode (three launches at M = 1) or as the
three entry points on one stream: shared_expert (independent of routing, so it
goes first), moe_route, moe_decode_fused (which adds the shared output before
its single fp16 rounding).  A stack captures every
layer's launches into one hipGraph (torch.cuda.CUDAGraph drives stream
capture; the captured nodes are this library's kernels), so one replay is one
host call.
"""
from __future__ import annotations

import torch

from .api import (moe_dbg_layer_stage, moe_dbg_prefill_stage, moe_decode_fused, moe_layer_decode, moe_layer_prefill,
                  moe_route, prefill_workspace, shared_expert, workspace)
from .synth import LayerShape


class DecodeLayer:
    """Weights, inputs and preallocated outputs of one layer (all on one device).

    forward() runs the layer through moe_layer_decode (three launches at M = 1);
    forward_separate() issues the three entry points one after another; with
    single=True (M = 1 only) forward() runs the single-launch layer instead.
    """

    def __init__(self, tensors: dict, shape: LayerShape, fused: bool = True,
                 single: bool = False):
        self.fused = fused
        self.single = single
        self.shape = shape
        self.t = tensors
        dev = tensors["x"].device
        M, H, E, K, I, Is = shape.M, shape.H, shape.E, shape.K, shape.I, shape.Is
        self.topk_ids = torch.empty((M, K), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((M, K), dtype=torch.float32, device=dev)
        self.logits = torch.empty((M, E), dtype=torch.float32, device=dev)
        self.s = torch.empty((M, H), dtype=torch.float32, device=dev) if Is > 0 else None
        self.y = torch.empty((M, H), dtype=torch.float16, device=dev)
        self.ws = workspace(max(M, 1), H, E, I, K, Is, dev)

    def forward(self, stream=None):
        if not self.fused:
            return self.forward_separate(stream)
        t, sh = self.t, self.shape
        if self.single:
            moe_dbg_layer_stage(5, t["x"], t["wr"], t["w13"], t["w2"], t["wsgu"], t["wsd"], sh.K,
                                sh.renormalize, self.topk_ids, self.topk_w, self.logits, self.y,
                                self.ws, stream=stream)
            return self.y
        moe_layer_decode(t["x"], t["wr"], t["w13"], t["w2"], t["wsgu"], t["wsd"], sh.K,
                         sh.renormalize, self.topk_ids, self.topk_w, self.logits, self.y, self.ws,
                         stream=stream)
        return self.y

    def forward_separate(self, stream=None):
        t, sh = self.t, self.shape
        if self.s is not None:
            shared_expert(t["x"], t["wsgu"], t["wsd"], s_out=self.s, ws=self.ws, stream=stream)
        moe_route(t["x"], t["wr"], sh.K, sh.renormalize, self.topk_ids, self.topk_w, self.logits,
                  stream=stream)
        moe_decode_fused(t["x"], t["w13"], t["w2"], self.topk_ids, self.topk_w,
                         shared_in=self.s, y=self.y, ws=self.ws, stream=stream)
        return self.y


class PrefillLayer:
    """One layer over T = shape.M tokens through moe_layer_prefill, with
    preallocated outputs; `ws` may be shared by layers that run one after
    another on one stream (the workspace holds nothing between calls)."""

    def __init__(self, tensors: dict, shape: LayerShape, ws=None):
        self.shape = shape
        self.t = tensors
        dev = tensors["x"].device
        T, H, E, K = shape.M, shape.H, shape.E, shape.K
        self.topk_ids = torch.empty((T, K), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        self.y = torch.empty((T, H), dtype=torch.float16, device=dev)
        self.ws = ws if ws is not None else prefill_workspace(max(T, 1), H, E, shape.I, K,
                                                              shape.Is, dev)

    def _args(self):
        t, sh = self.t, self.shape
        return (t["x"], t["wr"], t["w13"], t["w2"], t["wsgu"], t["wsd"], sh.K, sh.renormalize,
                self.topk_ids, self.topk_w, self.logits, self.y, self.ws)

    def forward(self, stream=None):
        moe_layer_prefill(*self._args(), stream=stream)
        return self.y

    def stage(self, stage: int, stream=None):
        """One of the six stages alone (1..6), reading what earlier ones left."""
        moe_dbg_prefill_stage(stage, *self._args(), stream=stream)


class DecodeStack:
    """Layers run in sequence; capture() records them into one hipGraph."""

    def __init__(self, layers):
        self.layers = list(layers)
        self.graph = None

    def forward_eager(self, stream=None):
        for layer in self.layers:
            layer.forward(stream)

    def capture(self):
        """Record every layer's launches into one hipGraph (works for decode and
        prefill layers alike)."""
        dev = self.layers[0].y.device
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            self.forward_eager()  # warm-up outside the graph
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize(dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.forward_eager()
        self.graph = g
        return g

    def replay(self):
        if self.graph is None:
            raise RuntimeError("capture() first")
        self.graph.replay()
