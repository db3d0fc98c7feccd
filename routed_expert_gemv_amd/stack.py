"""One decode layer's buffers and call sequence, and a hipGraph of many layers.

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

from .api import moe_decode_fused, moe_layer_decode, moe_route, shared_expert, workspace
from .synth import LayerShape


class DecodeLayer:
    """Weights, inputs and preallocated outputs of one layer (all on one device).

    forward() runs the layer through moe_layer_decode (three launches at M = 1);
    forward_separate() issues the three entry points one after another.
    """

    def __init__(self, tensors: dict, shape: LayerShape, fused: bool = True):
        self.fused = fused
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


class DecodeStack:
    """Layers run in sequence; capture() records them into one hipGraph."""

    def __init__(self, layers):
        self.layers = list(layers)
        self.graph = None

    def forward_eager(self, stream=None):
        for layer in self.layers:
            layer.forward(stream)

    def capture(self):
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
