"""A decode step's GEMV sequence, run eagerly, replayed from one captured graph, or run as
one persistent chain launch.

The sequence is a list of calls, each one weight matrix (or several that share X: the fused
QKV and gate_up projections), one input X and its outputs. Calls run in list order on one
stream, as the dependent GEMVs of a real decode step would; capturing the whole list into one
graph moves it across the host-device boundary once per step, which removes the host launch
gaps between the kernels (decode-GEMV page, "A strong answer", cause 3; GPU performance chains
page, "Launch gaps in a decode step").

Plans and one shared split-K workspace are created up front; calls never overlap on the
stream, so sharing the workspace is safe.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from ._binding import Chain, Graph, Plan, fused_run, run


@dataclass
class Call:
    weights: list          # bf16 [n_i, k] tensors (one, or the segments of a fused call)
    x: torch.Tensor        # bf16 [m, k]
    ys: list               # fp32 [m, n_i] tensors, one per weight
    plan: Plan = None

    @property
    def n(self) -> int:
        return sum(w.shape[0] for w in self.weights)


class Sequence:
    def __init__(self, calls: list[Call], device=None):
        self.calls = calls
        ws = 0
        for c in calls:
            if c.plan is None:
                c.plan = Plan(c.n, c.x.shape[-1], c.x.shape[0] if c.x.dim() == 2 else 1, device)
            ws = max(ws, c.plan.workspace_size)
        self.workspace = (torch.zeros(ws, dtype=torch.uint8, device=calls[0].x.device)
                          if ws else None)
        self.graph: Graph | None = None

    def run(self, stream=None):
        """Issue every call on `stream` (default: torch's current stream), asynchronously."""
        for c in self.calls:
            if len(c.weights) == 1:
                run(c.plan, c.weights[0], c.x, c.ys[0], self.workspace, stream)
            else:
                fused_run(c.plan, list(zip(c.weights, c.ys)), c.x, self.workspace, stream)

    def capture(self, stream) -> Graph:
        """Record the whole sequence on `stream` (not the legacy default stream) into a graph."""
        if self.graph is not None:
            self.graph.destroy()
        g = Graph(stream)
        with g:
            self.run(stream)
        self.graph = g
        return g

    def replay(self, stream=None):
        self.graph.launch(stream)

    def chain(self, **opts) -> Chain:
        """The same sequence as one persistent launch (batch-1 calls only): every call waits
        for the previous one to complete, but streams its weights ahead of that wait."""
        return Chain([(list(zip(c.weights, c.ys)), c.x) for c in self.calls], **opts)

    @property
    def weight_bytes(self) -> int:
        return sum(w.numel() * w.element_size() for c in self.calls for w in c.weights)

    @property
    def alg_bytes(self) -> int:
        """W and X read once, Y written once, summed over the calls."""
        total = 0
        for c in self.calls:
            total += sum(w.numel() * 2 for w in c.weights)
            total += c.x.numel() * 2
            total += sum(y.numel() * 4 for y in c.ys)
        return total
