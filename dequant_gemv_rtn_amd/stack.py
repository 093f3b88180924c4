"""Per-layer precision dispatch over a decoder stack of quantized linears.

Selective round-to-nearest keeps most linear layers in INT4 and raises a few
(the first and last decoder layers and the output head) to INT8 per channel
(Kogan, "Is (Selective) Round-To-Nearest Quantization All You Need?",
abstract; the layer bit-width allocation page, English abstract, on which
layers carry the latency gain).  A decode step runs every linear of the stack
once, each through the library's fused-dequantization call for its own format.

The step is one launch per linear on the current stream; ``capture`` records
it into a HIP graph so that host launch cost leaves the timed path.
"""

from __future__ import annotations

from typing import Dict, List, Tuple

import torch

from . import binding, synth


class DecodeStack:
    """Packed weights of every layer of a stack workload, plus per-batch
    activation and output buffers for one decode step."""

    def __init__(self, workload: synth.Workload, device="cuda"):
        self.workload = workload
        self.device = torch.device(device)
        self.layers: List[Tuple[synth.Layer, binding.QWeight]] = []
        for layer in workload.layers:
            w = synth.weights(layer, device=self.device)
            self.layers.append((layer, binding.pack(w, layer.fmt, layer.group)))
            del w
        torch.cuda.synchronize(self.device)
        self._io: Dict[int, Tuple[Dict[int, torch.Tensor], List[torch.Tensor]]] = {}

    def weight_bytes(self) -> int:
        return sum(qw.nbytes() for _, qw in self.layers)

    def step_bytes(self, b: int) -> int:
        """Algorithmic bytes of one step: packed weights and metadata of every
        layer, plus each call's activations and outputs."""
        return sum(qw.nbytes() + 2 * b * qw.k + 2 * b * qw.n for _, qw in self.layers)

    def io(self, b: int):
        """Activations (one per distinct K, seeded) and one output per layer."""
        if b not in self._io:
            ks = sorted({qw.k for _, qw in self.layers})
            xs = {k: synth.activations(b, k, self.workload.seed_x + b + k, device=self.device) for k in ks}
            ys = [torch.empty((b, qw.n), dtype=torch.float16, device=self.device) for _, qw in self.layers]
            self._io[b] = (xs, ys)
        return self._io[b]

    def step(self, b: int):
        xs, ys = self.io(b)
        for (_, qw), y in zip(self.layers, ys):
            binding.gemm_skinny(qw, xs[qw.k], out=y)

    def capture(self, b: int) -> torch.cuda.CUDAGraph:
        """Record one step into a graph (after one eager warm-up step)."""
        self.step(b)
        torch.cuda.synchronize(self.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(b)
        torch.cuda.synchronize(self.device)
        return g
