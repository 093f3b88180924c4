"""Per-layer precision dispatch over a decoder stack of quantized linears.

Selective round-to-nearest keeps most linear layers in INT4 and raises a few
(the first and last decoder layers and the output head) to INT8 per channel
(Kogan, "Is (Selective) Round-To-Nearest Quantization All You Need?",
abstract; the layer bit-width allocation page, English abstract, on which
layers carry the latency gain).  A decode step runs every linear of the stack
once, each through the library's fused-dequantization call for its own format.

The step is one launch per linear on the current stream (or per fused group
of linears that share their input); ``capture`` records it into a HIP graph
so that host launch cost leaves the timed path.
"""

from __future__ import annotations

from typing import Dict, List, Tuple

import torch

from . import binding, synth


# Linears of one decoder layer that read the same activations: their rows
# can be stacked into one matrix and served by one launch.
FUSIBLE = (("q", "k", "v"), ("gate", "up"))


class PrecisionMap:
    """Per-linear format choice of a decoder stack: a low-bit default and a
    set of up-precisioned linears (selective RTN: the first and last decoder
    layers and the output head in INT8 per channel, the rest INT4 g128).

    ``for_layer(name, k)`` returns (format, group) for a linear named
    ``l<i>.<module>`` or ``lm_head`` with input width k."""

    def __init__(self, n_layers: int = 32, high_layers=(0, 1, 30, 31), low=("int4_asym", 128),
                 high="int8", high_modules=("lm_head",)):
        self.n_layers = n_layers
        self.high_layers = frozenset(high_layers)
        self.low = low
        self.high = high
        self.high_modules = frozenset(high_modules)

    def is_high(self, name: str) -> bool:
        if name in self.high_modules:
            return True
        layer, _, _ = name.partition(".")
        return layer.startswith("l") and layer[1:].isdigit() and int(layer[1:]) in self.high_layers

    def for_layer(self, name: str, k: int) -> Tuple[str, int]:
        return (self.high, k) if self.is_high(name) else self.low


def fuse_layers(layers) -> List[Tuple[str, List[synth.Layer]]]:
    """Group the stack's linears into launches: q|k|v and gate|up of each
    decoder layer become one matrix each (same k, format and group), every
    other linear stays alone.  Returns (name, members) in stack order."""
    by_name = {l.name: l for l in layers}
    out, done = [], set()
    for l in layers:
        if l.name in done:
            continue
        prefix, _, mod = l.name.rpartition(".")
        members = [l]
        for grp in FUSIBLE:
            if mod == grp[0] and prefix:
                cand = [by_name.get(f"{prefix}.{m}") for m in grp]
                if all(c is not None and (c.k, c.fmt, c.group) == (l.k, l.fmt, l.group) for c in cand):
                    members = cand
        done.update(m.name for m in members)
        name = members[0].name if len(members) == 1 else f"{prefix}." + "_".join(m.name.rpartition(".")[2] for m in members)
        out.append((name, members))
    return out


class DecodeStack:
    """Packed weights of every layer of a stack workload, plus per-batch
    activation and output buffers for one decode step.

    fused=True stacks the rows of q|k|v and of gate|up of each decoder layer
    into one matrix each (one launch instead of three or two); the weights
    are the same draws, so every output row equals the unfused one's."""

    def __init__(self, workload: synth.Workload, device="cuda", fused: bool = False):
        self.workload = workload
        self.device = torch.device(device)
        self.fused = fused
        self.layers: List[Tuple[synth.Layer, binding.QWeight]] = []
        groups = fuse_layers(workload.layers) if fused else [(l.name, [l]) for l in workload.layers]
        for name, members in groups:
            w = torch.cat([synth.weights(m, device=self.device) for m in members], dim=0)
            head = members[0]
            layer = synth.Layer(name, w.shape[0], head.k, head.fmt, head.group, head.dist, head.seed_w)
            self.layers.append((layer, binding.pack(w, head.fmt, head.group)))
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
        """Activations (one per distinct K, seeded), one output per layer, and
        one workspace that the layers' calls share (they run in order on one
        stream)."""
        if b not in self._io:
            ks = sorted({qw.k for _, qw in self.layers})
            xs = {k: synth.activations(b, k, self.workload.seed_x + b + k, device=self.device) for k in ks}
            ys = [torch.empty((b, qw.n), dtype=torch.float16, device=self.device) for _, qw in self.layers]
            need = max(binding.workspace_bytes(qw, b) for _, qw in self.layers)
            ws = torch.empty(need, dtype=torch.uint8, device=self.device)
            self._io[b] = (xs, ys, ws)
        return self._io[b]

    def step(self, b: int):
        xs, ys, ws = self.io(b)
        for (_, qw), y in zip(self.layers, ys):
            binding.gemm_skinny(qw, xs[qw.k], out=y, workspace=ws)

    def stage_ids(self) -> List[int]:
        """Dependency stage of each launch: in a decoder q|k|v read the layer
        input, o the attention output, gate|up the normed residual, down the
        activation, and the head the last layer's output, so each decoder
        layer has four stages and linears of one stage read the same input."""
        ids, prev = [], None
        order = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3}
        for layer, _ in self.layers:
            if layer.name == "lm_head":
                key = (10 ** 6, 0)
            else:
                li, _, mod = layer.name.partition(".")
                key = (int(li[1:]), order[mod.split("_")[0]])
            ids.append(key)
        # dense numbering in order of appearance
        dense, out = {}, []
        for key in ids:
            dense.setdefault(key, len(dense))
            out.append(dense[key])
        return out

    def plan(self, b: int = 1) -> "binding.StackPlan":
        """The whole step as one persistent launch (b = 1): one entry per
        launch of step(), in stage order, on this stack's activations and
        outputs."""
        if b != 1:
            raise ValueError("the one-launch decode stack runs batch 1")
        xs, ys, _ = self.io(b)
        entries = [(qw, xs[qw.k], y, sid) for (_, qw), y, sid in zip(self.layers, ys, self.stage_ids())]
        return binding.StackPlan(entries)

    def capture(self, b: int) -> torch.cuda.CUDAGraph:
        """Record one step into a graph (after one eager warm-up step)."""
        self.step(b)
        torch.cuda.synchronize(self.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(b)
        torch.cuda.synchronize(self.device)
        return g
