"""Seeded synthetic inputs: weight matrices and activations of the workloads.

No quantization or product arithmetic lives here; both the HIP path and the
CPU oracle receive the tensors this module draws.  Trained weights and the
pages' evaluation data are not available, so every workload is synthetic with
the shapes and value distributions listed in WORKLOADS:

* "gauss_outliers": 0.02 * N(0,1), with 0.1% of entries (Bernoulli(0.001))
  multiplied by 20, then rounded to fp16;
* "student_t5": 0.015 * t(5) + 0.003, t(5) = z0 / sqrt(sum_{i=1..5} z_i^2 / 5)
  from six standard normals (heavy, asymmetric tails);
* "gauss": 0.02 * N(0,1);
* activations x ~ N(0,1) in fp16.

Draws are fp32 from a seeded torch.Generator on the requested device, then
rounded to fp16 (round-to-nearest-even).
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Tuple

import torch


@dataclass(frozen=True)
class Layer:
    """One linear layer: y[b, n] = sum_k W[n, k] x[b, k]."""

    name: str
    n: int
    k: int
    fmt: str
    group: int
    dist: str
    seed_w: int


@dataclass(frozen=True)
class Workload:
    name: str
    layers: Tuple[Layer, ...]
    batches: Tuple[int, ...]
    seed_x: int


def _llama3_8b_stack() -> Tuple[Layer, ...]:
    """32 decoder layers of q/k/v/o and gate/up/down plus lm_head, Llama-3-8B
    shapes; layers 0, 1, 30, 31 and lm_head in INT8 per channel, the rest INT4
    g128 (selective up-precision of the first and last layers)."""
    mods = (("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
            ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336))
    layers = []
    for li in range(32):
        hi = li in (0, 1, 30, 31)
        for mi, (m, n, k) in enumerate(mods):
            fmt, g = ("int8", k) if hi else ("int4_asym", 128)
            layers.append(Layer(f"l{li}.{m}", n, k, fmt, g, "gauss", 5000 + 16 * li + mi))
    layers.append(Layer("lm_head", 128256, 4096, "int8", 4096, "gauss", 5000 + 16 * 32))
    return tuple(layers)


WORKLOADS = {
    "int4_4096x4096": Workload(
        "int4_4096x4096",
        (Layer("linear", 4096, 4096, "int4_asym", 128, "gauss_outliers", 1001),), (1,), 2001),
    "razer_11008x4096": Workload(
        "razer_11008x4096",
        (Layer("linear", 11008, 4096, "fp4_razer", 128, "gauss_outliers", 1002),), (1, 8), 2002),
    "afpq_28672x8192": Workload(
        "afpq_28672x8192",
        (Layer("linear", 28672, 8192, "fp4_afpq", 64, "student_t5", 1003),), (1, 4, 16), 2003),
    "bfp6_13824x5120": Workload(
        "bfp6_13824x5120",
        (Layer("linear", 13824, 5120, "bfp6", 16, "gauss", 1004),), (16, 32, 64), 2004),
    "bfp4_13824x5120": Workload(
        "bfp4_13824x5120",
        (Layer("linear", 13824, 5120, "bfp4", 16, "gauss", 1004),), (16, 32, 64), 2004),
    "llama3_8b_decode_stack": Workload(
        "llama3_8b_decode_stack", _llama3_8b_stack(), (1, 8, 32, 64), 6000),
}


def weights(layer: Layer, device="cpu", rows=None) -> torch.Tensor:
    """fp16 [n, k] weights of ``layer`` (or the rows in ``rows``, a slice of
    row indices, drawn from the same full-matrix stream)."""
    gen = torch.Generator(device=device).manual_seed(layer.seed_w)
    shape = (layer.n, layer.k)
    if layer.dist in ("gauss", "gauss_outliers"):
        w = torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * 0.02
        if layer.dist == "gauss_outliers":
            mask = torch.rand(shape, generator=gen, device=device, dtype=torch.float32) < 0.001
            w = torch.where(mask, w * 20.0, w)
    elif layer.dist == "student_t5":
        z0 = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        chi = torch.zeros(shape, device=device, dtype=torch.float32)
        for _ in range(5):
            zi = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
            chi += zi * zi
        w = 0.015 * (z0 / torch.sqrt(chi / 5.0)) + 0.003
    else:
        raise ValueError(layer.dist)
    w = w.to(torch.float16)
    return w if rows is None else w[rows]


def activations(b: int, k: int, seed: int, device="cpu") -> torch.Tensor:
    """fp16 [b, k] activations ~ N(0, 1)."""
    gen = torch.Generator(device=device).manual_seed(seed)
    return torch.randn((b, k), generator=gen, device=device, dtype=torch.float32).to(torch.float16)


def small_weights(n: int, k: int, seed: int, dist: str = "gauss_outliers", device="cpu") -> torch.Tensor:
    """fp16 [n, k] weights of a named distribution for small parity cases."""
    return weights(Layer("small", n, k, "", 0, dist, seed), device=device)
