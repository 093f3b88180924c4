"""Decode-stack dispatch on the GPU: per-layer formats, and one step recorded
into a HIP graph gives the same bits as the eager step on every replay."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from dequant_gemv_rtn_amd import stack, synth
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

MINI = synth.Workload(
    "mini_stack",
    (
        synth.Layer("l0.q", 256, 1024, "int8", 1024, "gauss", 71),
        synth.Layer("l1.q", 320, 1024, "int4_asym", 128, "gauss", 72),
        synth.Layer("l1.down", 128, 2048, "int4_asym", 128, "gauss", 73),
        synth.Layer("l2.razer", 96, 1024, "fp4_razer", 128, "gauss_outliers", 74),
        synth.Layer("l2.afpq", 64, 1024, "fp4_afpq", 64, "student_t5", 75),
        synth.Layer("l2.bfp6", 80, 1024, "bfp6", 16, "gauss", 76),
        synth.Layer("head", 512, 1024, "int8", 1024, "gauss", 77),
    ),
    (1, 8, 16, 64),
    900,
)


@pytest.mark.parametrize("b", MINI.batches)
def test_stack_step_matches_oracle_and_graph_replays(b):
    dev = U.device()
    st = stack.DecodeStack(MINI, device=dev)
    st.step(b)
    torch.cuda.synchronize()
    xs, ys, _ = st.io(b)
    eager = [y.clone() for y in ys]
    for (layer, _), y in zip(st.layers, eager):
        w = synth.weights(layer, device=dev).cpu().numpy()  # same generator as the stack
        deq = oracle.dequantize(oracle.quantize(layer.fmt, w, layer.group))
        x = xs[layer.k].cpu().numpy()
        U.check_tolerance(y.cpu().numpy(), oracle.gemv_f64(deq, x), deq, x, f"{layer.name} b={b}")
    g = st.capture(b)
    for rep in range(3):
        for y in ys:
            y.fill_(7.0)  # eager work between replays; the replay must overwrite it
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (layer, _), y, ref in zip(st.layers, ys, eager):
            assert torch.equal(y, ref), f"replay {rep}: {layer.name} differs from the eager step"
    assert st.step_bytes(b) == sum(qw.nbytes() + 2 * b * qw.k + 2 * b * qw.n for _, qw in st.layers)
    assert np.isfinite(st.weight_bytes())


FUSE_MINI = synth.Workload(
    "fuse_mini",
    tuple(
        synth.Layer(f"l{li}.{m}", n, k, fmt, g, "gauss", 300 + 16 * li + mi)
        for li, (fmt, g) in enumerate((("int8", 512), ("int4_asym", 128)))
        for mi, (m, n, k) in enumerate((("q", 256, 512), ("k", 64, 512), ("v", 64, 512), ("o", 256, 512),
                                        ("gate", 384, 512), ("up", 384, 512), ("down", 256, 1152 if fmt != "int8" else 512)))
    ),
    (1, 8, 16, 40),
    950,
)


@pytest.mark.parametrize("b", FUSE_MINI.batches)
def test_fused_stack_equals_separate_launches(b):
    """q|k|v and gate|up packed as one matrix and served by one launch give
    the same bits, row for row, as the separate launches."""
    dev = U.device()
    sep = stack.DecodeStack(FUSE_MINI, device=dev)
    fus = stack.DecodeStack(FUSE_MINI, device=dev, fused=True)
    assert len(fus.layers) == len(sep.layers) - 2 * 3
    # the same activations for both: one per k
    xs_sep, ys_sep, _ = sep.io(b)
    xs_fus, ys_fus, _ = fus.io(b)
    for k in xs_sep:
        xs_fus[k].copy_(xs_sep[k])
    sep.step(b)
    fus.step(b)
    torch.cuda.synchronize()
    out_sep = {layer.name: y for (layer, _), y in zip(sep.layers, ys_sep)}
    for (layer, _), y in zip(fus.layers, ys_fus):
        prefix, _, mods = layer.name.rpartition(".")
        parts = [out_sep[f"{prefix}.{m}"] for m in mods.split("_")] if prefix else [out_sep[layer.name]]
        assert torch.equal(y, torch.cat(parts, dim=1)), layer.name
