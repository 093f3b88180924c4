"""The one-launch decode stack (q_stack_plan + q_gemv_stack) on the GPU.

Every entry's output is checked against the oracle's fp64 product on the same
dequantized weights (the benchmark spec's bounds), in both modes (stages free, and
chained with waits), and the two modes must give the same bits (the same
arithmetic runs in both).  Cases cover every format the kernel decodes, group
sizes 32 to 256, rows longer than one unit (k = 14336, INT8 k = 5120), ragged
units (k = 1056), several entries per stage, a chained stack whose stages
read the previous stage's output, repeated launches and graph replays, and
sampled rows of the full Llama-3-8B-shaped step.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from dequant_gemv_rtn_amd import binding, stack, synth
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _layer(name, n, k, fmt, group, dist, seed):
    return synth.Layer(name, n, k, fmt, group, dist, seed)


# (stage, layer): entries of one stage share their activations
MIXED = [
    (0, _layer("a.q", 300, 4096, "int4_asym", 128, "gauss_outliers", 11)),
    (0, _layer("a.k", 77, 4096, "int4_asym", 128, "gauss_outliers", 12)),
    (0, _layer("a.v", 64, 4096, "int4_asym", 128, "gauss_outliers", 13)),
    (1, _layer("b", 129, 14336, "int4_asym", 128, "gauss", 14)),      # 4 units per row, the last half full
    (2, _layer("c", 200, 5120, "int8", 5120, "gauss", 15)),           # 3 INT8 units per row, the last half full
    (3, _layer("d", 96, 1056, "int4_asym", 32, "gauss_outliers", 16)),  # 33 pieces: one ragged unit
    (4, _layer("e", 160, 2048, "fp4_e2m1", 64, "gauss_outliers", 17)),
    (5, _layer("f", 250, 4096, "fp4_razer", 128, "gauss_outliers", 18)),
    (6, _layer("g", 90, 8192, "fp4_afpq", 64, "student_t5", 19)),
    (7, _layer("h", 70, 4096, "fp4_razer", 256, "gauss_outliers", 20)),
    (8, _layer("i", 3000, 1024, "int8", 1024, "gauss", 21)),
    (9, _layer("j", 50, 16384, "fp4_afpq", 32, "student_t5", 22)),   # the largest k
]


def _build(entries_spec, dev, seed_x=300):
    """Packed weights, per-stage activations and NaN-filled outputs."""
    xs, entries, refs = {}, [], []
    for stage, layer in entries_spec:
        w = synth.weights(layer, device=dev)
        qw = binding.pack(w, layer.fmt, layer.group)
        if stage not in xs:
            xs[stage] = synth.activations(1, layer.k, seed_x + stage, device=dev).reshape(-1)
        y = torch.full((layer.n,), float("nan"), dtype=torch.float16, device=dev)
        entries.append((qw, xs[stage], y, stage))
        refs.append((layer, w.cpu().numpy()))
        del w
    return entries, refs


def _check_against_oracle(entries, refs, what):
    for (qw, x, y, _), (layer, w16) in zip(entries, refs):
        deq = oracle.dequantize(oracle.quantize(layer.fmt, w16, layer.group))
        xh = x.cpu().numpy().reshape(1, -1)
        U.check_tolerance(y.cpu().numpy().reshape(1, -1), oracle.gemv_f64(deq, xh), deq, xh,
                          f"{what} {layer.name} {layer.fmt} {layer.n}x{layer.k}")


@pytest.mark.parametrize("chain", [False, True])
def test_stack_every_format_matches_oracle(chain):
    dev = U.device()
    entries, refs = _build(MIXED, dev)
    plan = binding.StackPlan(entries)
    plan.run(chain=chain)
    torch.cuda.synchronize()
    assert not plan.aborted()
    _check_against_oracle(entries, refs, f"chain={chain}")
    # the same products as separate launches, up to fp32 summation order
    for (qw, x, y, _), (layer, _) in zip(entries, refs):
        y1 = binding.gemv(qw, x)
        torch.cuda.synchronize()
        d = (y.float() - y1.float()).abs().max().item()
        assert d <= 2e-3 * max(1.0, y1.float().abs().max().item()), f"{layer.name}: stack vs q_gemv {d}"


def test_stack_modes_give_the_same_bits_and_repeat():
    dev = U.device()
    entries, _ = _build(MIXED, dev)
    plan = binding.StackPlan(entries)
    plan.run(chain=False)
    torch.cuda.synchronize()
    free = [y.clone() for _, _, y, _ in entries]
    for rep in range(3):
        for _, _, y, _ in entries:
            y.fill_(float("nan"))
        plan.run(chain=True)
        torch.cuda.synchronize()
        assert not plan.aborted(), f"launch {rep}: a stage wait gave up"
        for (_, _, y, _), f in zip(entries, free):
            assert torch.equal(y.view(torch.int16), f.view(torch.int16)), f"launch {rep}"


def test_stack_graph_replays():
    """One chained launch recorded in a HIP graph: every replay, with eager
    work in between, gives the eager launch's bits (the stage counters are
    returned to zero by each launch, with no memset node)."""
    dev = U.device()
    entries, _ = _build(MIXED[:6], dev)
    plan = binding.StackPlan(entries)
    plan.run(chain=True)
    torch.cuda.synchronize()
    ref = [y.clone() for _, _, y, _ in entries]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(chain=True)
    for rep in range(3):
        for _, _, y, _ in entries:
            y.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (_, _, y, _), r in zip(entries, ref):
            assert torch.equal(y.view(torch.int16), r.view(torch.int16)), f"replay {rep}"
    assert not plan.aborted()


def test_stack_chained_stages_read_the_previous_output():
    """Stage s + 1 reads stage s's output (x of entry s + 1 is y of entry s):
    under Q_STACK_CHAIN every workgroup must see every row of it.  Outputs
    start as NaN, so a stage that read before its input was complete would
    show it; each stage is checked against the oracle on the input the GPU
    actually produced.  Weights are scaled so values stay near 1."""
    dev = U.device()
    n = 4096
    fmts = [("int4_asym", 128), ("int8", n), ("fp4_razer", 128), ("int4_asym", 64), ("fp4_afpq", 64),
            ("int8", n), ("fp4_e2m1", 128), ("int4_asym", 128)]
    x0 = synth.activations(1, n, 41, device=dev).reshape(-1)
    entries, refs = [], []
    x = x0
    for s, (fmt, g) in enumerate(fmts):
        layer = _layer(f"c{s}", n, n, fmt, g, "gauss", 500 + s)
        w = (synth.weights(layer, device=dev).float() * (0.8 / (0.02 * n ** 0.5))).half()
        qw = binding.pack(w, fmt, g)
        y = torch.full((n,), float("nan"), dtype=torch.float16, device=dev)
        entries.append((qw, x, y, s))
        refs.append((layer, w.cpu().numpy()))
        x = y
    plan = binding.StackPlan(entries)
    for rep in range(2):
        for _, _, y, _ in entries:
            y.fill_(float("nan"))
        plan.run(chain=True)
        torch.cuda.synchronize()
        assert not plan.aborted()
        _check_against_oracle(entries, refs, f"chained launch {rep}")
        for _, _, y, _ in entries:
            assert torch.isfinite(y.float()).all()


def test_stack_full_llama3_step_sampled():
    """The Llama-3-8B-shaped step at b = 1 as one chained launch (129
    entries, INT8 first/last two layers and head, INT4 g128 elsewhere):
    sampled rows of every distinct (shape, format) against the oracle."""
    dev = U.device()
    wl = synth.WORKLOADS["llama3_8b_decode_stack"]
    st = stack.DecodeStack(wl, device=dev, fused=True)
    plan = st.plan(1)
    plan.run(chain=True)
    torch.cuda.synchronize()
    assert not plan.aborted()
    xs, ys, _ = st.io(1)
    by_name = {l.name: l for l in wl.layers}
    rng = np.random.default_rng(5)
    seen = set()
    for (layer, qw), y in zip(st.layers, ys):
        members = [by_name[f"{layer.name.rpartition('.')[0]}.{m}"] for m in layer.name.rpartition(".")[2].split("_")] \
            if "." in layer.name else [by_name[layer.name]]
        key = (layer.n, layer.k, layer.fmt)
        if key in seen and layer.name not in ("l31.down", "lm_head"):
            continue
        seen.add(key)
        w_all = torch.cat([synth.weights(m, device=dev) for m in members], dim=0)
        rows = np.unique(np.concatenate([[0, layer.n - 1], rng.choice(layer.n, size=24, replace=False)]))
        w_rows = w_all[torch.from_numpy(rows).to(dev)].cpu().numpy()
        del w_all
        deq = oracle.dequantize(oracle.quantize(layer.fmt, w_rows, layer.group))
        xh = xs[layer.k].cpu().numpy()
        got = y[0, torch.from_numpy(rows).to(dev)].cpu().numpy().reshape(1, -1)
        U.check_tolerance(got, oracle.gemv_f64(deq, xh), deq, xh, f"stack {layer.name}")
    assert len(seen) == 9  # q|k|v, o, gate|up, down in INT4 and INT8, and the head
