#!/usr/bin/env python3
"""Benchmark of the fused-dequantization GEMV on one MI355X.

Default line: the Llama-3-8B-shaped decode step (32 decoder layers of
q|k|v, o, gate|up and down plus the 128256-row output head; INT4 g128 with
INT8 per-channel first/last two layers and head), weights packed once and
resident in HBM.  One step is every quantized linear of one decode step.
The headline is batch 1 with the stages in dependency order, as a decoder
runs them: the faster of 129 launches replayed as one HIP graph and one
launch of the decode-stack kernel whose stages wait for each other
(Q_STACK_CHAIN).  Reported alongside: both forms, the one-launch kernel with
its stages free (an upper bound a decoder cannot reach), the step at batch
8 / 32 / 64 (129 launches through the streaming MFMA kernels), and the RaZeR
11008x4096 and AFPQ 28672x8192 layers at batch 1.  Warmup steps run first;
then exactly --steps steps are timed between HIP events on the launch
stream, bracketed by torch.cuda.synchronize().

Prints one JSON line: metric, value (TB/s of algorithmic bytes per step),
the roofline of the headline form against 8 TB/s (with the HBM traffic the
committed counter summary measured for it), and the CPU oracle timed on the
host cores, composed per distinct (shape, format) of the step.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "dequant_gemv_rtn_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
METRIC = "W4A16 fused-dequant GEMV achieved HBM TB/s (% peak) + layer tok/s, batch 1-64"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


KERNEL_FILES = {
    "valu": ["common.hpp", "internal.hpp", "api.hip", "valu_dot.hpp", "gemv_valu.hip"],
    "stream": ["common.hpp", "internal.hpp", "api.hip", "gemm_stream.hip", "gemm_stream_geom.hpp",
               "gemm_stream_kernels.hpp"],
    "stack": ["common.hpp", "internal.hpp", "api.hip", "valu_dot.hpp", "stack.hip"],
}


def kernel_source_digest(kind: str) -> str:
    """sha256 over the sources of one kernel family (the b <= 8 vector-ALU
    GEMV, the streaming MFMA kernels, or the one-launch decode stack), to tell
    whether stored counter readings still describe the kernel being timed."""
    import hashlib

    h = hashlib.sha256()
    for name in KERNEL_FILES[kind]:
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    with open(os.path.join(ROOT, "include", "qgemv.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(profile: str, kind: str):
    """HBM bytes per launch from the committed counter summary
    profiles/<profile>.md, or None when there is none or the kernel sources
    changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{profile}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_digest") != kernel_source_digest(kind):
        return None
    try:
        return int(fields["hbm_traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def calibrate_copy(mib: int, reps: int):
    """A plain device-to-device copy of known size, for scaling the read and
    write byte counters (run under rocprofv3 --pmc)."""
    import torch

    n = mib * 2 ** 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy-calibration", "bytes_read": n, "bytes_written": n, "reps": reps}), flush=True)


def algorithmic_bytes(qw, b: int) -> int:
    """Packed codes + metadata + activations + outputs of one call."""
    return qw.nbytes() + b * qw.k * 2 + b * qw.n * 2


def time_gpu(qws, xs, b, steps, warmup, binding, torch):
    """Average duration of one launch: `steps` back-to-back launches (rotating
    over the weight copies) recorded in a HIP graph and replayed between two
    HIP events on the replay stream, so that host launch cost (a ctypes call
    takes several microseconds) stays out of the figure."""
    ys = [torch.empty((b, qws[0].n), dtype=torch.float16, device=xs.device) for _ in range(2)]
    ws = torch.empty(binding.workspace_bytes(qws[0], b), dtype=torch.uint8, device=xs.device)
    R = len(qws)
    for i in range(warmup):
        binding.gemm_skinny(qws[i % R], xs, out=ys[i & 1], workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            binding.gemm_skinny(qws[(warmup + i) % R], xs, out=ys[i & 1], workspace=ws)
    torch.cuda.synchronize()
    graph.replay()  # warm replay
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end)
    del graph
    return ms / steps, wall


def time_fp16_linear(layer, x, steps, warmup, rotate_mib, torch, synth):
    """Context row, not a target: torch's fp16 x @ W^T (hipBLASLt) on the
    same shape with the unquantized weights, cache-cold like the quantized
    call (rotated copies), timed the same way (graph replay between HIP
    events; eager launches if the library call cannot be captured)."""
    w0 = synth.weights(layer, device=x.device)
    per = w0.numel() * 2
    R = max(2, -(-rotate_mib * 2 ** 20 // per))
    ws = [w0] + [w0.clone() for _ in range(R - 1)]
    y = torch.empty((x.shape[0], layer.n), dtype=torch.float16, device=x.device)
    for i in range(warmup):
        torch.matmul(x, ws[i % R].t(), out=y)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    mode = "graph"
    try:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                torch.matmul(x, ws[(warmup + i) % R].t(), out=y)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        start.record(stream)
        graph.replay()
        end.record(stream)
        torch.cuda.synchronize()
        del graph
    except RuntimeError as e:  # capture not supported by this library build
        log(f"fp16 linear: graph capture failed ({e}); timing eager launches")
        mode = "eager"
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(steps):
            torch.matmul(x, ws[i % R].t(), out=y)
        end.record(stream)
        torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    nbytes = per + x.numel() * 2 + y.numel() * 2
    del ws, w0
    torch.cuda.empty_cache()
    return {"us_per_call": round(ms * 1e3, 3), "bytes_per_call": nbytes,
            "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1), "rotated_copies": R, "timing": mode}


def time_launches(st, b, steps, warmup, torch):
    """The step as separate launches (one per entry of the stack, q|k|v and
    gate|up fused): recorded in a HIP graph once, replayed `steps` times
    between HIP events after `warmup` replays."""
    g = st.capture(b)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    del g
    return start.elapsed_time(end) / steps


def time_one_launch(plan, steps, warmup, chain, torch):
    """The step as one launch of the decode-stack kernel: `warmup` launches,
    then exactly `steps` launches between HIP events on the launch stream
    (the kernel runs for about a millisecond, so the host's launch calls keep
    well ahead of it)."""
    for _ in range(warmup):
        plan.run(chain=chain)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        plan.run(chain=chain)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


def batch_entry(us, nbytes, b):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us_per_step": round(us, 2), "tok_per_s": round(b / (us * 1e-6), 1), "bytes_per_step": nbytes,
            "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def stack_members(st, synth):
    """Source layers of each entry of a fused DecodeStack (q|k|v, gate|up)."""
    by_name = {l.name: l for l in st.workload.layers}
    out = []
    for layer, _ in st.layers:
        if "." in layer.name:
            prefix, _, mods = layer.name.rpartition(".")
            out.append([by_name[f"{prefix}.{m}"] for m in mods.split("_")])
        else:
            out.append([by_name[layer.name]])
    return out


def stack_cpu_baseline(st, x_host_by_k, target_s, torch, synth):
    """The oracle timed on the host cores, composed as the step's distinct
    (shape, format) pairs, each timed once on a sample of its rows and summed
    with multiplicities (the oracle's cost is the same for every row of a
    matrix): the fp64 product (unpack + dequantize + fp64 GEMV) per step, and,
    reported beside it, the one-time RTN quantize + pack of the whole stack.
    Rows are the same fp16 weights the GPU packs."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    dev = st.device
    groups = {}
    for (layer, qw), members in zip(st.layers, stack_members(st, synth)):
        key = (layer.n, layer.k, layer.fmt, layer.group)
        groups.setdefault(key, [0, members])[0] += 1
    per_shape = target_s / max(1, len(groups)) / 2
    total_gemv = total_quant = 0.0
    detail = []
    t_all = time.perf_counter()
    for (n, k, fmt, group), (mult, members) in groups.items():
        w = torch.cat([synth.weights(m, device=dev) for m in members], dim=0)
        probe = min(n, 32)
        w_host = w[:probe].cpu().numpy()
        x = x_host_by_k[k]

        def run(w16):
            r = w16.shape[0]
            t0 = time.perf_counter()
            q = oracle.quantize(fmt, w16, group)
            buf = oracle.pack(q)
            t1 = time.perf_counter()
            deq = oracle.dequantize(oracle.unpack(fmt, r, k, group, buf))
            y = oracle.gemv_f64(deq, x)
            t2 = time.perf_counter()
            assert y.shape == (x.shape[0], r)
            return t1 - t0, t2 - t1

        tq, tg = run(w_host)
        rows = int(min(n, max(probe, probe * per_shape / max(tq + tg, 1e-6))))
        if rows > probe:
            w_host = w[:rows].cpu().numpy()
            tq, tg = run(w_host)
        del w
        per_row_q, per_row_g = tq / rows, tg / rows
        total_gemv += per_row_g * n * mult
        total_quant += per_row_q * n * mult
        detail.append(f"{fmt} {n}x{k} x{mult}: {rows} rows")
    nbytes = st.step_bytes(1)
    return {
        "value": round(nbytes / total_gemv / 1e12, 9),
        "unit": "TB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": ("composed: each distinct (shape, format) of the step timed once on a sample of its rows "
                   "(unpack + fp64 dequantize + fp64 product, batch 1) and summed with multiplicities -- "
                   + "; ".join(detail) + f"; {time.perf_counter() - t_all:.1f} s of host time (numpy; BLAS pool "
                   f"of {blas_threads} threads, {len(os.sched_getaffinity(0))} cores visible; the quantizer is "
                   "single-threaded numpy)"),
        "s_per_step": round(total_gemv, 3),
        "tok_per_s": round(1.0 / total_gemv, 4),
        "quantize_pack_s_whole_stack": round(total_quant, 1),
    }


def single_layer(name, b, steps, warmup, rotate_mib, torch, binding, synth):
    """One layer workload at batch b, cache-cold (rotated copies), as in the
    sweep; returns its figures and the packed weights' first copy."""
    wl = synth.WORKLOADS[name]
    layer = wl.layers[0]
    dev = torch.device("cuda", 0)
    w = synth.weights(layer, device=dev)
    qw0 = binding.pack(w, layer.fmt, layer.group)
    del w
    R = max(2, -(-rotate_mib * 2 ** 20 // qw0.nbytes()))
    qws = [qw0] + [binding.QWeight(layer.fmt, layer.n, layer.k, layer.group, device=dev,
                                   buffers={k: (None if v is None else v.clone()) for k, v in qw0.buffers.items()})
                   for _ in range(R - 1)]
    x = synth.activations(b, layer.k, wl.seed_x + b, device=dev)
    ms, _ = time_gpu(qws, x, b, steps, warmup, binding, torch)
    nbytes = algorithmic_bytes(qw0, b)
    gbs = nbytes / (ms * 1e-3) / 1e9
    del qws
    torch.cuda.empty_cache()
    return {"format": layer.fmt, "n": layer.n, "k": layer.k, "group": layer.group, "batch": b,
            "us_per_call": round(ms * 1e3, 3), "bytes_per_call": nbytes, "GB/s": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "tok_per_s": round(b / (ms * 1e-3), 1),
            "rotated_copies": R}


def fp16_step_context(st, steps, warmup, torch, synth):
    """Context, not a target: the same step with the unquantized fp16
    weights through torch's x @ W^T (hipBLASLt), 129 matmuls recorded in a
    graph -- the MI355X analogue of the pages' speedup over FP16.  About 15
    GB of fp16 weights, which the step streams (naturally cache-cold)."""
    dev = st.device
    ws = [torch.cat([synth.weights(m, device=dev) for m in members], dim=0) for members in stack_members(st, synth)]
    xs = {k: torch.randn((1, k), device=dev).half() for k in {w.shape[1] for w in ws}}
    ys = [torch.empty((1, w.shape[0]), dtype=torch.float16, device=dev) for w in ws]

    def step():
        for w, y in zip(ws, ys):
            torch.matmul(xs[w.shape[1]], w.t(), out=y)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) / steps * 1e3
    nbytes = sum(w.numel() * 2 + w.shape[1] * 2 + w.shape[0] * 2 for w in ws)
    del g, ws
    torch.cuda.empty_cache()
    return {"us_per_step": round(us, 1), "bytes_per_step": nbytes, "GB/s": round(nbytes / us / 1e3, 1),
            "timing": "graph of 129 matmuls"}


def sweep(args):
    """Every single-layer workload at each of its batch sizes, cache-cold,
    graph-replay timing as in the main line; one JSON line per case."""
    import torch

    from dequant_gemv_rtn_amd import binding, synth

    binding.lib()
    dev = torch.device("cuda", 0)
    for name, wl in synth.WORKLOADS.items():
        if len(wl.layers) != 1:
            continue
        layer = wl.layers[0]
        w = synth.weights(layer, device=dev)
        qw0 = binding.pack(w, layer.fmt, layer.group)
        del w
        R = max(2, -(-args.rotate_mib * 2 ** 20 // qw0.nbytes()))
        qws = [qw0] + [binding.QWeight(layer.fmt, layer.n, layer.k, layer.group, device=dev,
                                       buffers={k: (None if v is None else v.clone()) for k, v in qw0.buffers.items()})
                       for _ in range(R - 1)]
        torch.cuda.synchronize()
        for b in wl.batches:
            x = synth.activations(b, layer.k, wl.seed_x + b, device=dev)
            ms, _ = time_gpu(qws, x, b, args.steps, args.warmup, binding, torch)
            nbytes = algorithmic_bytes(qw0, b)
            gbs = nbytes / (ms * 1e-3) / 1e9
            print(json.dumps({"workload": name, "format": layer.fmt, "n": layer.n, "k": layer.k, "group": layer.group,
                              "batch": b, "us_per_call": round(ms * 1e3, 3), "bytes_per_call": nbytes,
                              "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                              "tok_per_s": round(b / (ms * 1e-3), 1)}), flush=True)
        del qws, qw0
        torch.cuda.empty_cache()


ATTN_CONFIGS = ((1, 4096), (8, 4096), (32, 4096), (8, 16384), (32, 16384))


def attention(args):
    """Decode attention over a RaZeR-quantized KV cache, Llama-3-8B layer
    shape (32 query heads, 8 KV heads, head_dim 128, group 128), at each
    (batch, sequence length) of ATTN_CONFIGS: cache-cold (rotated cache
    copies), graph replay between HIP events as in the main line.
    Algorithmic bytes = packed K and V (codes + scales + selectors) + q + out.
    One JSON line per configuration."""
    import torch

    from dequant_gemv_rtn_amd import binding

    binding.lib()
    dev = torch.device("cuda", 0)
    Hq, Hkv, D = 32, 8, 128
    gen = torch.Generator(device=dev)
    for B, L in ATTN_CONFIGS:
        gen.manual_seed(7000 + B * 131 + L)
        k16 = (torch.randn((B, Hkv, L, D), generator=gen, device=dev) * 0.5).half()
        v16 = (torch.randn((B, Hkv, L, D), generator=gen, device=dev) * 0.5).half()
        k0, v0 = binding.pack_kv(k16), binding.pack_kv(v16)
        del k16, v16
        per = k0.nbytes() + v0.nbytes()
        R = max(2, -(-args.rotate_mib * 2 ** 20 // per))

        def copy(qw):
            return binding.QWeight(qw.fmt, qw.n, qw.k, qw.group, device=dev,
                                   buffers={kk: (None if t is None else t.clone()) for kk, t in qw.buffers.items()})

        caches = [(k0, v0)] + [(copy(k0), copy(v0)) for _ in range(R - 1)]
        q = (torch.randn((B, Hq, D), generator=gen, device=dev) * 0.5).half()
        lens = torch.full((B,), L, dtype=torch.int32, device=dev)
        outs = [torch.empty_like(q) for _ in range(2)]
        ws = torch.empty(binding.attn_workspace_bytes(B, Hq, Hkv, L), dtype=torch.uint8, device=dev)
        for i in range(args.warmup):
            kq, vq = caches[i % R]
            binding.attn_decode(kq, vq, q, Hkv, L, lens, out=outs[i & 1], workspace=ws)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                kq, vq = caches[(args.warmup + i) % R]
                binding.attn_decode(kq, vq, q, Hkv, L, lens, out=outs[i & 1], workspace=ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        graph.replay()
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / args.steps
        del graph
        nbytes = per + 2 * q.numel() * 2
        gbs = nbytes / (ms * 1e-3) / 1e9
        print(json.dumps({"mode": "kv_attention_decode", "format": "fp4_razer", "group": 128, "batch": B,
                          "seq_len": L, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
                          "us_per_call": round(ms * 1e3, 3), "bytes_per_call": nbytes, "GB/s": round(gbs, 1),
                          "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "tok_per_s": round(B / (ms * 1e-3), 1),
                          "rotated_copies": R, "data": "synthetic"}), flush=True)
        del caches, k0, v0
        torch.cuda.empty_cache()


W8A8_SHAPES = (("lm_head", 128256, 4096), ("ffn_gate_up", 14336, 4096), ("ffn_down", 4096, 14336))
W8A8_BATCHES = (1, 2, 4, 8, 16, 32, 64)


def w8a8(args):
    """The W8A8 product (per-token INT8 activations, INT8 per-channel
    weights, int8 matrix cores) against the W8A16 INT8 product on the same
    packed weights, Llama-3-8B shapes (lm_head and FFN), each batch size of
    W8A8_BATCHES: cache-cold (rotated weight copies), graph replay between
    HIP events as in the main line.  Algorithmic bytes are the same for both:
    packed weight + fp16 activations + fp16 outputs.  At b <= 2 the product
    runs on the vector ALU (dot4, quantizer fused; at b = 2 not on the
    lm_head), up to b = 4 fused on the matrix cores where that applies; the
    other forms are timed beside it (b <= 2: the matrix-core forms,
    QGEMV_W8A8_DOT=0; b <= 4: the two-kernel form, with
    QGEMV_W8A8_FUSE_MAX_B=0 as well).  One JSON line per case."""
    import torch

    from dequant_gemv_rtn_amd import binding

    binding.lib()
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev)
    for name, n, k in W8A8_SHAPES:
        gen.manual_seed(9000 + n + k)
        w = (torch.randn((n, k), generator=gen, device=dev) * 0.02).half()
        qw0 = binding.pack(w, "int8", k)
        del w
        R = max(2, -(-args.rotate_mib * 2 ** 20 // qw0.nbytes()))
        qws = [qw0] + [binding.QWeight("int8", n, k, k, device=dev,
                                       buffers={kk: (None if t is None else t.clone()) for kk, t in qw0.buffers.items()})
                       for _ in range(R - 1)]
        for b in W8A8_BATCHES:
            x = (torch.randn((b, k), generator=gen, device=dev)).half()
            ys = [torch.empty((b, n), dtype=torch.float16, device=dev) for _ in range(2)]
            ws8 = torch.empty(binding.w8a8_workspace_bytes(b, k), dtype=torch.uint8, device=dev)
            ws16 = torch.empty(binding.workspace_bytes(qw0, b), dtype=torch.uint8, device=dev)
            calls = {
                "w8a8": lambda i: binding.gemm_w8a8(qws[i % R], x, out=ys[i & 1], workspace=ws8),
                "w8a16": lambda i: binding.gemm_skinny(qws[i % R], x, out=ys[i & 1], workspace=ws16),
            }
            # other forms of the same product, each forced by its tuning keys
            forms = {}
            if b <= 2:
                forms["w8a8_fused"] = {"QGEMV_W8A8_DOT": 0}
            if b <= 4:
                forms["w8a8_two_kernels"] = {"QGEMV_W8A8_DOT": 0, "QGEMV_W8A8_FUSE_MAX_B": 0}
            for key in forms:
                calls[key] = calls["w8a8"]
            us = {}
            for key, call in calls.items():
                for tk, tv in forms.get(key, {}).items():
                    binding.set_tuning(tk, tv)
                for i in range(args.warmup):
                    call(i)
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    for i in range(args.steps):
                        call(args.warmup + i)
                torch.cuda.synchronize()
                graph.replay()
                torch.cuda.synchronize()
                stream = torch.cuda.current_stream()
                start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                start.record(stream)
                graph.replay()
                end.record(stream)
                torch.cuda.synchronize()
                us[key] = start.elapsed_time(end) / args.steps * 1e3
                del graph
                for tk in forms.get(key, {}):
                    binding.clear_tuning(tk)
            nbytes = algorithmic_bytes(qw0, b)
            gbs = nbytes / (us["w8a8"] * 1e-6) / 1e9
            extra = {f"us_{key}": round(us[key], 3) for key in forms}
            print(json.dumps({"mode": "w8a8", "layer": name, "n": n, "k": k, "batch": b,
                              "us_w8a8": round(us["w8a8"], 3), **extra, "us_w8a16_int8": round(us["w8a16"], 3),
                              "speedup_vs_w8a16": round(us["w8a16"] / us["w8a8"], 3), "bytes_per_call": nbytes,
                              "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                              "rotated_copies": R, "data": "synthetic"}), flush=True)
        del qws, qw0
        torch.cuda.empty_cache()


BATCHED_SHAPES = (("bfp4_13824x5120", "bfp4", 13824, 5120, 16), ("bfp6_13824x5120", "bfp6", 13824, 5120, 16),
                  ("int4_gate_up_28672x4096", "int4_asym", 28672, 4096, 128),
                  ("int4_down_4096x14336", "int4_asym", 4096, 14336, 128),
                  ("int8_gate_up_28672x4096", "int8", 28672, 4096, 4096),
                  ("int8_down_4096x14336", "int8", 4096, 14336, 14336))
BATCHED_BATCHES = (16, 32, 64)


def batched(args):
    """The batched path (q_gemm_skinny with a workspace: the streaming or
    K-split MFMA form) on the block-format layers of the decode-stack
    benchmark (BFP4/BFP6 13824 x 5120) and on the decode stack's fused
    gate|up and down shapes in INT4 (groups of 128) and INT8, at b = 16, 32,
    64: cache-cold (rotated weight copies), graph replay between HIP events.
    One JSON line per case."""
    import torch

    from dequant_gemv_rtn_amd import binding

    binding.lib()
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev)
    only = [v for v in args.batched_layers.split(",") if v]
    sizes = [int(v) for v in args.batched_batches.split(",") if v] or list(BATCHED_BATCHES)
    for name, fmt, n, k, g in BATCHED_SHAPES:
        if only and name not in only:
            continue
        gen.manual_seed(9100 + n + k)
        w = (torch.randn((n, k), generator=gen, device=dev) * 0.02).half()
        qw0 = binding.pack(w, fmt, g)
        del w
        R = max(2, -(-args.rotate_mib * 2 ** 20 // qw0.nbytes()))
        qws = [qw0] + [binding.QWeight(fmt, n, k, g, device=dev,
                                       buffers={kk: (None if t is None else t.clone()) for kk, t in qw0.buffers.items()})
                       for _ in range(R - 1)]
        for b in sizes:
            x = torch.randn((b, k), generator=gen, device=dev).half()
            ys = [torch.empty((b, n), dtype=torch.float16, device=dev) for _ in range(2)]
            ws = torch.empty(max(1, binding.workspace_bytes(qw0, b)), dtype=torch.uint8, device=dev)
            for i in range(args.warmup):
                binding.gemm_skinny(qws[i % R], x, out=ys[i & 1], workspace=ws)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(args.steps):
                    binding.gemm_skinny(qws[(args.warmup + i) % R], x, out=ys[i & 1], workspace=ws)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            stream = torch.cuda.current_stream()
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            start.record(stream)
            graph.replay()
            end.record(stream)
            torch.cuda.synchronize()
            us = start.elapsed_time(end) / args.steps * 1e3
            del graph
            nbytes = algorithmic_bytes(qw0, b)
            gbs = nbytes / (us * 1e-6) / 1e9
            print(json.dumps({"mode": "batched", "layer": name, "format": fmt, "n": n, "k": k, "group": g,
                              "batch": b, "us_per_call": round(us, 3), "bytes_per_call": nbytes,
                              "workspace_bytes": binding.workspace_bytes(qw0, b), "GB/s": round(gbs, 1),
                              "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "rotated_copies": R,
                              "data": "synthetic"}), flush=True)
        del qws, qw0
        torch.cuda.empty_cache()


def cpu_baseline(qw, x_host, target_s: float):
    """Time the oracle (unpack + fp64 dequantize + fp64 product) on the
    first rows of the layer; scale to TB/s of the same algorithmic bytes."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    host = qw.to_host()
    logical = oracle.packed_nbytes(qw.fmt, qw.n, qw.k, qw.group)

    def rows_buf(nrows):
        out = {}
        for name, t in host.items():
            if t is None:
                out[name] = None
                continue
            a = t.numpy()[: logical[name]]  # drop the zero padding
            per = a.size // qw.n
            sub = a.reshape(qw.n, per)[:nrows].reshape(-1)
            dt = {"codes": np.uint32, "codes_hi": np.uint32, "aux": np.uint32,
                  "scales": np.float16}[name]
            if qw.fmt == "int8" and name == "codes":
                dt = np.int8
            if qw.fmt in ("bfp6", "bfp4") and name == "aux":
                dt = np.uint8
            out[name] = sub.view(dt).reshape(nrows, -1)
        return out

    def run(nrows, reps=1):
        buf = rows_buf(nrows)
        t = time.perf_counter()
        for _ in range(reps):
            q = oracle.unpack(qw.fmt, nrows, qw.k, qw.group, buf)
            y = oracle.gemv_f64(oracle.dequantize(q), x_host)
        dt = time.perf_counter() - t
        assert y.shape == (x_host.shape[0], nrows)
        return dt

    probe_rows = min(qw.n, 64)
    dt = run(probe_rows)
    rows = int(min(qw.n, max(probe_rows, probe_rows * target_s / max(dt, 1e-6))))
    if rows >= qw.n // 2:  # half the layer fits the budget: time whole passes
        rows = qw.n
    dt = run(rows)
    reps = 1
    if rows == qw.n and dt < target_s / 2:  # the whole layer is quick: repeat it
        reps = int(min(50, max(1, target_s / max(dt, 1e-6))))
        dt = run(rows, reps)
    b = x_host.shape[0]
    bytes_rows = qw.nbytes() * rows / qw.n + b * qw.k * 2 + b * rows * 2
    return {
        "value": bytes_rows * reps / dt / 1e12,
        "unit": "TB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{rows} of {qw.n} rows x {reps} passes, batch {b}: unpack + fp64 dequantize + fp64 product, "
                  f"{dt:.1f} s (numpy; BLAS pool of {blas_threads} threads, {len(os.sched_getaffinity(0))} cores visible)",
    }


def layer_line(args):
    """The single-layer line (--workload NAME): one fused-dequant call per
    step on a cache-cold layer, with its extra batch sizes, the one-copy cache
    check, the fp16 context and the oracle on a bounded sample."""
    import torch

    from dequant_gemv_rtn_amd import binding, synth

    binding.lib()
    dev = torch.device("cuda", 0)
    wl = synth.WORKLOADS[args.workload]
    layer = wl.layers[0]
    b = args.batch or wl.batches[0]

    w = synth.weights(layer, device=dev)
    qw0 = binding.pack(w, layer.fmt, layer.group)
    torch.cuda.synchronize()
    del w
    per_copy = qw0.nbytes()
    R = max(2, -(-args.rotate_mib * 2 ** 20 // per_copy))
    qws = [qw0]
    for _ in range(R - 1):
        bufs = {k: (None if v is None else v.clone()) for k, v in qw0.buffers.items()}
        qws.append(binding.QWeight(layer.fmt, layer.n, layer.k, layer.group, device=dev, buffers=bufs))
    torch.cuda.synchronize()
    log(f"workload {args.workload}: {layer.fmt} n={layer.n} k={layer.k} g={layer.group}; "
        f"{R} rotated copies x {per_copy / 2 ** 20:.1f} MiB")

    results = {}
    for bb in [b] + [int(v) for v in args.extra_batches.split(",") if v and int(v) != b]:
        x = synth.activations(bb, layer.k, wl.seed_x + bb, device=dev)
        ms, wall = time_gpu(qws, x, bb, args.steps, args.warmup, binding, torch)
        nbytes = algorithmic_bytes(qw0, bb)
        results[bb] = {"ms": ms, "bytes": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9, "wall": wall}
        log(f"batch {bb}: {ms * 1e3:.2f} us/call, {nbytes / 1e6:.2f} MB/call, "
            f"{results[bb]['gbs']:.0f} GB/s, {bb / (ms * 1e-3):.0f} tok/s")

    main_r = results[b]
    ach = main_r["gbs"]
    out = {
        "metric": METRIC,
        "value": round(ach / 1000.0, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_r["ms"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: RaZeR FP4 (E2M1, -0 remapped per group) linear K={layer.k} N={layer.n} "
                        f"g={layer.group}, batch {b}, packed weights cache-cold" if layer.fmt == "fp4_razer" else
                        f"{args.workload}: {layer.fmt} K={layer.k} N={layer.n} g={layer.group}, batch {b}",
            "batch": b,
            "n": layer.n,
            "k": layer.k,
            "format": layer.fmt,
            "group": layer.group,
            "bytes_per_call": main_r["bytes"],
            "tok_per_s": round(b / (main_r["ms"] * 1e-3), 1),
            "accumulate": "f32",
            "rotated_copies": R,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(ach, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(f"gemv_{args.workload}_b{b}", "valu" if b == 1 else "stream"),
        },
        "extra_batches": {str(k): {"us_per_call": round(v["ms"] * 1e3, 3), "GB/s": round(v["gbs"], 1),
                                   "frac_of_peak": round(v["gbs"] / HBM_PEAK_GBS, 4),
                                   "tok_per_s": round(k / (v["ms"] * 1e-3), 1)}
                          for k, v in results.items() if k != b},
    }
    # cache hygiene check: the same launches on one weight copy, which stays
    # in the last-level cache, against the rotated (cache-cold) figure
    x = synth.activations(b, layer.k, wl.seed_x + b, device=dev)
    if not args.no_cache_check:
        hot_ms, _ = time_gpu([qw0], x, b, args.steps, args.warmup, binding, torch)
        out["cache_check"] = {"rotated_us_per_call": round(main_r["ms"] * 1e3, 3),
                              "one_copy_us_per_call": round(hot_ms * 1e3, 3),
                              "note": "one copy stays in the 256 MB last-level cache; the rotated copies do not"}
    if not args.no_fp16_context:
        ctx = time_fp16_linear(layer, x, args.steps, args.warmup, args.rotate_mib, torch, synth)
        ctx["quantized_speedup"] = round(ctx["us_per_call"] / (main_r["ms"] * 1e3), 2)
        out["fp16_linear_context"] = ctx
        log(f"fp16 linear context: {ctx['us_per_call']:.2f} us/call ({ctx['timing']}), "
            f"quantized call {ctx['quantized_speedup']}x faster")
    if not args.no_cpu_baseline:
        x_host = synth.activations(b, layer.k, wl.seed_x + b, device=dev).cpu().numpy()
        out["cpu_baseline"] = cpu_baseline(qw0, x_host, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)




STACK = "llama3_8b_decode_stack"


def stack_line(args):
    """The default line: the Llama-3-8B-shaped decode step (see the module
    docstring)."""
    import torch

    from dequant_gemv_rtn_amd import binding, stack, synth

    binding.lib()
    dev = torch.device("cuda", 0)
    t_build = time.perf_counter()
    st = stack.DecodeStack(synth.WORKLOADS[STACK], device=dev, fused=True)
    log(f"{STACK}: {len(st.layers)} entries, {st.weight_bytes() / 1e9:.3f} GB packed "
        f"({time.perf_counter() - t_build:.1f} s to pack)")
    nbytes1 = st.step_bytes(1)
    # batch 1, the step's stages in dependency order: as one launch whose
    # stages wait for each other, and as 129 launches in stream order
    us_launches = time_launches(st, 1, args.steps, args.warmup, torch) * 1e3
    log(f"b=1 as {len(st.layers)} launches (graph replay): {us_launches:.1f} us/step")
    plan = st.plan(1)
    us_chain, wall_chain = time_one_launch(plan, args.steps, args.warmup, True, torch)
    us_chain *= 1e3
    if plan.aborted():
        raise RuntimeError("a stage wait of the chained launch gave up; the figure is invalid")
    log(f"b=1 one launch, chained stages: {us_chain:.1f} us/step")
    us_free, _ = time_one_launch(plan, args.steps, args.warmup, False, torch)
    us_free *= 1e3
    log(f"b=1 one launch, free stages: {us_free:.1f} us/step")
    batches = {"1": {"launches_129": batch_entry(us_launches, nbytes1, 1),
                     "one_launch_chained": batch_entry(us_chain, nbytes1, 1),
                     "one_launch_free_stages": batch_entry(us_free, nbytes1, 1)}}
    for b in [int(v) for v in args.stack_batches.split(",") if v and int(v) != 1]:
        us = time_launches(st, b, max(3, args.stack_steps), 3, torch) * 1e3
        batches.setdefault(str(b), {})["launches_129"] = batch_entry(us, st.step_bytes(b), b)
        log(f"b={b} as {len(st.layers)} launches: {us:.1f} us/step")
    # the headline keeps the decoder's dependencies: the faster of the two
    # dependent forms
    if us_launches <= us_chain:
        us_head, mode, kind = us_launches, "launches_129", "valu"
        kernel = (f"gemv_valu_kernel (q_gemm_skinny at b = 1), {len(st.layers)} launches per step replayed as one "
                  "HIP graph; achieved and traffic are per step")
        wall = None
    else:
        us_head, mode, kind = us_chain, "one_launch_chained", "stack"
        kernel = "stack_kernel<true> (q_gemv_stack with Q_STACK_CHAIN), one dispatch per step"
        wall = wall_chain
    ach = nbytes1 / (us_head * 1e-6) / 1e9
    out = {
        "metric": METRIC,
        "value": round(ach / 1000.0, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_head / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"{STACK}: Llama-3-8B-shaped decode step at batch 1 -- 32 layers of q|k|v 6144x4096, "
                        "o 4096x4096, gate|up 28672x4096, down 4096x14336, plus lm_head 128256x4096; INT4 "
                        "g128, INT8 per channel for layers 0, 1, 30, 31 and lm_head; weights ~ N(0, 0.02^2) "
                        "packed once and resident in HBM; every stage runs after the one before, as a "
                        "decoder's linears do",
            "batch": 1,
            "entries": len(st.layers),
            "headline_mode": mode,
            "bytes_per_step": nbytes1,
            "tok_per_s": round(1.0 / (us_head * 1e-6), 1),
            "accumulate": "f32",
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(ach, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(f"decode_stack_llama3_8b_b1_{mode}", kind),
            "kernel": kernel,
        },
        "batches": batches,
    }
    if wall is not None:
        out["timed_wall_s"] = round(wall, 4)
    if not args.no_secondary:
        out["secondary"] = {}
        for name in ("razer_11008x4096", "afpq_28672x8192"):
            out["secondary"][f"{name}_b1"] = single_layer(name, 1, 200, 50, args.rotate_mib, torch, binding, synth)
            log(f"secondary {name} b=1: {out['secondary'][f'{name}_b1']['us_per_call']} us/call")
    if not args.no_fp16_context:
        ctx = fp16_step_context(st, max(3, args.stack_steps), 2, torch, synth)
        ctx["quantized_speedup"] = round(ctx["us_per_step"] / us_head, 2)
        out["fp16_step_context"] = ctx
        log(f"fp16 step context: {ctx['us_per_step']} us/step")
    if not args.no_cpu_baseline:
        xs, _, _ = st.io(1)
        x_host = {k: v.cpu().numpy() for k, v in xs.items()}
        out["cpu_baseline"] = stack_cpu_baseline(st, x_host, args.cpu_seconds, torch, synth)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def profile_step(args):
    """Only the step in one form, `--steps` times after `--warmup`: the
    command the committed decode-stack profiles are taken with."""
    import torch

    from dequant_gemv_rtn_amd import binding, stack, synth

    binding.lib()
    st = stack.DecodeStack(synth.WORKLOADS[STACK], device=torch.device("cuda", 0), fused=True)
    if args.profile_step == "launches_129":
        us = time_launches(st, 1, args.steps, args.warmup, torch) * 1e3
    else:
        plan = st.plan(1)
        us, _ = time_one_launch(plan, args.steps, args.warmup, args.profile_step == "one_launch_chained", torch)
        us *= 1e3
    print(json.dumps({"mode": args.profile_step, "steps": args.steps, "us_per_step": round(us, 2),
                      "bytes_per_step": st.step_bytes(1),
                      "kernel_source_digest": kernel_source_digest("valu" if args.profile_step == "launches_129"
                                                                   else "stack")}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=STACK,
                    help=f"{STACK} (default) or a single-layer workload of synth.WORKLOADS")
    ap.add_argument("--batch", type=int, default=None, help="single-layer line: default the workload's first batch")
    ap.add_argument("--rotate-mib", type=int, default=512)
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cache-check", action="store_true",
                    help="single-layer line: skip the one-copy (cache-resident) timing of the same launches")
    ap.add_argument("--no-fp16-context", action="store_true",
                    help="skip the fp16 torch matmuls timed on the same shapes for context")
    ap.add_argument("--no-secondary", action="store_true", help="skip the single-layer secondary lines")
    ap.add_argument("--extra-batches", default="8", help="single-layer line: extra batch sizes reported alongside")
    ap.add_argument("--stack-batches", default="1,8,32,64",
                    help="batch sizes of the step as separate launches, reported alongside")
    ap.add_argument("--stack-steps", type=int, default=20)
    ap.add_argument("--sweep", action="store_true",
                    help="time every single-layer workload at each of its batch sizes (one JSON line each)")
    ap.add_argument("--attn", action="store_true",
                    help="time decode attention over a RaZeR KV cache (one JSON line per configuration)")
    ap.add_argument("--batched", action="store_true",
                    help="time the batched path (b = 16, 32, 64) on the block-format and stack FFN shapes")
    ap.add_argument("--batched-layers", default="", help="--batched: comma-separated layer names (default all)")
    ap.add_argument("--batched-batches", default="", help="--batched: comma-separated batch sizes (default 16,32,64)")
    ap.add_argument("--w8a8", action="store_true",
                    help="time the W8A8 product against the W8A16 INT8 product (one JSON line per case)")
    ap.add_argument("--profile-step", choices=["launches_129", "one_launch_chained", "one_launch_free"],
                    help="only time the decode step in this form (for profiling)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib, 10)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU layout is a design note, "
              "not a measured path.", file=sys.stderr)
        sys.exit(2)
    if args.profile_step:
        profile_step(args)
        return
    if args.sweep:
        sweep(args)
        return
    if args.attn:
        attention(args)
        return
    if args.batched:
        batched(args)
        return
    if args.w8a8:
        w8a8(args)
        return
    if args.workload == STACK:
        stack_line(args)
    else:
        layer_line(args)


if __name__ == "__main__":
    main()
