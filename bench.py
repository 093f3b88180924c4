#!/usr/bin/env python3
"""Benchmark of the fused-dequantization GEMV on one MI355X.

One step = one pass of the hot path over one batch: a fused-dequant GEMV /
skinny GEMM call on packed weights already resident in HBM (quantization is
the one-shot offline step and runs before timing).  Default workload: the
RaZeR FP4 linear layer K=4096, N=11008, group 128, batch 1.

Timing is cache-cold: R distinct copies of the packed weights (at least
--rotate-mib MiB in total, more than the 256 MiB last-level cache) are
rotated so every call streams its weights from HBM.  The timed launches are
recorded in a HIP graph and replayed; the timed region is bracketed by
torch.cuda.synchronize(), and HIP events on the replay stream give the
average launch duration.

Prints one JSON line: metric, value (TB/s of algorithmic bytes), roofline of
the GEMV kernel against 8 TB/s, and the CPU oracle timed on a bounded sample.
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


def kernel_source_digest(b: int = 1) -> str:
    """sha256 over the sources of the kernel that serves batch size b (the
    vector-ALU GEMV for b = 1, the streaming MFMA kernel otherwise), to tell
    whether stored counter readings still describe the kernel being timed."""
    import hashlib

    files = ["common.hpp", "internal.hpp", "api.hip", "gemv_valu.hip" if b == 1 else "gemm_stream.hip"]
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    with open(os.path.join(ROOT, "include", "qgemv.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, b: int):
    """HBM bytes per launch from the committed counter summary of this
    workload, or None when there is none or the kernel sources changed since
    the counters were taken."""
    path = os.path.join(PROFILES, f"gemv_{workload}_b{b}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_digest") != kernel_source_digest(b):
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


def time_stack(batches, steps, warmup, torch, fused=False):
    """Decode steps of the Llama-3-8B-shaped stack (225 quantized linears,
    INT8 first/last layers and lm_head, INT4 g128 elsewhere), each step one
    replay of a HIP graph holding its launches: 225, or 129 with q|k|v and
    gate|up of each decoder layer fused into one launch each."""
    from dequant_gemv_rtn_amd import stack, synth

    st = stack.DecodeStack(synth.WORKLOADS["llama3_8b_decode_stack"], device="cuda", fused=fused)
    out = {"launches": len(st.layers), "weight_bytes": st.weight_bytes(), "batches": {}}
    for b in batches:
        g = st.capture(b)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(steps):
            g.replay()
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
        nbytes = st.step_bytes(b)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out["batches"][str(b)] = {"us_per_step": round(ms * 1e3, 2), "tok_per_s": round(b / (ms * 1e-3), 1),
                                  "bytes_per_step": nbytes, "GB/s": round(gbs, 1),
                                  "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
        log(f"decode stack{' (fused)' if fused else ''} b={b}: {ms * 1e3:.1f} us/step, {gbs:.0f} GB/s, "
            f"{b / (ms * 1e-3):.0f} tok/s")
        del g
    del st
    torch.cuda.empty_cache()
    return out


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
W8A8_BATCHES = (1, 8, 16, 32, 64)


def w8a8(args):
    """The W8A8 product (per-token INT8 activations, INT8 per-channel
    weights, int8 matrix cores) against the W8A16 INT8 product on the same
    packed weights, Llama-3-8B shapes (lm_head and FFN), each batch size of
    W8A8_BATCHES: cache-cold (rotated weight copies), graph replay between
    HIP events as in the main line.  Algorithmic bytes are the same for both:
    packed weight + fp16 activations + fp16 outputs.  One JSON line per case."""
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
            us = {}
            for key, call in calls.items():
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
            nbytes = algorithmic_bytes(qw0, b)
            gbs = nbytes / (us["w8a8"] * 1e-6) / 1e9
            print(json.dumps({"mode": "w8a8", "layer": name, "n": n, "k": k, "batch": b,
                              "us_w8a8": round(us["w8a8"], 3), "us_w8a16_int8": round(us["w8a16"], 3),
                              "speedup_vs_w8a16": round(us["w8a16"] / us["w8a8"], 3), "bytes_per_call": nbytes,
                              "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                              "rotated_copies": R, "data": "synthetic"}), flush=True)
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="razer_11008x4096")
    ap.add_argument("--batch", type=int, default=None, help="default: the workload's first batch size")
    ap.add_argument("--rotate-mib", type=int, default=512)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cache-check", action="store_true",
                    help="skip the one-copy (cache-resident) timing of the same launches")
    ap.add_argument("--no-fp16-context", action="store_true",
                    help="skip the fp16 torch linear timed on the same shape for context")
    ap.add_argument("--extra-batches", default="8", help="comma list of extra batch sizes reported alongside")
    ap.add_argument("--stack-batches", default="1,8,32,64",
                    help="batch sizes for the decode-stack steps reported alongside ('' to skip)")
    ap.add_argument("--stack-steps", type=int, default=20)
    ap.add_argument("--sweep", action="store_true",
                    help="time every single-layer workload at each of its batch sizes (one JSON line each)")
    ap.add_argument("--attn", action="store_true",
                    help="time decode attention over a RaZeR KV cache (one JSON line per configuration)")
    ap.add_argument("--w8a8", action="store_true",
                    help="time the W8A8 product against the W8A16 INT8 product (one JSON line per case)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib, 10)
        return

    if args.sweep:
        sweep(args)
        return

    if args.attn:
        attention(args)
        return

    if args.w8a8:
        w8a8(args)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU layout is a design note, "
              "not a measured path.", file=sys.stderr)
        sys.exit(2)

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
            "traffic": measured_traffic(args.workload, b),
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
    stack_b = [int(v) for v in args.stack_batches.split(",") if v]
    if stack_b:
        del qws, qw0
        torch.cuda.empty_cache()
        out["decode_stack"] = time_stack(stack_b, args.stack_steps, 3, torch)
        out["decode_stack_fused"] = time_stack(stack_b, args.stack_steps, 3, torch, fused=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
