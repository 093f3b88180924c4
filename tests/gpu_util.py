"""Helpers for the GPU parity tests: oracle references and comparisons."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from dequant_gemv_rtn_amd import binding

BUFS = ("codes", "codes_hi", "scales", "aux")


def device():
    return torch.device("cuda", 0)


def oracle_buffers(fmt: str, w16: np.ndarray, group: int):
    """Oracle quantization and its buffers as device bytes (zero-padded)."""
    q = oracle.quantize(fmt, w16, group)
    n, k = w16.shape
    return q, oracle.device_bytes(fmt, n, k, group, oracle.pack(q))


def gpu_buffers(qw: binding.QWeight, rows=None):
    """Packed buffers copied to host: whole (with their padding), or only the
    packed bytes of the given rows."""
    logical = oracle.packed_nbytes(qw.fmt, qw.n, qw.k, qw.group)
    out = {}
    for name in BUFS:
        t = qw.buffers[name]
        if t is None:
            out[name] = None
            continue
        a = t.cpu().numpy()
        if rows is not None:
            a = a[: logical[name]]
            per_row = a.size // qw.n
            a = a.reshape(qw.n, per_row)[rows].reshape(-1)
        out[name] = a
    return out


def assert_packed_equal(got: dict, ref: dict, what: str):
    for name in BUFS:
        g, r = got[name], ref[name]
        if r is None:
            continue
        assert g is not None and g.size == r.size, f"{what}: {name} size {None if g is None else g.size} != {r.size}"
        if not np.array_equal(g, r):
            bad = np.flatnonzero(g != r)
            raise AssertionError(f"{what}: {name} differs at {bad.size} bytes, first at {bad[:8].tolist()}: "
                                 f"got {g[bad[:8]].tolist()} want {r[bad[:8]].tolist()}")


def check_tolerance(y: np.ndarray, y_ref: np.ndarray, deq: np.ndarray, x: np.ndarray, what: str):
    """Per batch row: relative L2 error <= 1e-3; per element:
    |y - y_ref| <= 1e-2 * ||x_b||_2 * max_k |W_deq[n, k]|."""
    y = y.astype(np.float64)
    x64 = x.astype(np.float64)
    rowmax = np.abs(deq).max(axis=1)
    for b in range(y.shape[0]):
        err = y[b] - y_ref[b]
        nref = np.linalg.norm(y_ref[b])
        if nref > 0:
            rel = np.linalg.norm(err) / nref
            assert rel <= 1e-3, f"{what}: batch row {b} relative L2 error {rel:.3e}"
        bound = 1e-2 * np.linalg.norm(x64[b]) * rowmax
        over = np.abs(err) > bound
        if over.any():
            i = int(np.flatnonzero(over)[0])
            raise AssertionError(f"{what}: batch row {b} output {i}: |{y[b, i]} - {y_ref[b, i]}| > {bound[i]}")


def awkward_rows(w: np.ndarray, rng, extremes: bool = True, tiny: bool = True) -> np.ndarray:
    """Overwrite a few rows with degenerate content: zeros, a constant, tiny
    subnormals, fp16 extremes, -0.0, values on power-of-two midpoints.
    ``extremes`` False keeps outputs inside fp16 range; ``tiny`` False skips
    the subnormal row (outside the MFMA path's fp16 operand range)."""
    w = w.copy()
    n, k = w.shape
    if n >= 8:
        w[0] = 0
        w[1] = np.float16(0.03125)
        if tiny:
            w[2] = np.float16(2.0 ** -24) * rng.integers(-3, 4, size=k)
        w[3, ::2] = np.float16(-0.0)
        if extremes:
            w[4, 0], w[4, 1] = np.float16(60000), np.float16(-60000)
        mids = np.array([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 4.5, 5, 5.5, 7, -5, -4.5, 0.5, 1.5, 15, -7, 8, 3, -3, -6])
        w[5] = np.resize(mids * 2.0 ** -6, k).astype(np.float16)
        w[6] = np.resize(np.arange(-7.5, 8.5, 0.5) * 2.0 ** -5, k).astype(np.float16)
    return w
