"""The allocation-free product (q_gemm_skinny_noalloc), called through the
C ABI: it must give exactly what q_gemm_skinny_ws gives with a caller-owned
workspace (the same kernels and K-split plan run on the library's static
scratch), on two calls in a row, the second with a smaller input, so that
what the first call left in the scratch cannot leak into the second.  A
call that needs no workspace (b = 1) runs as q_gemm_skinny."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
from dequant_gemv_rtn_amd import binding, synth
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

Q_OK = 0


def _ws_call(qw, x, y, ws):
    d = qw.desc()
    st = binding.lib().q_gemm_skinny_ws(ctypes.byref(d), ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                        x.shape[0], ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == Q_OK, binding.strerror(st)


def _noalloc_call(qw, x, y):
    d = qw.desc()
    st = binding.lib().q_gemm_skinny_noalloc(ctypes.byref(d), ctypes.c_void_p(x.data_ptr()),
                                             ctypes.c_void_p(y.data_ptr()), x.shape[0],
                                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == Q_OK, binding.strerror(st)


def test_noalloc_equals_workspace_call_twice_then_smaller():
    dev = U.device()
    big = synth.Layer("big", 11008, 4096, "fp4_razer", 128, "gauss_outliers", 1002)     # 22.5 MiB
    small = synth.Layer("small", 1536, 5120, "bfp4", 16, "gauss", 1004)
    cases = [(big, 64), (big, 24), (small, 40), (small, 9)]  # each call smaller than the one before
    qws, w16s = {}, {}
    for layer in (big, small):
        w = synth.weights(layer, device=dev)
        qws[layer.name] = binding.pack(w, layer.fmt, layer.group)
        w16s[layer.name] = w.cpu().numpy()
        del w
    for i, (layer, b) in enumerate(cases):
        qw = qws[layer.name]
        need = binding.workspace_bytes(qw, b)
        assert 0 < need <= (64 << 20), (layer.name, b, need)
        x = synth.activations(b, layer.k, 2000 + i, device=dev)
        y_ref = torch.full((b, layer.n), float("nan"), dtype=torch.float16, device=dev)
        ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=dev)
        assert ws.numel() * ws.element_size() == need  # the K-split form runs in both calls
        _ws_call(qw, x, y_ref, ws)
        y = torch.full((b, layer.n), float("nan"), dtype=torch.float16, device=dev)
        _noalloc_call(qw, x, y)
        torch.cuda.synchronize()
        got, want = y.cpu().numpy(), y_ref.cpu().numpy()
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), f"{layer.name} b={b}"
        # and the product is the right one: sampled rows against the oracle
        rows = np.arange(0, layer.n, max(1, layer.n // 40))
        w16 = w16s[layer.name][rows]
        deq = oracle.dequantize(oracle.quantize(layer.fmt, w16, layer.group))
        y_o = oracle.gemv_f64(deq, x.cpu().numpy())
        U.check_tolerance(got[:, rows], y_o, deq, x.cpu().numpy(), f"noalloc {layer.name} b={b}")


def test_noalloc_without_workspace_runs_plain_kernels():
    """b = 1 needs no workspace: the call runs q_gemm_skinny's kernel."""
    dev = U.device()
    layer = synth.Layer("l", 4096, 4096, "int4_asym", 128, "gauss_outliers", 1001)
    qw = binding.pack(synth.weights(layer, device=dev), layer.fmt, layer.group)
    assert binding.workspace_bytes(qw, 1) == 0
    x = synth.activations(1, layer.k, 2001, device=dev)
    y_ref = binding.gemm_skinny(qw, x)
    y = torch.empty_like(y_ref)
    _noalloc_call(qw, x, y)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
