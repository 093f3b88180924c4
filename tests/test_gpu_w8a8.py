"""GPU parity of the W8A8 product (q_gemm_w8a8) against the oracle.

Every step is integer arithmetic or one IEEE binary32 operation, so the
fp16 outputs must equal the oracle's bit for bit.  The weights are packed on
the device with q_pack; the oracle quantizes the same fp16 weights itself
(the INT8 packing is bit-exact, which the packing tests establish).

Cases: k with a half last 64-element step (k mod 64 = 32), row counts that
leave a partial 16-row tile, b from 1 to 64 (one to four batch tiles, rows
past b), per-input-channel smoothing, zero, extreme and subnormal activation
rows, a workspace full of NaN bytes, and sampled rows of a 128256 x 4096
lm_head.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from dequant_gemv_rtn_amd import binding
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _weights(rng, n, k):
    w = rng.standard_normal((n, k)) * 0.02
    w[rng.random(w.shape) < 0.001] *= 20  # outliers, as in the layer configs
    return w.astype(np.float16)


def _activations(rng, b, k, scale=1.0):
    return (rng.standard_normal((b, k)) * scale).astype(np.float16)


def _check(n, k, b, seed, smooth=False, x=None):
    rng = np.random.default_rng(seed)
    dev = U.device()
    w = _weights(rng, n, k)
    m = rng.uniform(0.25, 4.0, size=k).astype(np.float32) if smooth else None
    if m is not None:  # the caller folds the smoothing factors into the weights
        w = (w.astype(np.float32) * m).astype(np.float16)
    if x is None:
        x = _activations(rng, b, k)
    qw = binding.pack(torch.from_numpy(w).to(dev), "int8", k)
    ws = torch.full((binding.w8a8_workspace_bytes(b, k),), 0xFF, dtype=torch.uint8, device=dev)  # NaN bytes
    y = binding.gemm_w8a8(qw, torch.from_numpy(x).to(dev), None if m is None else torch.from_numpy(m).to(dev),
                          workspace=ws).cpu().numpy()
    q = oracle.quantize("int8", w, k)
    want, acc, _, _ = oracle.gemm_w8a8(x, q.codes, q.scales, m)
    if not np.array_equal(y.view(np.uint16), want.view(np.uint16)):
        bad = np.argwhere(y.view(np.uint16) != want.view(np.uint16))[0]
        raise AssertionError(f"n={n} k={k} b={b} smooth={smooth}: y{tuple(bad)} = {y[tuple(bad)]} vs {want[tuple(bad)]} "
                             f"(acc {acc[tuple(bad)]})")


@pytest.mark.parametrize("n,k", [(37, 160), (50, 1056), (100, 4096), (33, 4128), (21, 8192), (16, 16384), (300, 10240)])
@pytest.mark.parametrize("b", [1, 3, 16, 17, 40, 64])
def test_w8a8_bit_exact(n, k, b):
    _check(n, k, b, seed=n * 131 + k + b)


@pytest.mark.parametrize("b", [2, 33])
def test_w8a8_smoothing(b):
    _check(300, 2048, b, seed=7 + b, smooth=True)
    _check(65, 4128, b, seed=9 + b, smooth=True)


def test_w8a8_degenerate_activation_rows():
    """A zero row (scale 0, output 0), a row at fp16's extremes, a row of
    subnormals, a single non-zero element, and ties of the rounding."""
    rng = np.random.default_rng(5)
    k = 1024
    x = _activations(rng, 6, k)
    x[0] = 0
    x[1] = np.where(rng.random(k) < 0.5, 65504.0, -65504.0).astype(np.float16)
    x[2] = (rng.standard_normal(k) * 2.0 ** -20).astype(np.float16)
    x[3] = 0
    x[3, 517] = -3.0
    x[4] = (rng.integers(-254, 255, size=k) / 2.0).astype(np.float16)  # absmax 127 gives s = 1: ties at .5
    x[4, 0] = 127.0
    _check(70, k, 6, seed=11, x=x)


def test_w8a8_repeatable_and_lm_head_sampled():
    """The 128256 x 4096 INT8 lm_head at b = 32: sampled rows against the
    oracle (rows are quantized one by one, so the sample needs only its own
    rows), and a second call giving the same bits."""
    rng = np.random.default_rng(17)
    dev = U.device()
    n, k, b = 128256, 4096, 32
    w_dev = (torch.randn((n, k), device=dev) * 0.02).half()
    qw = binding.pack(w_dev, "int8", k)
    x = _activations(rng, b, k)
    xd = torch.from_numpy(x).to(dev)
    y1 = binding.gemm_w8a8(qw, xd)
    y2 = binding.gemm_w8a8(qw, xd)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    rows = np.sort(rng.choice(n, size=512, replace=False))
    w_rows = w_dev[torch.from_numpy(rows).to(dev)].cpu().numpy()
    q = oracle.quantize("int8", w_rows, k)
    want, _, _, _ = oracle.gemm_w8a8(x, q.codes, q.scales)
    got = y1.cpu().numpy()[:, rows]
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def _tie_case():
    """A seeded product in which some binary32 outputs (s_x s_w) acc fall on
    an fp16 tie while the unrounded product does not: there a kernel that
    rounds once, straight to fp16, differs from the oracle's two roundings.
    The seed search uses the oracle alone."""
    n, k, b = 64, 256, 64
    for seed in range(200):
        rng = np.random.default_rng(1000 + seed)
        w = _weights(rng, n, k)
        x = _activations(rng, b, k)
        q = oracle.quantize("int8", w, k)
        want, acc, _, sx = oracle.gemm_w8a8(x, q.codes, q.scales)
        scale = sx[:, None].astype(np.float32) * q.scales.astype(np.float32)[None, :]
        once = (scale.astype(np.float64) * acc.astype(np.float64)).astype(np.float16)
        if np.count_nonzero(once.view(np.uint16) != want.view(np.uint16)) >= 1:
            return w, x
    raise AssertionError("no fp16 tie in the seeded search")


def test_w8a8_rounds_twice_on_fp16_ties():
    w, x = _tie_case()
    dev = U.device()
    k = w.shape[1]
    qw = binding.pack(torch.from_numpy(w).to(dev), "int8", k)
    y = binding.gemm_w8a8(qw, torch.from_numpy(x).to(dev)).cpu().numpy()
    q = oracle.quantize("int8", w, k)
    want, _, _, _ = oracle.gemm_w8a8(x, q.codes, q.scales)
    assert np.array_equal(y.view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("waves", ["4", "8", "16"])
def test_w8a8_every_workgroup_shape(waves, monkeypatch):
    """Each waves-per-workgroup instance (forced), with one to eight steps
    per wave, one workgroup for all batch tiles or one per tile, ragged last
    steps (k mod 128 = 32, 64, 96), partial row tiles,
    grids of fewer than 8 row groups or not a multiple of 8 (plain batch
    tile mapping), and a small grid whose workgroups stride over many tiles
    (XCD-aligned mapping)."""
    monkeypatch.setenv("QGEMV_W8A8_WAVES", waves)
    for n, k, b in ((45, 4000, 5), (70, 2080, 20), (33, 8128, 40), (129, 1088, 64), (20, 416, 2)):
        _check(n, k, b, seed=int(waves) * 7 + b)
    monkeypatch.setenv("QGEMV_W8A8_WAVES_PER_CU", "1")
    _check(8000, 512, 33, seed=int(waves) + 3)  # 500 tiles over 80 row groups
    if waves == "16":
        _check(64, 16384, 64, seed=5)  # 8 steps per wave: four rounds of weight loads
    monkeypatch.setenv("QGEMV_W8A8_JOINT", "0")  # one workgroup per batch tile where one would serve all
    _check(129, 1088, 64, seed=int(waves) + 9)

