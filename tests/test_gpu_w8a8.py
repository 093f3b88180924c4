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


def _tie_case(n=64, k=256, b=64):
    """A seeded product in which some binary32 outputs (s_x s_w) acc fall on
    an fp16 tie while the unrounded product does not: there a kernel that
    rounds once, straight to fp16, differs from the oracle's two roundings.
    The seed search uses the oracle alone."""
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


@pytest.mark.parametrize("shape", [(64, 256, 64), (1024, 256, 4)], ids=["two_kernels", "fused"])
def test_w8a8_rounds_twice_on_fp16_ties(shape):
    w, x = _tie_case(*shape)
    dev = U.device()
    k = w.shape[1]
    qw = binding.pack(torch.from_numpy(w).to(dev), "int8", k)
    y = binding.gemm_w8a8(qw, torch.from_numpy(x).to(dev)).cpu().numpy()
    q = oracle.quantize("int8", w, k)
    want, _, _, _ = oracle.gemm_w8a8(x, q.codes, q.scales)
    assert np.array_equal(y.view(np.uint16), want.view(np.uint16))


def test_w8a8_hand_worked_cases():
    """The two hand-worked cases of tests/golden/w8a8_examples.json through
    the C ABI: a smoothed row whose second code is 38 from the rounded
    binary32 quotient (39 from the exact one), and a rescale that gives
    588.0 after two binary32 roundings (587.5 after one).  Expected values
    come from the fixture's derivations, recomputed in exact rationals."""
    import json
    import os
    from fractions import Fraction

    from tests.exact import to_f16, to_f32

    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "w8a8_examples.json")))
    dev = U.device()
    k = 64
    # quotient: rows 0 and 1 of W are unit vectors at k = 0 and k = 1 (code 127, scale f16(1/127))
    gq = g["quotient"]
    x = np.zeros((1, k), dtype=np.float16)
    x[0, :2] = gq["x"]
    m = np.ones(k, dtype=np.float32)
    m[0] = np.float32(float(Fraction(gq["smooth"][0])))
    assert Fraction(float(m[0])) == Fraction(gq["smooth"][0])
    w = np.zeros((2, k), dtype=np.float16)
    w[0, 0] = w[1, 1] = 1.0
    q = oracle.quantize("int8", w, k)
    assert q.codes[0, 0] == q.codes[1, 1] == 127 and Fraction(float(q.scales[0])) == to_f16(Fraction(1, 127))
    qw = binding.pack(torch.from_numpy(w).to(dev), "int8", k)
    y = binding.gemm_w8a8(qw, torch.from_numpy(x).to(dev), torch.from_numpy(m).to(dev)).cpu().numpy()
    s, sw = Fraction(gq["s"]), to_f16(Fraction(1, 127))
    for n, code in enumerate(gq["codes"]):
        want = to_f16(to_f32(to_f32(s * sw) * Fraction(127 * code)))
        other = to_f16(to_f32(to_f32(s * sw) * Fraction(127 * gq["codes_exact_quotient"][n])))
        assert Fraction(float(y[0, n])) == want, (n, float(y[0, n]), float(want))
        if n == 1:
            assert want != other
    # rescale
    gr = g["rescale"]
    x = np.zeros((1, k), dtype=np.float16)
    x[0, :len(gr["x"])] = gr["x"]
    sw16 = np.float16(float(Fraction(gr["w_scale"])))
    w = np.zeros((1, k), dtype=np.float16)
    w[0, :len(gr["w_codes"])] = [np.float16(c * float(sw16)) for c in gr["w_codes"]]
    q = oracle.quantize("int8", w, k)  # the packing reproduces the fixture's codes and scale
    assert q.codes[0, :len(gr["w_codes"])].tolist() == gr["w_codes"] and float(q.scales[0]) == float(sw16)
    qw = binding.pack(torch.from_numpy(w).to(dev), "int8", k)
    y = binding.gemm_w8a8(qw, torch.from_numpy(x).to(dev)).cpu().numpy()
    assert float(y[0, 0]) == gr["y"] != gr["y_one_rounding"]


@pytest.mark.parametrize("waves", ["4", "8", "16"])
def test_w8a8_every_workgroup_shape(waves, tune):
    """Each waves-per-workgroup instance (forced), with one to eight steps
    per wave, one workgroup for all batch tiles or one per tile, ragged last
    steps (k mod 128 = 32, 64, 96), partial row tiles,
    grids of fewer than 8 row groups or not a multiple of 8 (plain batch
    tile mapping), and a small grid whose workgroups stride over many tiles
    (XCD-aligned mapping)."""
    tune.set("QGEMV_W8A8_WAVES", waves)
    tune.set("QGEMV_W8A8_FUSE_MAX_B", "0")  # the two-kernel form also at b <= 4
    tune.set("QGEMV_W8A8_DOT", "0")
    for n, k, b in ((45, 4000, 5), (70, 2080, 20), (33, 8128, 40), (129, 1088, 64), (20, 416, 2)):
        _check(n, k, b, seed=int(waves) * 7 + b)
    tune.set("QGEMV_W8A8_WAVES_PER_CU", "1")
    _check(8000, 512, 33, seed=int(waves) + 3)  # 500 tiles over 80 row groups
    if waves == "16":
        _check(64, 16384, 64, seed=5)  # 8 steps per wave: four rounds of weight loads
    tune.set("QGEMV_W8A8_JOINT", "0")  # one workgroup per batch tile where one would serve all
    _check(129, 1088, 64, seed=int(waves) + 9)



# The fused form (one launch, b <= 4): one case per instance, named by the
# waves per workgroup and k-steps per wave its k selects, each with a ragged
# last step (k mod 128 != 0) and a partial last row tile, at every b up to
# the largest the instance takes (b * k / 8 within its prologue's pieces).
FUSED_INSTANCES = [
    ("w4s1", 37, 160, 4),     # 2 steps
    ("w8s1", 50, 608, 4),     # 5 steps
    ("w16s1", 45, 1056, 4),   # 9 steps
    ("w16s2", 33, 2080, 4),   # 17 steps
    ("w16s4", 70, 4128, 3),   # 33 steps
    ("w16s4_b2", 21, 8192, 2),
    ("w16s8", 19, 10272, 1),  # 81 steps
    ("w16s8_max_k", 16, 16384, 1),
]


@pytest.mark.parametrize("name,n,k,bmax", FUSED_INSTANCES, ids=[c[0] for c in FUSED_INSTANCES])
def test_w8a8_fused_every_instance(name, n, k, bmax, tune):
    tune.set("QGEMV_W8A8_DOT", "0")  # b = 1 through the fused form too
    for b in range(1, bmax + 1):
        _check(n, k, b, seed=k + 7 * b)
    _check(n, k, bmax, seed=k + 1, smooth=True)


def test_w8a8_fused_many_tiles_per_workgroup():
    """Workgroups that stride over several tiles: the ring runs M tiles
    ahead and a group's tiles past the last load and store nothing (4.9
    tiles per workgroup at 16 waves and 2 k-steps, 2.4 at 4 waves with two
    tiles in the ring, 2.2 at 16 waves and one k-step), and a layer past the
    fused form's 8 tiles per workgroup (two-kernel form, also exact)."""
    binding.set_tuning("QGEMV_W8A8_DOT", 0)  # b = 1 through the fused form too
    try:
        _check(20000, 4096, 1, seed=3)
        _check(20000, 4096, 4, seed=4)
        _check(40000, 160, 2, seed=5)
        _check(9000, 1056, 3, seed=6)
        _check(40000, 4096, 1, seed=7)
    finally:
        binding.clear_tuning("QGEMV_W8A8_DOT")


def test_w8a8_fused_degenerate_rows():
    """The degenerate rows of test_w8a8_degenerate_activation_rows, four at a
    time through the fused form: zero rows (s = 0), fp16 extremes,
    subnormals, a single non-zero element, exact .5 ties."""
    rng = np.random.default_rng(5)
    k = 1024
    x = _activations(rng, 6, k)
    x[0] = 0
    x[1] = np.where(rng.random(k) < 0.5, 65504.0, -65504.0).astype(np.float16)
    x[2] = (rng.standard_normal(k) * 2.0 ** -20).astype(np.float16)
    x[3] = 0
    x[3, 517] = -3.0
    x[4] = (rng.integers(-254, 255, size=k) / 2.0).astype(np.float16)
    x[4, 0] = 127.0
    _check(70, k, 4, seed=11, x=x[:4])
    binding.set_tuning("QGEMV_W8A8_DOT", 0)  # b <= 2 through the fused form too
    try:
        _check(70, k, 2, seed=12, x=x[4:])
        _check(70, k, 1, seed=13, x=x[1:2])
    finally:
        binding.clear_tuning("QGEMV_W8A8_DOT")
    for b0 in (0, 2, 4):  # and through the dot4 form, two rows at a time
        _check(70, k, 2, seed=14 + b0, x=x[b0:b0 + 2])


def test_w8a8_two_kernel_form_at_small_b(tune):
    """b <= 4 through the two-kernel form: forced (QGEMV_W8A8_FUSE_MAX_B=0),
    and where the fused form does not apply (b * k / 8 past its prologue's
    pieces; more tiles per workgroup than its LDS scale table holds)."""
    tune.set("QGEMV_W8A8_DOT", "0")  # b = 1 not on the vector-ALU form
    _check(100, 16384, 2, seed=21)  # b * k / 8 = 4096 > 2 * 1024
    _check(600000, 32, 1, seed=22)  # 37500 tiles: 37 per workgroup of 4 waves
    tune.set("QGEMV_W8A8_FUSE_MAX_B", "0")
    for b in (1, 2, 4):
        _check(77, 4128, b, seed=23 + b)
        _check(50, 608, b, seed=27 + b, smooth=True)


def test_w8a8_fused_full_size_sampled():
    """The 28672 x 4096 fused gate|up at b = 1 and 4 (fused: 7 tiles per
    workgroup): sampled rows against the oracle, and the fused result equal
    to the two-kernel form's bit for bit."""
    rng = np.random.default_rng(19)
    dev = U.device()
    n, k = 28672, 4096
    w_dev = (torch.randn((n, k), device=dev) * 0.02).half()
    qw = binding.pack(w_dev, "int8", k)
    rows = np.sort(rng.choice(n, size=512, replace=False))
    w_rows = w_dev[torch.from_numpy(rows).to(dev)].cpu().numpy()
    q = oracle.quantize("int8", w_rows, k)
    for b in (1, 4):
        x = _activations(rng, b, k)
        xd = torch.from_numpy(x).to(dev)
        y = binding.gemm_w8a8(qw, xd)  # b = 1: the vector-ALU form
        binding.set_tuning("QGEMV_W8A8_DOT", 0)
        try:
            y1 = binding.gemm_w8a8(qw, xd)  # the fused matrix-core form
            binding.set_tuning("QGEMV_W8A8_FUSE_MAX_B", 0)
            y2 = binding.gemm_w8a8(qw, xd)  # the two-kernel form
        finally:
            binding.clear_tuning("QGEMV_W8A8_FUSE_MAX_B")
            binding.clear_tuning("QGEMV_W8A8_DOT")
        torch.cuda.synchronize()
        assert torch.equal(y, y1) and torch.equal(y, y2)
        want, _, _, _ = oracle.gemm_w8a8(x, q.codes, q.scales)
        got = y.cpu().numpy()[:, rows]
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


# The b = 1 vector-ALU form (w8a8_dot_kernel, the default at b = 1): one
# to eight stages per row (k = 160 .. 16384, ragged: k mod 1024 and
# k mod 4096 != 0), fewer rows than waves and many rows per wave with odd
# stage counts, smoothing, and launch widths; each result bit-exact against
# the oracle and equal to the fused matrix-core form's.

DOT_CASES = [(37, 160), (50, 1056), (100, 4096), (33, 4128), (21, 8192), (300, 10240), (16, 16384),
             (5000, 4096), (3001, 12320), (1, 14336)]


@pytest.mark.parametrize("wpc,p,s", [("12", "4", "2"), ("4", "4", "2"), ("16", "4", "4"), ("8", "2", "2"), ("12", "2", "4")])
def test_w8a8_dot_form(wpc, p, s, tune):
    """Every instance of the dot4 form (2 or 4 KiB per stage, 2 or 4 stages
    in flight) at several launch widths."""
    tune.set("QGEMV_W8A8_DOT_WAVES_PER_CU", wpc)
    tune.set("QGEMV_W8A8_DOT_P", p)
    tune.set("QGEMV_W8A8_DOT_S", s)
    for n, k in DOT_CASES:
        for b in ((1, 2) if k <= 8192 else (1,)):
            _check(n, k, b, seed=n + 3 * k + int(wpc) + b)
    _check(300, 2048, 1, seed=41, smooth=True)
    _check(65, 4128, 1, seed=42, smooth=True)
    _check(40, 16384, 1, seed=43, smooth=True)
    _check(300, 2048, 2, seed=45, smooth=True)
    _check(65, 8192, 2, seed=46, smooth=True)


@pytest.mark.parametrize("walkers", ["1", "2", "4"])
def test_w8a8_dot_split_form(walkers, tune):
    """k > 8192 at b = 1 and 2 (forced for every such k): rows over 5, 6, 7 and 8
    waves (k = 9216, 11264, 14336, 16384; k = 12320 leaves most of the
    seventh wave's slice past k),
    fewer rows than walkers, ragged last batches of 16 rows and rounds of 4,
    1 to 4 walkers per compute unit, smoothing; then the same shapes with
    the split off (one wave per row)."""
    tune.set("QGEMV_W8A8_DOT_WALKERS_PER_CU", walkers)
    tune.set("QGEMV_W8A8_DOT_SPLIT", "1")  # (by default only from k > 12288)
    for n, k in ((37, 9216), (700, 11264), (4096, 14336), (3001, 12320), (5, 16384), (1029, 14336)):
        for b in (1, 2):
            _check(n, k, b, seed=n + k + int(walkers) + b)
    _check(300, 14336, 1, seed=44, smooth=True)
    _check(300, 10240, 2, seed=47, smooth=True)
    _check(33, 16384, 2, seed=48, smooth=True)
    tune.set("QGEMV_W8A8_DOT_SPLIT", "0")
    for n, k in ((37, 9216), (1029, 14336)):
        _check(n, k, 1, seed=n + k + 7)


def test_w8a8_dot_degenerate_rows():
    """b = 1 on the vector-ALU form: a zero row (scale 0, output 0), fp16's
    extremes, subnormals, a single non-zero element and exact .5 ties."""
    rng = np.random.default_rng(6)
    for k in (4128, 14336):
        _dot_degenerate(rng, k)


def _dot_degenerate(rng, k):
    rows = [np.zeros(k, np.float16),
            np.where(rng.random(k) < 0.5, 65504.0, -65504.0).astype(np.float16),
            (rng.standard_normal(k) * 2.0 ** -20).astype(np.float16)]
    one = np.zeros(k, np.float16)
    one[k - 28] = -3.0
    ties = (rng.integers(-254, 255, size=k) / 2.0).astype(np.float16)
    ties[7] = 127.0
    rows += [one, ties]
    for i, xr in enumerate(rows):
        _check(700, k, 1, seed=50 + i, x=xr[None, :])


def test_w8a8_dot_equals_fused_form():
    """The same bits from the dot4 and the matrix-core forms at b = 1 and 2
    on the Llama-3-8B FFN shapes, with and without smoothing."""
    rng = np.random.default_rng(61)
    dev = U.device()
    for n, k, b in ((14336, 4096, 1), (4096, 14336, 1), (14336, 4096, 2), (4096, 14336, 2)):
        qw = binding.pack((torch.randn((n, k), device=dev) * 0.02).half(), "int8", k)
        xd = torch.from_numpy(_activations(rng, b, k)).to(dev)
        for m in (None, torch.from_numpy(rng.uniform(0.25, 4.0, size=k).astype(np.float32)).to(dev)):
            y = binding.gemm_w8a8(qw, xd, m)
            binding.set_tuning("QGEMV_W8A8_DOT", 0)
            try:
                y1 = binding.gemm_w8a8(qw, xd, m)
            finally:
                binding.clear_tuning("QGEMV_W8A8_DOT")
            torch.cuda.synchronize()
            assert torch.equal(y, y1), f"{n}x{k} b={b} smooth={m is not None}"
