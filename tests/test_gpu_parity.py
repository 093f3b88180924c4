"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

* q_pack output is byte-identical to the oracle's packed buffers;
* q_gemv / q_gemm_skinny meet the tolerance (relative L2 <= 1e-3 per batch
  row, |err| <= 1e-2 * ||x_b|| * max|W_deq[n,:]| per output) for every
  format and for batch sizes that cross both kernels' tile edges;
* in an exact regime (integer activations, scales with few significant bits)
  every output is bit-identical to the oracle's rounded fp64 result;
* full-size workloads (the configurations the benchmark times) match on
  sampled rows: bit-exact packing and tolerance products;
* edge cases: minimum and maximum k, ragged n, zero inputs, determinism.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from dequant_gemv_rtn_amd import binding, synth
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

ALL = ("int4_asym", "fp4_e2m1", "fp4_razer", "fp4_afpq", "bfp6", "bfp4", "int8", "fp3_razer", "fp3_afpq")
AFPQ = ("fp4_afpq", "fp3_afpq")  # heavy-tailed asymmetric weights, groups of 64 by default


def _group(fmt, k, g=128):
    return {"bfp6": 16, "bfp4": 16, "int8": k}.get(fmt, g)


def _weights(n, k, seed, dist="gauss_outliers"):
    return synth.small_weights(n, k, seed, dist).numpy()


def _run(fmt, w16: np.ndarray, g: int, xs: np.ndarray):
    dev = U.device()
    qw = binding.pack(torch.from_numpy(w16).to(dev), fmt, g)
    x = torch.from_numpy(xs).to(dev)
    y = binding.gemm_skinny(qw, x)
    torch.cuda.synchronize()
    return qw, y.cpu().numpy()


# ------------------------------------------------------------- packing --

PACK_CASES = [
    ("int4_asym", 37, 4096, 128), ("int4_asym", 9, 1056, 32), ("int4_asym", 5, 2048, 256), ("int4_asym", 11, 4096, 64),
    ("fp4_e2m1", 37, 4096, 128), ("fp4_e2m1", 9, 1056, 32),
    ("fp4_razer", 37, 4096, 128), ("fp4_razer", 9, 1056, 32), ("fp4_razer", 6, 2048, 256), ("fp4_razer", 10, 1024, 64),
    ("fp4_afpq", 37, 8192, 64), ("fp4_afpq", 9, 1056, 32),
    ("bfp6", 37, 5120, 16), ("bfp6", 9, 1056, 16),
    ("bfp4", 37, 5120, 16), ("bfp4", 9, 1056, 16),
    ("int8", 37, 4096, None), ("int8", 9, 1056, None), ("int8", 3, 16384, None),
    ("fp3_razer", 37, 4096, 128), ("fp3_razer", 9, 1056, 32), ("fp3_razer", 6, 2048, 256), ("fp3_razer", 10, 1024, 64),
    ("fp3_afpq", 37, 8192, 64), ("fp3_afpq", 9, 1056, 32), ("fp3_afpq", 5, 2048, 256),
]


@pytest.mark.parametrize("fmt,n,k,g", PACK_CASES)
def test_pack_bit_exact(fmt, n, k, g):
    g = g or k
    rng = np.random.default_rng(n * 7 + k)
    dist = "student_t5" if fmt in AFPQ else "gauss_outliers"
    w = U.awkward_rows(_weights(n, k, 100 + n, dist), rng)
    qw = binding.pack(torch.from_numpy(w).to(U.device()), fmt, g)
    torch.cuda.synchronize()
    _, ref = U.oracle_buffers(fmt, w, g)
    U.assert_packed_equal(U.gpu_buffers(qw), ref, f"{fmt} {n}x{k} g{g}")



@pytest.mark.parametrize("fmt,n,k,g", PACK_CASES)
def test_dequant_bit_exact(fmt, n, k, g):
    """q_dequant decodes the device-packed buffers to the oracle's W_deq
    rounded once to fp16, bit for bit (every value is exact before that
    rounding on both sides)."""
    g = k if g is None else g
    w = U.awkward_rows(_weights(n, k, 17 * n + k), np.random.default_rng(n + k))
    qw = binding.pack(torch.from_numpy(w).to(U.device()), fmt, g)
    got = binding.dequant(qw).cpu().numpy()
    want = oracle.dequantize(oracle.quantize(fmt, w, g)).astype(np.float16)
    bad = np.flatnonzero(got.view(np.uint16) != want.view(np.uint16))
    assert bad.size == 0, (f"{fmt} {n}x{k} g{g}: {bad.size} values differ, first at {np.unravel_index(bad[0], w.shape)}: "
                           f"{got.flat[bad[0]]} vs {want.flat[bad[0]]}")

# -------------------------------------------------------- tolerance --

BATCHES = (1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 32, 33, 48, 64)


@pytest.mark.parametrize("fmt", ALL)
def test_gemm_tolerance_all_batches(fmt):
    n = 100
    k = 5120 if fmt in ("bfp6", "bfp4") else 4096
    g = _group(fmt, k, 64 if fmt in AFPQ else 128)
    rng = np.random.default_rng(3)
    dist = "student_t5" if fmt in AFPQ else "gauss_outliers"
    w = U.awkward_rows(_weights(n, k, 7, dist), rng, extremes=False, tiny=False)
    deq = oracle.dequantize(oracle.quantize(fmt, w, g))
    dev = U.device()
    qw = binding.pack(torch.from_numpy(w).to(dev), fmt, g)
    for b in BATCHES:
        x = synth.activations(b, k, 1000 + b).numpy()
        y = binding.gemm_skinny(qw, torch.from_numpy(x).to(dev)).cpu().numpy()
        U.check_tolerance(y, oracle.gemv_f64(deq, x), deq, x, f"{fmt} b={b}")


@pytest.mark.parametrize("fmt", ALL)
def test_subnormal_rows(fmt):
    """Rows of fp16-subnormal weights.  The group formats scale in fp32 on
    both paths; the MFMA path of the block formats folds the block step
    relative to the row slice's largest block into fp16 operands and applies
    the rest in fp32, which these rows (every block tiny) exercise."""
    n, k = 16, 1024
    g = _group(fmt, k, 32)
    rng = np.random.default_rng(4)
    w = U.awkward_rows(_weights(n, k, 8), rng, extremes=False, tiny=True)
    deq = oracle.dequantize(oracle.quantize(fmt, w, g))
    for b in (1, 2, 4, 8, 16, 40):
        x = synth.activations(b, k, 77 + b).numpy()
        _, y = _run(fmt, w, g, x)
        U.check_tolerance(y, oracle.gemv_f64(deq, x), deq, x, f"{fmt} b={b} subnormal rows")


# ----------------------------------------------------------- exact regime --

def _exact_weights(fmt, n, k, g, rng):
    """Weights on a coarse grid whose group extremes give scales with few
    significant bits, so every product and partial sum is exact in fp32 and
    every folded fp16 operand is exact."""
    p = 2.0 ** -4
    if fmt == "int4_asym":
        v = rng.integers(-7, 9, size=(n, k)).astype(np.float64)
        v[:, ::g] = -7
        v[:, 1::g] = 8
    elif fmt in ("fp4_e2m1", "fp4_afpq"):
        v = rng.choice([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -2, -3, -4, -6], size=(n, k)).astype(np.float64)
        v[:, ::g] = 6
        v[:, 1::g] = -6
    elif fmt == "fp4_razer":
        v = rng.choice([0, 1, 2, 3, 4, 6, -1, -2, -3, -4, -6], size=(n, k)).astype(np.float64)
        v[:, ::g] = 8  # the +8 candidate represents every value exactly
    elif fmt == "fp3_razer":
        v = rng.choice([0, 1, 2, 4, -1, -2, -4], size=(n, k)).astype(np.float64)
        v[:, ::g] = 8  # the +8 candidate (scale 1) represents every value exactly
    elif fmt == "fp3_afpq":
        v = rng.choice([0, 1, 2, 4, -1, -2, -4], size=(n, k)).astype(np.float64)
        v[:, ::g] = 4
        v[:, 1::g] = -4
    elif fmt in ("bfp6", "bfp4"):
        lim = 31 if fmt == "bfp6" else 7
        v = rng.integers(-lim, lim + 1, size=(n, k)).astype(np.float64) / 4
    else:
        v = rng.integers(-127, 128, size=(n, k)).astype(np.float64)
        v[:, 0] = 127
    return (v * p).astype(np.float16)


@pytest.mark.parametrize("fmt", ALL)
def test_exact_regime_bit_identical(fmt):
    n, k = 70, 2048
    g = _group(fmt, k, 64 if fmt in AFPQ else 128)
    rng = np.random.default_rng(5)
    w = _exact_weights(fmt, n, k, g, rng)
    q = oracle.quantize(fmt, w, g)
    deq = oracle.dequantize(q)
    dev = U.device()
    qw = binding.pack(torch.from_numpy(w).to(dev), fmt, g)
    for b in (1, 3, 8, 9, 16, 40, 64):
        x = rng.integers(-2, 3, size=(b, k)).astype(np.float16)
        y = binding.gemm_skinny(qw, torch.from_numpy(x).to(dev)).cpu().numpy()
        ref = oracle.gemv_f64(deq, x)
        assert np.all(np.abs(ref) < 60000)
        want = ref.astype(np.float16)
        if not np.array_equal(y.view(np.uint16), want.view(np.uint16)):
            bad = np.argwhere(y.view(np.uint16) != want.view(np.uint16))
            bb, nn = bad[0]
            raise AssertionError(f"{fmt} b={b}: {len(bad)} outputs differ; first [{bb},{nn}] {y[bb, nn]} != {want[bb, nn]}")


# ------------------------------------------------------- full-size sampled --

def _sample_rows(n, rng, count=48):
    rows = np.unique(np.concatenate([[0, 1, n - 2, n - 1], rng.choice(n, size=count, replace=False)]))
    return np.sort(rows)


def _full_layer_check(layer: synth.Layer, batches, seed_x):
    dev = U.device()
    rng = np.random.default_rng(layer.seed_w)
    w_dev = synth.weights(layer, device=dev)
    qw = binding.pack(w_dev, layer.fmt, layer.group)
    rows = _sample_rows(layer.n, rng)
    w_rows = w_dev[torch.from_numpy(rows).to(dev)].cpu().numpy()
    torch.cuda.synchronize()
    del w_dev
    q, ref = U.oracle_buffers(layer.fmt, w_rows, layer.group)
    ref = {name: (None if v is None else v[: oracle.packed_nbytes(layer.fmt, len(rows), layer.k, layer.group)[name]])
           for name, v in ref.items()}  # sampled rows: packed bytes only
    U.assert_packed_equal(U.gpu_buffers(qw, rows), ref, f"{layer.name} {layer.n}x{layer.k} sampled rows")
    deq = oracle.dequantize(q)
    for b in batches:
        x = synth.activations(b, layer.k, seed_x + b, device=dev)
        y = binding.gemm_skinny(qw, x)[:, torch.from_numpy(rows).to(dev)].cpu().numpy()
        xh = x.cpu().numpy()
        U.check_tolerance(y, oracle.gemv_f64(deq, xh), deq, xh, f"{layer.name} b={b}")
    del qw
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["int4_4096x4096", "razer_11008x4096", "afpq_28672x8192",
                                  "bfp6_13824x5120", "bfp4_13824x5120"])
def test_full_size_workload_sampled(name):
    wl = synth.WORKLOADS[name]
    for layer in wl.layers:
        _full_layer_check(layer, wl.batches, wl.seed_x)


@pytest.mark.parametrize("layer_name", ["l0.q", "l0.k", "l2.gate", "l2.down", "l31.down", "lm_head"])
def test_full_size_decode_stack_layers_sampled(layer_name):
    wl = synth.WORKLOADS["llama3_8b_decode_stack"]
    layer = [l for l in wl.layers if l.name == layer_name][0]
    _full_layer_check(layer, wl.batches, wl.seed_x)


def test_full_size_fused_step_every_shape_sampled():
    """The Llama-3-8B-shaped step as the benchmark runs it -- fused q|k|v
    (6144 x 4096) and gate|up (28672 x 4096), one launch per entry through
    step() with the shared workspace, so the K-split forms serve what they
    serve there -- at b = 1, 8, 32 and 64: for every distinct (shape, format)
    of the step (INT4 q|k|v, o, gate|up, down; INT8 the same and the head),
    the packed bytes of sampled rows equal the oracle's and every output of
    those rows, for every batch row, meets the tolerance against the oracle's
    fp64 product."""
    from dequant_gemv_rtn_amd import stack

    dev = U.device()
    wl = synth.WORKLOADS["llama3_8b_decode_stack"]
    st = stack.DecodeStack(wl, device=dev, fused=True)
    by_name = {l.name: l for l in wl.layers}
    picks = {}
    for idx, (layer, qw) in enumerate(st.layers):
        picks.setdefault((layer.n, layer.k, layer.fmt), idx)
    assert len(picks) == 9
    outs = {}
    for b in (1, 8, 32, 64):
        st.step(b)
        torch.cuda.synchronize()
        xs, ys, _ = st.io(b)
        outs[b] = ({k: v.cpu().numpy() for k, v in xs.items()}, {i: ys[i] for i in picks.values()})
    rng = np.random.default_rng(11)
    for (n, k, fmt), idx in picks.items():
        layer, qw = st.layers[idx]
        if "." in layer.name:
            prefix, _, mods = layer.name.rpartition(".")
            members = [by_name[f"{prefix}.{m}"] for m in mods.split("_")]
        else:
            members = [by_name[layer.name]]
        w = torch.cat([synth.weights(m, device=dev) for m in members], dim=0)
        rows = _sample_rows(n, rng, count=24)
        w_rows = w[torch.from_numpy(rows).to(dev)].cpu().numpy()
        del w
        q, ref = U.oracle_buffers(fmt, w_rows, layer.group)
        ref = {name: (None if v is None else v[: oracle.packed_nbytes(fmt, len(rows), k, layer.group)[name]])
               for name, v in ref.items()}
        U.assert_packed_equal(U.gpu_buffers(qw, rows), ref, f"{layer.name} {n}x{k} sampled rows")
        deq = oracle.dequantize(q)
        for b, (xs, ys) in outs.items():
            y = ys[idx][:, torch.from_numpy(rows).to(dev)].cpu().numpy()
            U.check_tolerance(y, oracle.gemv_f64(deq, xs[k]), deq, xs[k], f"{layer.name} ({fmt} {n}x{k}) b={b}")
    del st
    torch.cuda.empty_cache()


# ----------------------------------------------- streaming MFMA kernel --
#
# The weight-streaming MFMA kernel serves 1 <= b <= 64 for k <= 8192; the
# routing between kernels is tunable, so these cases force it (QGEMV_PATH=2)
# and check it like every other path.

# Each streaming case runs in every form: full K per workgroup
# (QGEMV_SPLIT_MIN_B=0) and K-split for every batch (QGEMV_SPLIT_MIN_B=1,
# wherever K spans more than one workgroup's part: k > 1024, or k > 2048 for
# groups of 256) with one chunk per wave, two chunks per wave at one batch
# tile (QGEMV_SPLIT_KC=2), or the activations in LDS.  By default a
# per-shape minimum batch picks the form when a workspace is given, which the
# binding does.
SPLIT = {"full": ("0", "0", "0"), "split": ("1", "0", "1"), "split_kc2": ("1", "0", "2"),
         "split_lds": ("1", "1", "1")}


def _set_form(tune, form):
    min_b, lds, kc = SPLIT[form]
    tune.set("QGEMV_SPLIT_MIN_B", min_b)
    tune.set("QGEMV_SPLIT_LDS", lds)
    tune.set("QGEMV_SPLIT_KC", kc)

STREAM_SHAPES = [  # (n, k, group for the group formats): chunk counts 1, 9, 32, 40, 64, partial chunks, and
    # k above 8192, where the activation slices are streamed with the weights (112 and 128 chunks)
    (37, 160, 32), (50, 1056, 32), (100, 4096, 128), (33, 4096, 64), (40, 5120, 256), (21, 8192, 64), (16, 8192, 128),
    (19, 14336, 128), (35, 16384, 64),
]


@pytest.mark.parametrize("form", list(SPLIT))
@pytest.mark.parametrize("fmt", ALL)
def test_stream_kernel_tolerance(fmt, form, tune):
    tune.set("QGEMV_PATH", "2")
    _set_form(tune, form)
    dev = U.device()
    rng = np.random.default_rng(13)
    for n, k, g in STREAM_SHAPES:
        g = _group(fmt, k, g)
        dist = "student_t5" if fmt in AFPQ else "gauss_outliers"
        w = U.awkward_rows(_weights(n, k, n + 3 * k, dist), rng, extremes=False, tiny=False)
        deq = oracle.dequantize(oracle.quantize(fmt, w, g))
        qw = binding.pack(torch.from_numpy(w).to(dev), fmt, g)
        for b in (1, 2, 3, 4, 5, 8, 9, 13, 16, 17, 33, 64):
            x = synth.activations(b, k, 500 + b).numpy()
            y = binding.gemm_skinny(qw, torch.from_numpy(x).to(dev)).cpu().numpy()
            U.check_tolerance(y, oracle.gemv_f64(deq, x), deq, x, f"stream {form} {fmt} {n}x{k} g{g} b={b}")


@pytest.mark.parametrize("form", list(SPLIT))
@pytest.mark.parametrize("fmt", ALL)
def test_stream_kernel_exact_regime(fmt, form, tune):
    tune.set("QGEMV_PATH", "2")
    _set_form(tune, form)
    n, k = 70, 2048
    g = _group(fmt, k, 64 if fmt in AFPQ else 128)
    rng = np.random.default_rng(15)
    w = _exact_weights(fmt, n, k, g, rng)
    deq = oracle.dequantize(oracle.quantize(fmt, w, g))
    dev = U.device()
    qw = binding.pack(torch.from_numpy(w).to(dev), fmt, g)
    for b in (1, 4, 7, 16, 31, 64):
        x = rng.integers(-2, 3, size=(b, k)).astype(np.float16)
        y = binding.gemm_skinny(qw, torch.from_numpy(x).to(dev)).cpu().numpy()
        want = oracle.gemv_f64(deq, x).astype(np.float16)
        assert np.array_equal(y.view(np.uint16), want.view(np.uint16)), f"stream {form} {fmt} b={b}"


@pytest.mark.parametrize("form", list(SPLIT))
@pytest.mark.parametrize("fmt", ALL)
def test_stream_kernel_many_tiles_per_workgroup(fmt, form, tune):
    """20000 rows = 1250 row tiles: every persistent workgroup walks several
    tiles (its main loop and the leftover tiles both run).  Full K: k = 1024
    and 2560 give slices of 1 and 4 chunks per wave, k = 14336 the
    streamed-activation kernel.  Split: k = 2560 and 14336 cut into 3 and 14
    parts (85 and 18 workgroups per part, 14-15 and 69-70 tiles each), or 2
    and 7 with two chunks per wave."""
    tune.set("QGEMV_PATH", "2")
    _set_form(tune, form)
    for k in (1024, 2560, 14336):
        g = _group(fmt, k, 64 if fmt in AFPQ else 128)
        layer = synth.Layer(f"tiles{k}", 20000, k, fmt, g, "gauss_outliers", 31 + k)
        _full_layer_check(layer, (1, 5, 16, 48), 77)


@pytest.mark.parametrize("form", list(SPLIT))
@pytest.mark.parametrize("name", ["int4_4096x4096", "razer_11008x4096", "afpq_28672x8192"])
def test_stream_kernel_full_size_sampled(name, form, tune):
    tune.set("QGEMV_PATH", "2")
    _set_form(tune, form)
    wl = synth.WORKLOADS[name]
    for layer in wl.layers:
        _full_layer_check(layer, tuple(sorted(set(wl.batches) | {1, 8, 16})), wl.seed_x)


@pytest.mark.parametrize("fmt", ALL)
def test_split_workspace_contract(fmt, tune):
    """The K-split form through q_gemm_skinny_ws: a workspace full of NaN
    bytes needs no clearing; repeated calls give the same bits; the result
    agrees with the full-K form (another fp32 summation order) within the
    tolerance and differs from it by one fp16 place at most (plus fp32
    reordering error where the sum cancels); a workspace one byte short, or
    none, runs the full-K kernels."""
    tune.set("QGEMV_SPLIT_MIN_B", "16")
    n, k = 300, 4096 if fmt not in ("bfp6", "bfp4") else 5120
    g = _group(fmt, k, 64 if fmt in AFPQ else 128)
    dev = U.device()
    w = U.awkward_rows(_weights(n, k, 41, "student_t5" if fmt in AFPQ else "gauss_outliers"),
                       np.random.default_rng(41), extremes=False, tiny=False)
    deq = oracle.dequantize(oracle.quantize(fmt, w, g))
    qw = binding.pack(torch.from_numpy(w).to(dev), fmt, g)
    for b in (16, 40, 64):
        need = binding.workspace_bytes(qw, b)
        assert need == -(-k // 1024) * -(-n // 16) * -(-b // 16) * 1024
        x = synth.activations(b, k, 900 + b, device=dev)
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev)  # NaN bit patterns
        y1 = binding.gemm_skinny(qw, x, workspace=ws)
        y2 = binding.gemm_skinny(qw, x, workspace=ws)
        full = binding.gemm_skinny(qw, x, workspace=torch.empty(0, dtype=torch.uint8, device=dev))
        short = binding.gemm_skinny(qw, x, workspace=ws[: need - 1])
        torch.cuda.synchronize()
        assert torch.equal(y1, y2), f"{fmt} b={b}: split form not deterministic"
        assert torch.equal(short, full), f"{fmt} b={b}: a short workspace must run the full-K kernels"
        xh = x.cpu().numpy()
        ref = oracle.gemv_f64(deq, xh)
        U.check_tolerance(y1.cpu().numpy(), ref, deq, xh, f"split {fmt} b={b}")
        U.check_tolerance(full.cpu().numpy(), ref, deq, xh, f"full {fmt} b={b}")
        a = y1.cpu().numpy().astype(np.float64)
        c = full.cpu().numpy().astype(np.float64)
        # one fp16 place, plus fp32 reordering error where the sum cancels
        ulp = np.spacing(np.maximum(np.abs(a), np.abs(c)).astype(np.float16)).astype(np.float64)
        reorder = 2.0 ** -16 * (np.abs(xh.astype(np.float64)) @ np.abs(deq).T)
        assert np.all(np.abs(a - c) <= ulp + reorder), f"{fmt} b={b}: split and full-K differ beyond rounding"


# --------------------------------------- vector-ALU kernel, shared x --
#
# For b <= 2 several row walkers share a workgroup and one LDS copy of the
# activations (QGEMV_VALU_SHARE walkers when one wave covers a row).  Cases:
# fewer rows than walkers (walkers with nothing to do still take part in the
# LDS fill and in the per-row barriers), k = 8192 at b = 1 and k = 4096 at
# b = 2 (16 KiB with one wave per row), rows split over two waves (k = 14336
# and 16384 at b = 1, 8192 at b = 2: 4 walkers of 2 waves, up to 32 KiB),
# over four waves (k = 16384 at b = 2, no sharing), a partial last piece
# range, and sharing off.

@pytest.mark.parametrize("share", ["1", "4", "8"])
@pytest.mark.parametrize("fmt", ALL)
def test_valu_kernel_shared_activations(fmt, share, tune):
    tune.set("QGEMV_PATH", "1")
    tune.set("QGEMV_VALU_SHARE", share)
    dev = U.device()
    rng = np.random.default_rng(17)
    for n, k, g, batches in ((3, 160, 32, (1, 2)), (37, 1056, 32, (1, 2)), (1000, 4096, 128, (1, 2)),
                             (13, 8192, 64, (1, 2)), (301, 6144, 128, (1,)), (29, 14336, 128, (1,)),
                             (6, 16384, 64, (1, 2)), (517, 12288, 128, (1, 2))):
        g = _group(fmt, k, g)
        dist = "student_t5" if fmt in AFPQ else "gauss_outliers"
        w = U.awkward_rows(_weights(n, k, n + 5 * k, dist), rng, extremes=False, tiny=False)
        deq = oracle.dequantize(oracle.quantize(fmt, w, g))
        qw = binding.pack(torch.from_numpy(w).to(dev), fmt, g)
        for b in batches:
            x = synth.activations(b, k, 700 + b).numpy()
            y = binding.gemm_skinny(qw, torch.from_numpy(x).to(dev)).cpu().numpy()
            U.check_tolerance(y, oracle.gemv_f64(deq, x), deq, x, f"valu share={share} {fmt} {n}x{k} g{g} b={b}")


# ---------------------------------------------------------------- edges --

@pytest.mark.parametrize("fmt", ALL)
def test_edges_min_max_and_ragged(fmt):
    dev = U.device()
    for n, k, batches in ((1, 32, (1, 9)), (65, 4128, (1, 2, 8, 16, 64)), (3, 16384, (1, 8, 64)), (17, 160, (5, 33))):
        g = _group(fmt, k, 32)
        w = _weights(n, k, n + k)
        deq = oracle.dequantize(oracle.quantize(fmt, w, g))
        qw = binding.pack(torch.from_numpy(w).to(dev), fmt, g)
        _, ref = U.oracle_buffers(fmt, w, g)
        U.assert_packed_equal(U.gpu_buffers(qw), ref, f"{fmt} {n}x{k}")
        for b in batches:
            x = synth.activations(b, k, b).numpy()
            y = binding.gemm_skinny(qw, torch.from_numpy(x).to(dev)).cpu().numpy()
            U.check_tolerance(y, oracle.gemv_f64(deq, x), deq, x, f"{fmt} {n}x{k} b={b}")


@pytest.mark.parametrize("fmt", ALL)
def test_zero_inputs_give_zero(fmt):
    dev = U.device()
    n, k = 40, 512
    g = _group(fmt, k, 64)
    qw = binding.pack(torch.zeros((n, k), dtype=torch.float16, device=dev), fmt, g)
    for b in (1, 8, 16):
        x = synth.activations(b, k, 5, device=dev)
        assert torch.count_nonzero(binding.gemm_skinny(qw, x)).item() == 0
    w = synth.small_weights(n, k, 9).to(dev)
    qw = binding.pack(w, fmt, g)
    for b in (1, 8, 16):
        y = binding.gemm_skinny(qw, torch.zeros((b, k), dtype=torch.float16, device=dev))
        assert torch.count_nonzero(y).item() == 0


def test_deterministic_and_gemv_matches_gemm():
    dev = U.device()
    w = synth.small_weights(300, 4096, 11).to(dev)
    for fmt in ALL:
        g = _group(fmt, 4096, 128)
        qw = binding.pack(w, fmt, g)
        qw2 = binding.pack(w, fmt, g)
        for name in U.BUFS:
            if qw.buffers[name] is not None:
                assert torch.equal(qw.buffers[name], qw2.buffers[name])
        x = synth.activations(1, 4096, 3, device=dev)
        y1 = binding.gemv(qw, x[0])
        y2 = binding.gemm_skinny(qw, x)[0]
        assert torch.equal(y1, y2)
        for b in (8, 64):
            xb = synth.activations(b, 4096, 4, device=dev)
            assert torch.equal(binding.gemm_skinny(qw, xb), binding.gemm_skinny(qw, xb))


def test_linear_flattens_leading_dimensions():
    """binding.linear on x [2, 3, k] (and [k]) gives the rows of gemm_skinny
    on the flattened [6, k] activations, bit for bit, in shape [2, 3, n]."""
    dev = U.device()
    w = synth.small_weights(200, 2048, 13).to(dev)
    qw = binding.pack(w, "int4_asym", 128)
    x = synth.activations(6, 2048, 14, device=dev)
    y = binding.linear(x.view(2, 3, 2048), qw)
    assert tuple(y.shape) == (2, 3, 200)
    assert torch.equal(y.reshape(6, 200), binding.gemm_skinny(qw, x))
    y1 = binding.linear(x[0], qw)
    assert tuple(y1.shape) == (200,) and torch.equal(y1, binding.gemv(qw, x[0]))
    out = torch.empty((2, 3, 200), dtype=torch.float16, device=dev)
    assert binding.linear(x.view(2, 3, 2048), qw, out=out).data_ptr() == out.data_ptr()
    assert torch.equal(out, y)


def test_side_stream_and_error_paths():
    dev = U.device()
    w = synth.small_weights(64, 1024, 12).to(dev)
    qw = binding.pack(w, "fp4_razer", 128)
    x = synth.activations(4, 1024, 6, device=dev)
    ref = binding.gemm_skinny(qw, x)
    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        y = binding.gemm_skinny(qw, x)
    s.synchronize()
    assert torch.equal(y, ref)
    buf = torch.empty(1024 + 8, dtype=torch.float16, device=dev)
    with pytest.raises(binding.QError) as e:
        binding.gemv(qw, buf[1:1025])
    assert e.value.status == -3  # misaligned x
