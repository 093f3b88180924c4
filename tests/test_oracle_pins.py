"""Pins of the CPU oracle to things other than itself (CPU only).

* hand-worked examples (tests/golden/hand_examples.json);
* scales re-derived with exact rational IEEE rounding (tests/exact.py);
* brute-force nearest-code search over every code of every format, in exact
  rational arithmetic, on small random and constructed groups;
* invariants the pages state: RaZeR's remapped code never decodes to zero,
  AFPQ's positive codes depend only on the positive scale, the block format's
  6.5-bit width gives the stated 5x / 1.2x memory densities;
* special cases that reduce to something known: AFPQ with equal extremes is
  plain E2M1, the E8M0 exponent byte decodes like torch.float8_e8m0fnu;
* the fp64 product against math.fsum and against unit vectors;
* planted mistakes in the oracle that the checks above must catch.
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from oracle import layout as L
from tests import exact as X

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


# ------------------------------------------------------------ test inputs --

def _mixed_groups(rng, n, k, scale=0.02):
    """Small awkward inputs: gaussian with outliers, plus rows of exact
    zeros, constant values, tiny subnormals, -0.0, fp16 extremes."""
    w = rng.standard_normal((n, k)) * scale
    w[rng.random((n, k)) < 0.02] *= 20
    w = w.astype(np.float16)
    if n >= 6:
        w[1, :] = 0
        w[2, :] = np.float16(0.03125)
        w[3, :] = np.float16(2.0 ** -24) * rng.integers(-3, 4, size=k)
        w[4, : k // 2] = np.float16(-0.0)
        w[5, 0] = np.float16(65504)
        w[5, 1] = np.float16(-65504)
    return w


def _f(v):
    return Fraction(float(v))


# ------------------------------------------------ independent re-derivation --

def check_scales_and_codes(fmt: str, w16: np.ndarray, g: int, quantize=None):
    """Re-derive every stored scale/zero/selector/exponent and every code of
    ``quantize(fmt, w16, g)`` with exact rationals and brute force."""
    quantize = quantize or oracle.quantize
    q = quantize(fmt, w16, g)
    n, k = w16.shape
    G = k // g
    for r in range(n):
        for j in range(G):
            seg = [_f(v) for v in w16[r, j * g:(j + 1) * g]]
            codes = q.codes[r, j * g:(j + 1) * g]
            if fmt == "int4_asym":
                lo = min(min(seg), Fraction(0))
                hi = max(max(seg), Fraction(0))
                s = X.to_f16(X.to_f32(X.to_f32(hi - lo) / 15))
                assert _f(q.scales[r, j]) == s
                if s == 0:
                    assert q.zeros[r, j] == 0 and not codes.any()
                    continue
                z = X.nearest_code(-lo / s, {c: Fraction(c) for c in range(16)}, X.even_int_prefer)
                assert q.zeros[r, j] == z
                table, prefer = X.int4_table(z, s), X.int4_prefer(z)
            elif fmt == "fp4_e2m1":
                s = X.to_f16(X.to_f32(max(abs(v) for v in seg) / 6))
                assert _f(q.scales[r, j]) == s
                table, prefer = X.e2m1_table(s), X.e2m1_prefer
            elif fmt == "fp4_razer":
                amax = max(abs(v) for v in seg)
                best = None
                per = []
                for ci, v in enumerate((5, -5, 8, -8)):
                    s = X.to_f16(X.to_f32(amax / max(6, abs(v))))
                    t = X.razer_table(s, Fraction(v))
                    cs = [X.nearest_code(x, t, X.razer_prefer) for x in seg]
                    sse = sum(((x - t[c]) ** 2 for x, c in zip(seg, cs)), Fraction(0))
                    per.append((sse, s, t, cs))
                    if best is None or sse < per[best][0]:
                        best = ci
                sel = int(q.selectors[r, j])
                tol = per[best][0] * Fraction(1, 10 ** 12)
                assert per[sel][0] - per[best][0] <= tol
                if all(abs(per[c][0] - per[best][0]) > tol for c in range(4) if c != best):
                    assert sel == best
                sse, s, table, cs = per[sel]
                assert _f(q.scales[r, j]) == s
                assert list(codes) == cs
                continue
            elif fmt == "fp4_afpq":
                sp = X.to_f16(X.to_f32(max(max(seg), Fraction(0)) / 6))
                sn = X.to_f16(X.to_f32(max(-min(seg), Fraction(0)) / 6))
                assert _f(q.scales[r, j, 0]) == sp and _f(q.scales[r, j, 1]) == sn
                table, prefer = X.afpq_table(sp, sn), X.e2m1_prefer
            elif fmt in ("bfp6", "bfp4"):
                mb = 5 if fmt == "bfp6" else 3
                a = max(abs(v) for v in seg)
                if a == 0:
                    assert q.exps[r, j] == 0 and not codes.any()
                    continue
                E = 0
                while Fraction(2) ** E > a:
                    E -= 1
                while Fraction(2) ** (E + 1) <= a:
                    E += 1
                assert int(q.exps[r, j]) == E + 127
                table, prefer = X.bfp_table(mb, Fraction(2) ** (E - mb + 1)), X.even_int_prefer
            elif fmt == "int8":
                s = X.to_f16(X.to_f32(max(abs(v) for v in seg) / 127))
                assert _f(q.scales[r]) == s
                if s == 0:
                    assert not codes.any()
                    continue
                table, prefer = X.int8_table(s), X.even_int_prefer
            else:
                raise AssertionError(fmt)
            expect = [X.nearest_code(x, table, prefer) for x in seg]
            assert list(codes) == expect, (fmt, r, j)
    return q


FMT_GROUPS = [
    ("int4_asym", 32), ("fp4_e2m1", 32), ("fp4_razer", 32), ("fp4_afpq", 32),
    ("bfp6", 16), ("bfp4", 16), ("int8", 48),
]


@pytest.mark.parametrize("fmt,g", FMT_GROUPS)
def test_bruteforce_random_and_awkward(fmt, g):
    rng = np.random.default_rng(11)
    k = 48 if fmt == "int8" else 64
    if fmt == "fp4_razer" or fmt == "int8":
        k = 48 if fmt == "int8" else 32
    w = _mixed_groups(rng, 6, k)
    check_scales_and_codes(fmt, w, g)


@pytest.mark.parametrize("fmt,g", FMT_GROUPS)
def test_bruteforce_constructed_ties(fmt, g):
    """Groups whose elements sit exactly on decision boundaries."""
    rng = np.random.default_rng(5)
    rows = []
    k = 48 if fmt == "int8" else 32
    for _ in range(3):
        s = float(2.0 ** rng.integers(-8, 2))
        if fmt in ("fp4_e2m1", "fp4_razer", "fp4_afpq"):
            mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 4.5, 5.0, 5.5, 7.0])
            vals = np.concatenate([[6.0], mids, -mids])
        elif fmt == "int4_asym":
            vals = np.concatenate([[-5.0, 10.0], np.arange(-4.5, 10, 1.0)])
        elif fmt == "int8":
            vals = np.concatenate([[127.0], np.arange(-126.5, 127, 7.0)])
        else:
            vals = np.concatenate([[16.0, -30.5], np.arange(0.5, 31, 1.0)])
        row = np.resize(vals * s, k)
        rng.shuffle(row)
        rows.append(row)
    w = np.array(rows).astype(np.float16)
    check_scales_and_codes(fmt, w, g if fmt != "int8" else k)


# ------------------------------------------------------ hand-worked examples --

def _golden():
    with open(GOLDEN) as fh:
        return json.load(fh)["examples"]


@pytest.mark.parametrize("ex", _golden(), ids=lambda e: e["name"])
def test_hand_examples(ex):
    k = ex["k"]
    w = np.zeros((1, k), dtype=np.float16)
    w[0, : len(ex["w"])] = np.array(ex["w"], dtype=np.float64).astype(np.float16)
    q = oracle.quantize(ex["fmt"], w, ex["group"])
    buf = oracle.pack(q)
    if "words" in ex:
        assert [f"{int(v):08X}" for v in buf["codes"][0]] == ex["words"]
    if "hi_words" in ex:
        assert [f"{int(v):08X}" for v in buf["codes_hi"][0]] == ex["hi_words"]
    if "aux_words" in ex:
        assert [f"{int(v):08X}" for v in buf["aux"][0]] == ex["aux_words"]
    if "exp_bytes" in ex:
        assert [f"{int(v):02X}" for v in buf["aux"][0]] == ex["exp_bytes"]
    if "int8" in ex:
        assert list(buf["codes"][0, : len(ex["int8"])]) == ex["int8"]
    if "scale_bits" in ex:
        bits = buf["scales"].reshape(-1).view(np.uint16)
        assert [f"{int(v):04X}" for v in bits] == ex["scale_bits"]


# ---------------------------------------------------------- code tables --

def test_e2m1_table_matches_bitfield_closed_form():
    for c in range(8):
        assert X.e2m1_value(c) == Fraction(F.E2M1_MAGNITUDES[c])
    # the 16 codes hold 15 distinct values; the only repeat is +0 / -0
    vals = [X.e2m1_value(c) for c in range(16)]
    assert len(set(vals)) == 15 and vals[0] == vals[8] == 0


def test_e8m0_exponent_byte_matches_torch():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((4, 64)) * 10.0 ** rng.integers(-4, 3, size=(4, 1))).astype(np.float16)
    for fmt, mb in (("bfp6", 5), ("bfp4", 3)):
        q = oracle.quantize(fmt, w, 16)
        scale_t = torch.from_numpy(q.exps.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
        a = np.abs(w.astype(np.float64)).reshape(4, 4, 16).max(-1)
        # 2^E is the largest power of two <= the block max
        assert np.all(scale_t <= a) and np.all(a < 2 * scale_t)
        deq = oracle.dequantize(q).reshape(4, 4, 16)
        steps = scale_t * 2.0 ** (1 - mb)
        m = deq / steps[..., None]
        assert np.all(m == np.rint(m)) and np.all(np.abs(m) <= 2 ** mb - 1)


def test_block_width_matches_page_density():
    # "Revisiting Block-based Quantisation" (abstract): 6-bit block format has
    # 5x the memory density of float32 and 1.2x that of 8-bit.
    n, k = 64, 4096
    sz = oracle.packed_nbytes("bfp6", n, k, 16)
    bits = 8 * sum(sz.values()) / (n * k)
    assert bits == 6.5
    assert round(32 / bits, 1) == 4.9 and round(32 / bits) == 5
    assert round(8 / bits, 1) == 1.2
    # a 5-bit element would miss both figures
    assert round(32 / 5.5) != 5 or round(8 / 5.5, 1) != 1.2


def test_afpq_metadata_equals_asym_int_metadata():
    # "AFPQ" (abstract): no extra storage compared with asymmetric INT, whose
    # per-group metadata is an fp16 scale and an fp16 zero-point.
    n, k, g = 8, 1024, 64
    sz = oracle.packed_nbytes("fp4_afpq", n, k, g)
    assert sz["scales"] == n * (k // g) * (2 + 2)
    assert sz["codes"] == n * k // 2


# ----------------------------------------------------------- invariants --

def test_razer_special_code_never_decodes_to_zero():
    rng = np.random.default_rng(7)
    w = _mixed_groups(rng, 16, 256)
    q = oracle.quantize("fp4_razer", w, 128)
    deq = oracle.dequantize(q).reshape(16, 2, 128)
    codes = q.codes.reshape(16, 2, 128)
    s = q.scales.astype(np.float64)
    special = codes == 8
    assert special.any()
    assert np.all(deq[special] != 0)
    nz_groups = (s != 0)[..., None] & special
    assert np.array_equal(nz_groups, special & (s[..., None] != 0))
    # and the value it decodes to is the selected special times the scale
    v = np.asarray(F.RAZER_SPECIALS)[q.selectors][..., None] * s[..., None]
    assert np.all(deq[special] == np.broadcast_to(v, deq.shape)[special])


def test_afpq_positive_codes_depend_only_on_positive_scale():
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((8, 128)) * 0.02).astype(np.float16)
    w2 = w.copy()
    neg = w2 < 0
    w2[neg] = (w2[neg].astype(np.float32) * 3.0).astype(np.float16)  # moves s- only
    q1 = oracle.quantize("fp4_afpq", w, 64)
    q2 = oracle.quantize("fp4_afpq", w2, 64)
    pos = w > 0
    assert np.array_equal(q1.scales[..., 0], q2.scales[..., 0])
    assert not np.array_equal(q1.scales[..., 1], q2.scales[..., 1])
    assert np.array_equal(q1.codes[pos], q2.codes[pos])


def test_afpq_with_equal_extremes_is_plain_e2m1():
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((8, 64)) * 0.02).astype(np.float16)
    w[:, 0] = np.float16(0.09)
    w[:, 1] = np.float16(-0.09)
    w = np.clip(w, np.float16(-0.09), np.float16(0.09))
    a = oracle.quantize("fp4_afpq", w, 64)
    e = oracle.quantize("fp4_e2m1", w, 64)
    assert np.array_equal(a.codes, e.codes)
    assert np.array_equal(a.scales[..., 0], e.scales) and np.array_equal(a.scales[..., 1], e.scales)


def _few_bit_extremes(rng, fmt, n, k, g):
    """Random groups whose extremes make every decoded value fp16-exact:
    each group's scale comes out with at most 6 significant bits."""
    w = rng.standard_normal((n, k)) * 0.02
    for r in range(n):
        for j in range(k // g):
            c = float(rng.integers(32, 64)) * 2.0 ** int(rng.integers(-16, -10))
            seg = w[r, j * g:(j + 1) * g]
            if fmt == "fp4_afpq":
                c2 = float(rng.integers(32, 64)) * 2.0 ** int(rng.integers(-16, -10))
                np.clip(seg, -6 * c2, 6 * c, out=seg)
                seg[0], seg[1] = 6 * c, -6 * c2
            else:
                c4 = float(rng.integers(8, 16)) * 2.0 ** int(rng.integers(-16, -10))
                top = {"fp4_e2m1": 6 * c, "fp4_razer": 24 * c, "int8": 127 * c4}.get(fmt, 6 * c)
                np.clip(seg, -top, top, out=seg)
                seg[0] = top if rng.random() < 0.5 else -top
    return w.astype(np.float16)


@pytest.mark.parametrize("fmt,g", [f for f in FMT_GROUPS if f[0] != "int4_asym"])
def test_requantizing_decoded_values_is_identity(fmt, g):
    rng = np.random.default_rng(12)
    k = 48 if fmt == "int8" else 256
    gg = g if fmt != "int8" else k
    w = _few_bit_extremes(rng, fmt, 8, k, gg)
    q = oracle.quantize(fmt, w, gg)
    deq = oracle.dequantize(q)
    w2 = deq.astype(np.float16)
    assert np.array_equal(w2.astype(np.float64), deq)  # decoded values are fp16-exact here
    q2 = oracle.quantize(fmt, w2, gg)
    assert np.array_equal(oracle.dequantize(q2), deq)
    if fmt != "fp4_razer":
        assert np.array_equal(q2.codes, q.codes)


def test_int4_requantize_identity_when_full_range_used():
    """Groups spanning [-z0*c, (15-z0)*c] with a few-bit c: decoded values are
    fp16-exact, the range is fully used, and requantizing is the identity."""
    rng = np.random.default_rng(13)
    n, k, g = 16, 512, 128
    w = np.empty((n, k))
    for r in range(n):
        for j in range(k // g):
            c = float(rng.integers(32, 64)) * 2.0 ** int(rng.integers(-16, -10))
            z0 = int(rng.integers(0, 16))
            seg = rng.uniform(-z0 * c, (15 - z0) * c, size=g)
            seg[0], seg[1] = -z0 * c, (15 - z0) * c
            w[r, j * g:(j + 1) * g] = seg
    w = w.astype(np.float16)
    q = oracle.quantize("int4_asym", w, g)
    deq = oracle.dequantize(q)
    assert np.array_equal(deq.astype(np.float16).astype(np.float64), deq)
    q2 = oracle.quantize("int4_asym", deq.astype(np.float16), g)
    assert np.array_equal(oracle.dequantize(q2), deq)
    assert np.array_equal(q2.codes, q.codes) and np.array_equal(q2.zeros, q.zeros)


def test_dequant_is_nearest_representable_error_bounds():
    rng = np.random.default_rng(14)
    w = (rng.standard_normal((8, 512)) * 0.02).astype(np.float16)
    w64 = w.astype(np.float64)
    q = oracle.quantize("int4_asym", w, 128)
    err = np.abs(oracle.dequantize(q) - w64).reshape(8, 4, 128)
    s = q.scales.astype(np.float64)[..., None]
    assert np.all(err <= s / 2 * (1 + 2 ** -10) + 1e-12)
    q = oracle.quantize("int8", w, 512)
    err = np.abs(oracle.dequantize(q) - w64)
    assert np.all(err <= q.scales.astype(np.float64)[:, None] / 2 * (1 + 2 ** -10))


# ----------------------------------------------------------------- GEMV --

def test_gemv_matches_exactly_rounded_sum():
    rng = np.random.default_rng(15)
    w = (rng.standard_normal((6, 256)) * 0.02).astype(np.float16)
    x = rng.standard_normal((3, 256)).astype(np.float16)
    for fmt, g in (("int4_asym", 128), ("fp4_razer", 128), ("bfp6", 16), ("int8", 256)):
        deq = oracle.dequantize(oracle.quantize(fmt, w, g))
        y = oracle.gemv_f64(deq, x)
        assert y.shape == (3, 6)
        for b in range(3):
            for n in range(6):
                exact = math.fsum(float(a) * float(c) for a, c in zip(deq[n], x[b].astype(np.float64)))
                assert abs(y[b, n] - exact) <= 1e-14 * max(1.0, abs(exact))


def test_gemv_unit_vector_returns_column():
    rng = np.random.default_rng(16)
    w = (rng.standard_normal((5, 64)) * 0.02).astype(np.float16)
    deq = oracle.dequantize(oracle.quantize("fp4_afpq", w, 32))
    for kk in (0, 17, 63):
        x = np.zeros((1, 64), dtype=np.float16)
        x[0, kk] = 1
        assert np.array_equal(oracle.gemv_f64(deq, x)[0], deq[:, kk])


# ------------------------------------------------------------ layout --

def test_layout_closed_forms():
    codes = np.arange(16, dtype=np.int64)[None, :].repeat(2, 0)
    q = F.Quantized("fp4_e2m1", 2, 16, 16, codes, scales=np.ones((2, 1), np.float16))
    buf = oracle.pack(q)
    assert buf["codes"].tolist() == [[0x76543210, 0xFEDCBA98]] * 2
    sel = np.array([[0, 1, 2, 3, 3, 2, 1, 0, 1]], dtype=np.int64)
    assert L._pack_fields(sel, 2).tolist() == [[0b01_00_01_10_11_11_10_01_00]]
    hi = np.arange(16) % 4
    word = L._pack_bfp6_hi(hi[None, :])[0, 0]
    for e in range(16):
        pos = 16 * ((e % 8) // 4) + 8 * (e // 8) + 2 * (e % 4)
        assert (int(word) >> pos) & 3 == hi[e]


@pytest.mark.parametrize("fmt,g", FMT_GROUPS)
def test_pack_unpack_roundtrip_and_sizes(fmt, g):
    rng = np.random.default_rng(17)
    k = 96 if fmt == "int8" else 256
    n = 5
    w = _mixed_groups(rng, n, k)
    q = oracle.quantize(fmt, w, g if fmt != "int8" else k)
    buf = oracle.pack(q)
    sz = oracle.packed_nbytes(fmt, n, k, q.group)
    for name, arr in buf.items():
        assert (0 if arr is None else arr.nbytes) == sz[name]
    q2 = oracle.unpack(fmt, n, k, q.group, buf)
    assert np.array_equal(oracle.dequantize(q2), oracle.dequantize(q))


# ------------------------------------------------- planted mistakes --

def _fails(fn) -> bool:
    try:
        fn()
    except AssertionError:
        return True
    return False


def _rand(rng, n=4, k=64):
    w = _mixed_groups(rng, max(n, 6), k)
    return w


def test_planted_mistakes_are_caught(monkeypatch):
    rng = np.random.default_rng(21)
    w = _rand(rng)
    ties = np.resize(np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0]), 32)[None, :].astype(np.float16)

    # wrong E2M1 table entry
    with monkeypatch.context() as m:
        m.setattr(F, "E2M1_MAGNITUDES", np.array([0, 0.5, 1, 1.5, 2, 3, 4, 5.0]))
        assert _fails(lambda: check_scales_and_codes("fp4_e2m1", w, 32))
    # ties to odd instead of even
    orig = F._nearest_magnitude_index

    def odd_ties(mag, scale):
        cand = F.E2M1_MAGNITUDES * scale[..., None]
        d = np.abs(mag[..., None] - cand)
        return (d == d.min(-1, keepdims=True)).cumsum(-1).argmax(-1)
    with monkeypatch.context() as m:
        m.setattr(F, "_nearest_magnitude_index", odd_ties)
        assert _fails(lambda: check_scales_and_codes("fp4_e2m1", ties, 32))
    assert F._nearest_magnitude_index is orig
    # INT4 zero-point with the wrong sign
    with monkeypatch.context() as m:
        m.setattr(F, "_rne_quotient", lambda a, s: np.rint(np.abs(a) / s) * np.sign(a))
        assert not _fails(lambda: check_scales_and_codes("int4_asym", w, 32))  # control: same values
        m.setattr(F, "_rne_quotient", lambda a, s: np.floor(a / s + 0.5))  # ties up, not even
        tie_w = np.resize(np.array([-5.0, 10.0, 0.5, 1.5, 2.5, -0.5, -1.5]), 32)[None, :].astype(np.float16)
        assert _fails(lambda: check_scales_and_codes("int4_asym", tie_w, 32))
    # RaZeR picks the worst candidate / a permuted candidate list
    with monkeypatch.context() as m:
        m.setattr(F, "RAZER_SPECIALS", (5.0, -5.0, -8.0, 8.0))
        assert _fails(lambda: check_scales_and_codes("fp4_razer", w, 32))
    # AFPQ scales swapped
    real = F.quantize_fp4_afpq

    def swapped(w16, g):
        q = real(w16, g)
        q.scales = q.scales[..., ::-1].copy()
        return q
    with monkeypatch.context() as m:
        m.setattr(F, "quantize_fp4_afpq", swapped)
        assert _fails(lambda: check_scales_and_codes("fp4_afpq", w, 32, quantize=lambda f, a, g: swapped(a, g)))
    # block exponent off by one
    real_bfp = F.quantize_bfp

    def off_by_one(w16, fmt):
        q = real_bfp(w16, fmt)
        q.exps = np.where(q.exps > 0, q.exps + 1, 0).astype(np.uint8)
        return q
    assert _fails(lambda: check_scales_and_codes("bfp6", w, 16, quantize=lambda f, a, g: off_by_one(a, f)))
    # GEMV with a dropped term / transposed operand
    deq = oracle.dequantize(oracle.quantize("int8", w[:4, :64], 64))
    x = rng.standard_normal((2, 64)).astype(np.float16)

    def gemv_check(fn):
        y = fn(deq, x)
        for b in range(2):
            for n in range(4):
                ex = math.fsum(float(a) * float(c) for a, c in zip(deq[n], x[b].astype(np.float64)))
                assert abs(y[b, n] - ex) <= 1e-12 * max(1.0, abs(ex))
    assert not _fails(lambda: gemv_check(oracle.gemv_f64))
    assert _fails(lambda: gemv_check(lambda d, xx: xx[:, :-1].astype(np.float64) @ d[:, :-1].T))
    assert _fails(lambda: gemv_check(lambda d, xx: np.flip(xx.astype(np.float64) @ d.T, axis=1)))
    # nibble order reversed in the packer
    real_pack = L._pack_fields

    def hi_first(values, bits):
        per = 32 // bits
        v = values.reshape(values.shape[0], -1, per)[:, :, ::-1].reshape(values.shape)
        return real_pack(v, bits)
    with monkeypatch.context() as m:
        m.setattr(L, "_pack_fields", hi_first)
        ex = [e for e in _golden() if e["name"] == "fp4_e2m1_ties_and_signs"][0]
        assert _fails(lambda: test_hand_examples(ex))
