"""Pins of the W8A8 oracle (oracle/w8a8.py) against facts fixed outside it:
hand-worked values (tests/golden/w8a8_examples.json: one case where taking
the code from the binary32 quotient differs from the exact quotient, one
where two binary32 roundings of the rescale differ from one), exact-rational
recomputation of every step from the IEEE rounding definition
(tests/exact.py), brute-force integer sums, exact invariants of the
per-token quantizer, and the RTN error bound against the fp64 product.
Mutants planted in the oracle (a wrong rounding, a decision on the exact
quotient, a one-rounding rescale, a transposed operand, a missing scale)
must each fail one of them."""

from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.w8a8 as w8
from tests.exact import to_f16, to_f32

rng = np.random.default_rng(2024)
GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "w8a8_examples.json")))


def _fr(v) -> Fraction:
    return Fraction(v) if isinstance(v, str) else Fraction(float(v))


def _f32(fr: Fraction) -> np.float32:
    v = np.float32(float(fr))
    assert Fraction(float(v)) == fr, "not a binary32 value"
    return v


def _rne_int(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def _codes_exact(x_row, m_row):
    """The activation reading recomputed in exact rationals: each step one
    IEEE binary32 rounding (tests/exact.py), the code the nearest integer of
    the rounded quotient, ties to even, clamped to +-127."""
    a = [to_f32(Fraction(float(xv)) / (Fraction(float(mv)) if m_row is not None else 1))
         for xv, mv in zip(x_row, m_row if m_row is not None else [1] * len(x_row))]
    s = to_f32(max(abs(v) for v in a) / 127)
    if s == 0:
        return [0] * len(a), s
    return [max(-127, min(127, _rne_int(to_f32(v / s)))) for v in a], s


def test_golden_quotient_rounding_decision():
    g = GOLDEN["quotient"]
    x = np.array([g["x"]], dtype=np.float16)
    m = np.array([_f32(_fr(v)) for v in g["smooth"]], dtype=np.float32)
    q, s = oracle.quantize_activations(x, m)
    assert Fraction(float(s[0])) == _fr(g["s"])
    assert q[0].tolist() == g["codes"]
    # the hand derivation agrees with the exact-rational recomputation
    codes, s_exact = _codes_exact(g["x"], [_fr(v) for v in g["smooth"]])
    assert codes == g["codes"] and s_exact == _fr(g["s"])
    assert _rne_int(Fraction(1) / _fr(g["s"])) == g["codes_exact_quotient"][1] != g["codes"][1]


def test_golden_rescale_two_roundings():
    g = GOLDEN["rescale"]
    x = np.array([g["x"]], dtype=np.float16)
    qw = np.array([g["w_codes"]], dtype=np.int8)
    sw = np.array([float(_fr(g["w_scale"]))], dtype=np.float16)
    assert Fraction(float(sw[0])) == _fr(g["w_scale"])
    y, acc, qx, sx = oracle.gemm_w8a8(x, qw, sw)
    assert sx[0] == 1.0 and qx[0].tolist() == g["x"]
    assert int(acc[0, 0]) == g["acc"]
    assert float(y[0, 0]) == g["y"] != g["y_one_rounding"]


def test_activation_codes_exact_rational():
    """Random rows, smoothed by factors with full binary32 significands and
    unsmoothed, with values spread over decades: every code and scale equals
    the exact-rational recomputation of the reading."""
    for trial in range(12):
        k = 48
        x = (rng.standard_normal((3, k)) * 10.0 ** rng.uniform(-3, 3, size=(3, 1))).astype(np.float16)
        m = rng.uniform(0.3, 3.0, size=k).astype(np.float32) if trial % 2 else None
        q, s = oracle.quantize_activations(x, m)
        for b in range(3):
            codes, s_exact = _codes_exact(x[b], None if m is None else m)
            assert Fraction(float(s[b])) == s_exact
            assert q[b].tolist() == codes, (trial, b)


def test_rescale_exact_rational_including_large_accumulators():
    """y = f16(f32(f32(s_x s_w) f32(acc))) recomputed from the IEEE
    definition, with s_x a full binary32 significand (a row whose absmax is
    not a multiple of 127) and accumulators beyond 2^24, whose binary32
    conversion rounds."""
    B, N, K = 3, 6, 2048
    x = rng.uniform(90, 120, size=(B, K)).astype(np.float16)
    x[:, 0] = np.array([113.3, 119.7, 101.1], dtype=np.float16)
    x[:, 1:] = np.minimum(x[:, 1:], x[:, :1])
    qw = rng.integers(100, 128, size=(N, K)).astype(np.int8)
    qw[1] = -qw[1]
    sw = rng.uniform(1e-5, 4e-5, size=N).astype(np.float16)
    y, acc, qx, sx = oracle.gemm_w8a8(x, qw, sw)
    assert (np.abs(acc) > 2 ** 24).all() and (acc % 2 != 0).any()
    for b in range(B):
        codes, s_exact = _codes_exact(x[b], None)
        assert Fraction(float(sx[b])) == s_exact and qx[b].tolist() == codes
        assert s_exact.denominator.bit_length() > 20  # not a short binary fraction
        for n in range(N):
            acc_exact = sum(int(a) * int(w) for a, w in zip(codes, qw[n]))
            assert acc_exact == int(acc[b, n])
            want = to_f16(to_f32(to_f32(s_exact * Fraction(float(sw[n]))) * to_f32(Fraction(acc_exact))))
            assert Fraction(float(y[b, n])) == want, (b, n)


def test_hand_example_scale_ties_and_clamp():
    # absmax 127 gives s = 1 exactly; -63.5 and 2.5 are ties (to even: -64, 2)
    x = np.array([[127.0, -63.5, 2.5, 0.25, -127.0, 0.0]], dtype=np.float16)
    q, s = oracle.quantize_activations(x)
    assert s.tolist() == [1.0]
    assert q.tolist() == [[127, -64, 2, 0, -127, 0]]
    # absmax 2: 2^27 * 2 / 127 = 2113665.008, so s = 2113665 * 2^-27 in binary32;
    # 1 / s = 63.5 + 1/4227330, whose binary32 rounding is 63.5 (spacing 2^-18
    # there), a tie that goes to the even 64
    x = np.array([[2.0, 1.0, -1.0]], dtype=np.float16)
    q, s = oracle.quantize_activations(x)
    assert Fraction(float(s[0])) == Fraction(2113665, 2 ** 27)
    assert q[0].tolist() == [127, 64, -64]


def test_zero_row_and_smoothing_by_powers_of_two():
    x = np.zeros((2, 64), dtype=np.float16)
    x[1] = rng.standard_normal(64).astype(np.float16)
    q, s = oracle.quantize_activations(x)
    assert s[0] == 0 and not q[0].any()
    # dividing by a power of two is exact, so smoothing by 2^j equals scaling x
    m = (2.0 ** rng.integers(-3, 4, size=64)).astype(np.float32)
    q1, s1 = oracle.quantize_activations(x, m)
    xs = (x.astype(np.float32) / m).astype(np.float16)  # exact: fp16 range, power-of-two steps
    q2, s2 = oracle.quantize_activations(xs)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_largest_magnitude_maps_to_127_and_codes_in_range():
    x = (rng.standard_normal((8, 256)) * rng.uniform(0.01, 100, size=(8, 1))).astype(np.float16)
    q, s = oracle.quantize_activations(x)
    assert q.dtype == np.int8 and np.abs(q.astype(int)).max() <= 127
    for b in range(8):
        i = int(np.argmax(np.abs(x[b].astype(np.float32))))
        assert abs(int(q[b, i])) == 127
    # power-of-two scaling of a row scales s exactly and leaves q unchanged
    q2, s2 = oracle.quantize_activations((x.astype(np.float32) * 4).astype(np.float16))
    assert np.array_equal(q, q2) and np.array_equal(s2, s * 4)


def test_integer_product_brute_force():
    qx = rng.integers(-127, 128, size=(3, 40)).astype(np.int8)
    qw = rng.integers(-127, 128, size=(5, 40)).astype(np.int8)
    acc = oracle.integer_product(qx, qw)
    for b in range(3):
        for n in range(5):
            assert acc[b, n] == sum(int(qx[b, k]) * int(qw[n, k]) for k in range(40))
    # the largest magnitude the kernel's int32 accumulators meet (k = 16384)
    big = oracle.integer_product(np.full((1, 16384), 127, np.int8), np.full((1, 16384), -127, np.int8))
    assert big[0, 0] == -127 * 127 * 16384 and abs(big[0, 0]) < 2 ** 31


def test_output_error_bound():
    """|y - x W_deq^T| stays inside the RTN bound sum_k (s_x / 2) |W_deq[n, k]|
    plus the fp16 output rounding."""
    B, N, K = 4, 24, 512
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    x = rng.standard_normal((B, K)).astype(np.float16)
    qwt = oracle.quantize("int8", w, K)
    deq = oracle.dequantize(qwt)
    y, acc, qx, sx = oracle.gemm_w8a8(x, qwt.codes, qwt.scales)
    exact = x.astype(np.float64) @ deq.T
    bound = (sx[:, None].astype(np.float64) / 2) @ np.ones((1, K)) @ np.abs(deq).T \
        + np.spacing(np.abs(exact).astype(np.float16)).astype(np.float64) + 1e-6 * np.abs(exact)
    assert np.all(np.abs(y.astype(np.float64) - exact) <= bound)


@pytest.mark.parametrize("mutant", ["floor", "truncate", "transpose", "drop_weight_scale", "exact_quotient",
                                    "one_rounding"])
def test_planted_mistakes_fail_a_pin(mutant, monkeypatch):
    orig_q, orig_p = w8.quantize_activations, w8.integer_product
    if mutant == "exact_quotient":  # the code taken from the binary64 quotient
        def bad(x16, smooth=None):
            q, s = orig_q(x16, smooth)
            a = np.asarray(x16, np.float16).astype(np.float32)
            if smooth is not None:
                a = a / np.asarray(smooth, np.float32)[None, :]
            d = np.where(s > 0, s, 1).astype(np.float64)[:, None]
            qq = np.where(s[:, None] > 0, np.clip(np.rint(a.astype(np.float64) / d), -127, 127), 0).astype(np.int8)
            return qq, s
        monkeypatch.setattr(w8, "quantize_activations", bad)
        monkeypatch.setattr(oracle, "quantize_activations", bad)
    elif mutant == "one_rounding":  # the rescale in binary64, one rounding to fp16
        def bad(x16, qw, sw16, smooth=None):
            qx, sx = w8.quantize_activations(x16, smooth)
            acc = w8.integer_product(qx, qw)
            y = (sx[:, None].astype(np.float64) * np.asarray(sw16, np.float16).astype(np.float64)[None, :]
                 * acc.astype(np.float64)).astype(np.float16)
            return y, acc, qx, sx
        monkeypatch.setattr(w8, "gemm_w8a8", bad)
        monkeypatch.setattr(oracle, "gemm_w8a8", bad)
    elif mutant == "floor":  # rounding down instead of to nearest
        def bad(x16, smooth=None):
            q, s = orig_q(x16, smooth)
            a = np.asarray(x16, np.float16).astype(np.float32)
            qq = np.where(s[:, None] > 0, np.floor(a / np.where(s > 0, s, 1)[:, None]), 0).astype(np.int8)
            return qq, s
        monkeypatch.setattr(w8, "quantize_activations", bad)
        monkeypatch.setattr(oracle, "quantize_activations", bad)
    elif mutant == "truncate":
        def bad(x16, smooth=None):
            q, s = orig_q(x16, smooth)
            a = np.asarray(x16, np.float16).astype(np.float32)
            qq = np.where(s[:, None] > 0, np.trunc(a / np.where(s > 0, s, 1)[:, None]), 0).astype(np.int8)
            return qq, s
        monkeypatch.setattr(w8, "quantize_activations", bad)
        monkeypatch.setattr(oracle, "quantize_activations", bad)
    elif mutant == "transpose":
        def bad(qx, qw):  # activations paired with the wrong k (reversed)
            return orig_p(np.asarray(qx)[:, ::-1], qw)
        monkeypatch.setattr(w8, "integer_product", bad)
        monkeypatch.setattr(oracle, "integer_product", bad)
    else:
        orig_g = w8.gemm_w8a8

        def bad(x16, qw, sw16, smooth=None):
            y, acc, qx, sx = orig_g(x16, qw, np.ones_like(sw16), smooth)
            return y, acc, qx, sx
        monkeypatch.setattr(w8, "gemm_w8a8", bad)
        monkeypatch.setattr(oracle, "gemm_w8a8", bad)
    failed = 0
    for pin in (test_hand_example_scale_ties_and_clamp, test_integer_product_brute_force,
                test_output_error_bound, test_largest_magnitude_maps_to_127_and_codes_in_range,
                test_golden_quotient_rounding_decision, test_golden_rescale_two_roundings,
                test_activation_codes_exact_rational):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"mutant {mutant} passed every pin"
