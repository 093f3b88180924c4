"""Pins of the W8A8 oracle (oracle/w8a8.py) against facts fixed outside it:
hand-worked values, brute-force integer sums, exact invariants of the
per-token quantizer, and the RTN error bound against the fp64 product.
Mutants planted in the oracle (a dropped clamp, a wrong rounding, a
transposed operand, a missing scale) must each fail one of them."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import oracle.w8a8 as w8

rng = np.random.default_rng(2024)


def test_hand_example_scale_ties_and_clamp():
    # absmax 127 gives s = 1 exactly; -63.5 and 2.5 are ties (to even: -64, 2)
    x = np.array([[127.0, -63.5, 2.5, 0.25, -127.0, 0.0]], dtype=np.float16)
    q, s = oracle.quantize_activations(x)
    assert s.tolist() == [1.0]
    assert q.tolist() == [[127, -64, 2, 0, -127, 0]]
    # absmax 2 gives s = 2/127 in binary32; 1.0 maps to rne(63.5 after fp32 division)
    x = np.array([[2.0, 1.0, -1.0]], dtype=np.float16)
    q, s = oracle.quantize_activations(x)
    assert s[0] == np.float32(2.0) / np.float32(127.0)
    assert q[0, 0] == 127 and q[0, 1] == int(np.rint(np.float32(1.0) / s[0])) and q[0, 2] == -q[0, 1]


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


def test_output_formula_and_error_bound():
    """y = f16((s_x s_w) f32(acc)); and |y - x W_deq^T| stays inside the RTN
    bound sum_k (s_x / 2) |W_deq[n, k]| plus the fp16 output rounding."""
    B, N, K = 4, 24, 512
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    x = rng.standard_normal((B, K)).astype(np.float16)
    qwt = oracle.quantize("int8", w, K)
    deq = oracle.dequantize(qwt)
    y, acc, qx, sx = oracle.gemm_w8a8(x, qwt.codes, qwt.scales)
    sw = qwt.scales.astype(np.float32)
    want = ((sx[:, None] * sw[None, :]) * acc.astype(np.float32)).astype(np.float16)
    assert np.array_equal(y.view(np.uint16), want.view(np.uint16))
    exact = x.astype(np.float64) @ deq.T
    bound = (sx[:, None].astype(np.float64) / 2) @ np.ones((1, K)) @ np.abs(deq).T \
        + np.spacing(np.abs(exact).astype(np.float16)).astype(np.float64) + 1e-6 * np.abs(exact)
    assert np.all(np.abs(y.astype(np.float64) - exact) <= bound)


@pytest.mark.parametrize("mutant", ["floor", "truncate", "transpose", "drop_weight_scale"])
def test_planted_mistakes_fail_a_pin(mutant, monkeypatch):
    orig_q, orig_p = w8.quantize_activations, w8.integer_product
    if mutant == "floor":  # rounding down instead of to nearest
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
                test_output_formula_and_error_bound, test_largest_magnitude_maps_to_127_and_codes_in_range):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"mutant {mutant} passed every pin"
