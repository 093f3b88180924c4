"""Pins of the oracle's 3-bit formats (fp3_razer, fp3_afpq) to things other
than themselves (CPU only).

The pages name 3-bit RaZeR ("The Power of Negative Zero", abstract) and
sub-4-bit AFPQ ("AFPQ", abstract) without printing a codebook; the readings
(FP3 = E2M0, specials {+-3, +-8}, scales max/4) are stated in
oracle/formats.py.  Pins:

* every stored scale and selector re-derived with exact rational IEEE
  rounding, and every code by brute force over all 8 codes (tests/exact.py,
  written from the bit-field definitions);
* hand-worked groups with their codes and packed words
  (tests/golden/fp3_examples.json);
* invariants: the remapped code never decodes to 0, positive AFPQ codes
  depend only on s+, AFPQ with equal extremes is symmetric FP3 with
  s = absmax / 4, and the special-value rule regenerates the 4-bit set
  {+-5, +-8} from the E2M1 grid;
* the layout identity the GPU decoder relies on (masks and shifts of the
  three words give E2M1 codes with mantissa 0);
* planted mistakes that these checks catch.
"""

from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import formats as F
from oracle import layout as L
from tests import exact as X

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp3_examples.json")


def _f(v):
    return Fraction(float(v))


def _groups(rng, n, k):
    w = rng.standard_normal((n, k)) * 0.02
    w[rng.random((n, k)) < 0.03] *= 20
    w = w.astype(np.float16)
    if n >= 6:
        w[1, :] = 0
        w[2, :] = np.float16(0.03125)
        w[3, :] = np.float16(2.0 ** -24) * rng.integers(-3, 4, size=k)
        w[4, : k // 2] = np.float16(-0.0)
        w[5, 0], w[5, 1] = np.float16(65504), np.float16(-65504)
    return w


def check_fp3(fmt, w16, g, quantize=None):
    """Re-derive every scale, selector and code of quantize(fmt, w16, g) in
    exact rationals, by brute force over every code."""
    q = (quantize or oracle.quantize)(fmt, w16, g)
    n, k = w16.shape
    for r in range(n):
        for j in range(k // g):
            seg = [_f(v) for v in w16[r, j * g:(j + 1) * g]]
            codes = list(q.codes[r, j * g:(j + 1) * g])
            if fmt == "fp3_afpq":
                sp = X.to_f16(X.to_f32(max(max(seg), Fraction(0)) / 4))
                sn = X.to_f16(X.to_f32(max(-min(seg), Fraction(0)) / 4))
                assert (_f(q.scales[r, j, 0]), _f(q.scales[r, j, 1])) == (sp, sn)
                t = X.afpq3_table(sp, sn)
                assert codes == [X.nearest_code(x, t, X.fp3_prefer) for x in seg], (r, j)
                continue
            amax = max(abs(v) for v in seg)
            per = []
            for v in (3, -3, 8, -8):
                s = X.to_f16(X.to_f32(amax / max(4, abs(v))))
                t = X.razer3_table(s, Fraction(v))
                cs = [X.nearest_code(x, t, X.razer3_prefer) for x in seg]
                per.append((sum(((x - t[c]) ** 2 for x, c in zip(seg, cs)), Fraction(0)), s, cs))
            best = min(range(4), key=lambda c: per[c][0])
            sel = int(q.selectors[r, j])
            tol = per[best][0] * Fraction(1, 10 ** 12)
            assert per[sel][0] - per[best][0] <= tol
            if all(abs(per[c][0] - per[best][0]) > tol for c in range(4) if c != best):
                assert sel == best, (r, j)
            assert _f(q.scales[r, j]) == per[sel][1]
            assert codes == per[sel][2], (r, j)
    return q


@pytest.mark.parametrize("fmt", ["fp3_razer", "fp3_afpq"])
@pytest.mark.parametrize("g", [32, 64])
def test_fp3_bruteforce(fmt, g):
    rng = np.random.default_rng(31 + g)
    check_fp3(fmt, _groups(rng, 8, 2 * g), g)


@pytest.mark.parametrize("fmt", ["fp3_razer", "fp3_afpq"])
def test_fp3_bruteforce_constructed_ties(fmt):
    """Groups whose elements sit exactly on the decision thresholds
    (half-way between FP3 grid values, at the special intervals' ends)."""
    rng = np.random.default_rng(7)
    amax = np.float16(1.0)
    ratios = np.array([0.5, 1.5, 3.0, 2.5, 3.5, 6.0, 0.25, 0.75, 2.0, 4.0, 1.0, 0.125])
    rows = []
    for sgn in (1, -1):
        for base in (4, 8):
            w = np.zeros(32)
            w[0] = amax
            w[1:1 + ratios.size] = sgn * ratios / base
            w[20:] = rng.choice([-1, 1], size=12) * rng.choice(ratios, size=12) / base
            rows.append(w)
    check_fp3(fmt, np.asarray(rows, dtype=np.float16), 32)


def _golden():
    return json.load(open(GOLDEN))["examples"]


@pytest.mark.parametrize("ex", _golden(), ids=lambda e: e["name"])
def test_fp3_hand_examples(ex):
    w = np.zeros((1, 32), dtype=np.float16)
    for i, v in ex["weights"].items():
        w[0, int(i)] = np.float16(v)
    q = oracle.quantize(ex["fmt"], w, 32)
    want = np.zeros(32, dtype=np.int64)
    for i, c in ex["codes"].items():
        want[int(i)] = c
    assert list(q.codes[0]) == list(want)
    assert [float(v) for v in np.ravel(q.scales[0, 0])] == ex["scales"]
    if "selector" in ex:
        assert int(q.selectors[0, 0]) == ex["selector"]
    assert [int(v) for v in oracle.pack(q)["codes"][0]] == ex["words"]


def test_special_rule_regenerates_the_four_bit_set():
    """The reading behind RAZER3_SPECIALS -- midpoint of the two largest grid
    magnitudes, and the first value of the next binade -- applied to the
    E2M1 grid gives the workload's 4-bit candidates {+-5, +-8}."""
    def rule(grid):
        top, second = grid[-1], grid[-2]
        nxt = 2.0 ** np.ceil(np.log2(top + 1e-9))
        nxt = nxt if nxt > top else 2 * nxt
        return {(top + second) / 2, nxt}
    assert rule(F.E2M1_MAGNITUDES) == {abs(v) for v in F.RAZER_SPECIALS}
    assert rule(F.FP3_MAGNITUDES) == {abs(v) for v in F.RAZER3_SPECIALS}
    assert [X.fp3_value(c) for c in range(4)] == [Fraction(int(v)) for v in F.FP3_MAGNITUDES]


def test_razer3_special_never_decodes_to_zero():
    rng = np.random.default_rng(3)
    w = _groups(rng, 16, 256)
    q = oracle.quantize("fp3_razer", w, 64)
    deq = oracle.dequantize(q).reshape(16, 4, 64)
    s = q.scales.astype(np.float64)
    c = q.codes.reshape(16, 4, 64)
    used = (c == 4) & (s[..., None] != 0)
    assert used.any()
    assert np.all(deq[used] != 0)


def test_afpq3_positive_codes_depend_only_on_positive_scale():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((6, 128)) * 0.02).astype(np.float16)
    w[1, :] = 0
    w2 = w.copy()
    neg = w2 < 0
    w2[neg] = (w2[neg].astype(np.float32) * np.float32(1.75)).astype(np.float16)  # only s- changes
    q1, q2 = oracle.quantize("fp3_afpq", w, 64), oracle.quantize("fp3_afpq", w2, 64)
    pos = w > 0
    assert np.array_equal(q1.codes[pos], q2.codes[pos])
    assert np.array_equal(q1.scales[..., 0], q2.scales[..., 0])


def test_afpq3_with_equal_extremes_is_symmetric_fp3():
    """max+ = max-: both scales are absmax / 4, and every code is the nearest
    symmetric FP3 value (brute force with one scale)."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((4, 64)) * 0.02).astype(np.float16)
    w[:, 0], w[:, 1] = np.float16(0.09375), np.float16(-0.09375)
    w = np.clip(w, -0.09375, 0.09375).astype(np.float16)
    q = oracle.quantize("fp3_afpq", w, 64)
    s = X.to_f16(X.to_f32(Fraction(3, 32) / 4))
    t = {c: X.fp3_value(c) * s for c in range(8)}
    for r in range(4):
        assert _f(q.scales[r, 0, 0]) == s == _f(q.scales[r, 0, 1])
        assert list(q.codes[r]) == [X.nearest_code(_f(x), t, X.fp3_prefer) for x in w[r]]


def test_layout_identity_gives_e2m1_codes():
    """Word q div 2 masked with 0x66666666 (rotated right by 2 for odd q) or
    the sign word shifted left by q and masked with 0x88888888 is the q-th
    group of eight codes as E2M1 codes sign<<3 | index<<1 -- the identity
    the GPU decoder uses -- and that E2M1 code decodes to the same value."""
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 8, size=(3, 64))
    words = L._pack_fp3(codes).reshape(3, 2, 3)
    rotr2 = lambda v: ((v >> 2) | (v << 30)) & 0xFFFFFFFF
    for r in range(3):
        for p in range(2):
            w0, w1, sg = (int(v) for v in words[r, p])
            for qq in range(4):
                src = (w0, w1)[qq // 2]
                src = rotr2(src) if qq % 2 else src
                nib = (src & 0x66666666) | ((sg << qq) & 0x88888888)
                for n in range(8):
                    c = int(codes[r, 32 * p + 8 * qq + n])
                    e2m1 = (nib >> (4 * n)) & 0xF
                    assert e2m1 == ((c >> 2) << 3) | ((c & 3) << 1)
                    assert X.e2m1_value(e2m1) == X.fp3_value(c)


@pytest.mark.parametrize("fmt", ["fp3_razer", "fp3_afpq"])
def test_fp3_pack_roundtrip_and_sizes(fmt):
    rng = np.random.default_rng(8)
    w = _groups(rng, 7, 320)
    q = oracle.quantize(fmt, w, 32)
    buf = oracle.pack(q)
    q2 = oracle.unpack(fmt, 7, 320, 32, buf)
    assert np.array_equal(q.codes, q2.codes)
    assert np.array_equal(oracle.dequantize(q), oracle.dequantize(q2))
    sizes = oracle.packed_nbytes(fmt, 7, 320, 32)
    assert sizes["codes"] == 7 * 10 * 12 == buf["codes"].nbytes  # 32 codes per 3 dwords
    assert sizes["scales"] == buf["scales"].nbytes
    if fmt == "fp3_razer":
        assert sizes["aux"] == buf["aux"].nbytes == 7 * 4


def test_fp3_planted_mistakes_are_caught(monkeypatch):
    rng = np.random.default_rng(9)
    w = _groups(rng, 6, 64)
    # ties to the odd index
    with monkeypatch.context() as m:
        real = F._nearest_magnitude_index

        def odd(mag, scale, table=None):
            table = F.E2M1_MAGNITUDES if table is None else table
            cand = table * scale[..., None]
            dist = np.abs(mag[..., None] - cand)
            tied = dist == dist.min(axis=-1, keepdims=True)
            return table.size - 1 - tied[..., ::-1].argmax(axis=-1)
        m.setattr(F, "_nearest_magnitude_index", odd)
        with pytest.raises(AssertionError):
            for g_ex in _golden():
                test_fp3_hand_examples(g_ex)
        m.setattr(F, "_nearest_magnitude_index", real)
    # the 4-bit special set reused for 3 bits
    with monkeypatch.context() as m:
        m.setattr(F, "RAZER3_SPECIALS", (5.0, -5.0, 8.0, -8.0))
        with pytest.raises(AssertionError):
            check_fp3("fp3_razer", w, 32)
    # the E2M1 divisor (6) for the FP3 scale
    with monkeypatch.context() as m:
        m.setattr(F, "FP3_MAX", 6.0)
        with pytest.raises(AssertionError):
            check_fp3("fp3_afpq", w, 32)
    # sign bits in the wrong order inside the sign word
    with monkeypatch.context() as m:
        real_pos = L._fp3_positions
        m.setattr(L, "_fp3_positions", lambda e: real_pos(e)[:3] + (4 * (e % 8) + e // 8,))
        with pytest.raises(AssertionError):
            test_layout_identity_gives_e2m1_codes()
