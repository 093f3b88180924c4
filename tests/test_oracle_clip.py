"""Pins of the oracle's per-group clipping search (oracle.quantize_clipped),
for INT4 asym, E2M1, AFPQ and RaZeR.

The pages name clipping but fix no procedure, so the ratio grid (20 - c)/20
and the tie order are the reading taken here (parity unpinned by the pages).
What is pinned independently of the oracle's own code:

* one candidate is plain RTN, which the format pins already fix;
* the chosen candidate's SSE is never above plain RTN's (the search's
  purpose), measured on the dequantized values by a plain fp64 sum;
* brute force from the definition on small inputs: every candidate's codes
  and SSE in exact rational arithmetic (fractions.Fraction, exact
  round-half-even), the minimum taken exactly, compared with the oracle's
  choice wherever the exact minimum is clear of the fp64 rounding;
* on heavy-tailed groups some clipping is chosen, and never on a group whose
  values all lie on the plain RTN grid (SSE 0 already);
* planted mistakes in the oracle (argmax for argmin, the ratio applied to one
  bound only, a shifted ratio grid) each fail one of these pins.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import formats as F

FMTS = ("int4_asym", "fp4_e2m1", "fp4_afpq", "fp4_razer")


def _weights(seed, n, k, heavy=False):
    rng = np.random.default_rng(seed)
    w = rng.standard_t(3, size=(n, k)) * 0.02 if heavy else rng.standard_normal((n, k)) * 0.02
    return w.astype(np.float16)


def _group_sse(q, w16):
    deq = oracle.dequantize(q).reshape(q.n, q.k // q.group, q.group)
    w = w16.astype(np.float64).reshape(deq.shape)
    return ((w - deq) ** 2).sum(axis=-1)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("g", [32, 64, 128, 256])
def test_one_candidate_is_plain_rtn(fmt, g):
    w = _weights(1 + g, 6, 512, heavy=True)
    a, b = oracle.quantize_clipped(fmt, w, g, 1), oracle.quantize(fmt, w, g)
    assert np.array_equal(a.codes, b.codes)
    assert np.array_equal(a.scales.view(np.uint16), b.scales.view(np.uint16))
    if fmt == "int4_asym":
        assert np.array_equal(a.zeros, b.zeros)
    if fmt == "fp4_razer":
        assert np.array_equal(a.selectors, b.selectors)


@pytest.mark.parametrize("fmt", FMTS)
def test_search_never_worse_and_clips_heavy_tails(fmt):
    w = _weights(7, 64, 1024, heavy=True)
    plain = _group_sse(oracle.quantize(fmt, w, 128), w)
    clipped = _group_sse(oracle.quantize_clipped(fmt, w, 128, 10), w)
    assert np.all(clipped <= plain * (1 + 1e-12))
    assert np.mean(clipped < plain * (1 - 1e-9)) > 0.2  # heavy tails: clipping pays in many groups


@pytest.mark.parametrize("fmt", FMTS)
def test_groups_on_the_grid_are_not_clipped(fmt):
    rng = np.random.default_rng(3)
    n, g = 8, 32
    if fmt == "int4_asym":  # values (q - 7) * 0.5 with the extremes present: scale 0.5, zero 7
        q = rng.integers(0, 16, size=(n, g))
        q[:, 0], q[:, 1] = 0, 15
        w = ((q - 7) * 0.5).astype(np.float16)
    else:  # signed E2M1 values with +6 and -6 present: every scale 1 (RaZeR: no special is nearer)
        mags = F.E2M1_MAGNITUDES[rng.integers(0, 8, size=(n, g))]
        w = (mags * rng.choice([-1.0, 1.0], size=(n, g))).astype(np.float16)
        w[:, 0], w[:, 1] = 6.0, -6.0
    q = oracle.quantize_clipped(fmt, w, g, 10)
    assert np.array_equal(q.codes, oracle.quantize(fmt, w, g).codes)
    assert np.all(_group_sse(q, w) == 0)


# ------------------------------------------------------------ brute force --

def _rne(fr: Fraction) -> int:
    """Round half to even of an exact rational."""
    f = fr.numerator // fr.denominator
    rem = fr - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return f


def _bound(v, c):  # the ratio (20 - c)/20 in binary32: exact product, one rounded division
    return np.float32(np.float32(v) * np.float32(20 - c)) / np.float32(20)


def _int4_exact(wg, c):
    lo = min(np.float32(wg.astype(np.float32).min()), np.float32(0))
    hi = max(np.float32(wg.astype(np.float32).max()), np.float32(0))
    lo_c, hi_c = _bound(lo, c), _bound(hi, c)
    s = Fraction(float(np.float16(np.float32(hi_c - lo_c) / np.float32(15))))
    if s == 0:
        return [0] * len(wg), s, 0, sum(Fraction(float(x)) ** 2 for x in wg)
    z = min(max(_rne(-Fraction(float(lo_c)) / s), 0), 15)
    codes, sse = [], Fraction(0)
    for x in wg:
        q = min(max(z + _rne(Fraction(float(x)) / s), 0), 15)
        codes.append(q)
        sse += (Fraction(float(x)) - (q - z) * s) ** 2
    return codes, s, z, sse


def _e2m1_exact(wg, c):
    a = np.float32(np.abs(wg.astype(np.float32)).max())
    s = Fraction(float(np.float16(_bound(a, c) / np.float32(6))))
    mags = [Fraction(m).limit_denominator(2) for m in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    codes, sse = [], Fraction(0)
    for x in wg:
        fx = Fraction(float(x))
        dist = [abs(abs(fx) - m * s) for m in mags]
        best = min(dist)
        ties = [i for i, d in enumerate(dist) if d == best]
        idx = next((i for i in ties if i % 2 == 0), ties[0])
        codes.append(((8 if (fx < 0 and idx > 0) else 0) | idx))
        val = mags[idx] * s
        sse += (fx - (-val if fx < 0 else val)) ** 2
    return codes, s, None, sse


_MAGS = [Fraction(m).limit_denominator(2) for m in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]


def _nearest(fx, s):
    """Signed E2M1 code and value of fx under scale s, ties to the even index."""
    dist = [abs(abs(fx) - m * s) for m in _MAGS]
    best = min(dist)
    ties = [i for i, d in enumerate(dist) if d == best]
    idx = next((i for i in ties if i % 2 == 0), ties[0])
    val = _MAGS[idx] * s
    return ((8 if (fx < 0 and idx > 0) else 0) | idx), (-val if fx < 0 else val)


def _afpq_exact(wg, c):
    w32 = wg.astype(np.float32)
    pos = max(np.float32(w32.max()), np.float32(0))
    neg = max(np.float32(-w32.min()), np.float32(0))
    sp = Fraction(float(np.float16(_bound(pos, c) / np.float32(6))))
    sn = Fraction(float(np.float16(_bound(neg, c) / np.float32(6))))
    codes, sse = [], Fraction(0)
    for x in wg:
        fx = Fraction(float(x))
        code, val = _nearest(fx, sn if fx < 0 else sp)
        codes.append(code)
        sse += (fx - val) ** 2
    return codes, (sp, sn), None, sse


def _razer_exact(wg, c, v):
    a = np.float32(np.abs(wg.astype(np.float32)).max())
    s = Fraction(float(np.float16(_bound(a, c) / np.float32(max(6.0, abs(v))))))
    codes, sse = [], Fraction(0)
    for x in wg:
        fx = Fraction(float(x))
        code, val = _nearest(fx, s)
        spec = Fraction(v) * s
        if abs(fx - spec) < abs(fx - val):  # the special value only when strictly nearer
            code, val = 8, spec
        codes.append(code)
        sse += (fx - val) ** 2
    return codes, s, None, sse


@pytest.mark.parametrize("fmt", FMTS)
def test_brute_force_exact_rational(fmt):
    g, cands = 32, 10
    w = _weights(11, 3, 128, heavy=True)
    if fmt == "fp4_razer":
        cands = 5  # 20 candidates per group with the four specials
    got = oracle.quantize_clipped(fmt, w, g, cands)
    checked = 0
    for r in range(w.shape[0]):
        for gi in range(w.shape[1] // g):
            wg = w[r, gi * g:(gi + 1) * g]
            if fmt == "fp4_razer":
                res = [_razer_exact(wg, c, v) for c in range(cands) for v in F.RAZER_SPECIALS]
            else:
                exact = {"int4_asym": _int4_exact, "fp4_e2m1": _e2m1_exact, "fp4_afpq": _afpq_exact}[fmt]
                res = [exact(wg, c) for c in range(cands)]
            sses = [x[3] for x in res]
            m = min(sses)
            best = sses.index(m)
            runner = min((x for i, x in enumerate(sses) if i != best), default=None)
            if runner is not None and m > 0 and (runner - m) / m < Fraction(1, 10 ** 9):
                continue  # a near tie: fp64 may order it either way
            codes, s, z, _ = res[best]
            assert list(got.codes[r, gi * g:(gi + 1) * g]) == codes, (r, gi, best)
            if fmt == "fp4_afpq":
                assert (Fraction(float(got.scales[r, gi, 0])), Fraction(float(got.scales[r, gi, 1]))) == s
            else:
                assert Fraction(float(got.scales[r, gi])) == s
            if z is not None:
                assert got.zeros[r, gi] == z
            if fmt == "fp4_razer":
                assert got.selectors[r, gi] == best % 4
            checked += 1
    assert checked >= 9


# ------------------------------------------------------------------ mutants --

@pytest.mark.parametrize("mutant", ["argmax", "hi_only", "shifted_grid"])
def test_planted_mistakes_fail_a_pin(mutant, monkeypatch):
    if mutant == "argmax":
        real_stack = np.stack

        class _Neg(np.ndarray):
            def argmin(self, axis=None, **kw):
                return np.asarray(self).argmax(axis=axis)

        monkeypatch.setattr(F.np, "stack", lambda a, axis=0: real_stack(a, axis=axis).view(_Neg))
    elif mutant == "hi_only":  # the ratio shrinks the upper bound only (lo <= 0 stays)
        real_bound = F.clip_bound
        monkeypatch.setattr(F, "clip_bound", lambda v, c: np.where(np.asarray(v) > 0, real_bound(v, c),
                                                                   np.asarray(v, dtype=np.float32)))
    else:
        real_bound = F.clip_bound
        monkeypatch.setattr(F, "clip_bound", lambda v, c: real_bound(v, c + 1))
    failed = 0
    for pin in (lambda: test_one_candidate_is_plain_rtn("int4_asym", 32),
                lambda: test_search_never_worse_and_clips_heavy_tails("int4_asym"),
                lambda: test_brute_force_exact_rational("int4_asym")):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"mutant {mutant} passed every pin"

