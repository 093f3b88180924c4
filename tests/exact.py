"""Exact-arithmetic reference pieces used to pin the oracle (tests only).

Written independently of ``oracle/``: IEEE round-to-nearest-even onto binary32
and binary16 from exact rationals, the format code tables from their bit-field
definitions, and a brute-force nearest-code search over every code of a
format with the tie rules stated in the header (ties to the even integer /
even E2M1 mantissa bit, +0 for zero, RaZeR special only when strictly
nearer).
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np


def round_ieee(x: Fraction, mant_bits: int, emin: int, emax: int) -> Fraction:
    """Round x to the nearest binary floating-point value with ``mant_bits``
    stored fraction bits, minimum normal exponent ``emin`` (subnormals below)
    and maximum exponent ``emax``; ties to even; overflow -> inf (not used)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - mant_bits)
    q = a / ulp
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r >= Fraction(2) ** (emax + 1):
        raise OverflowError
    return sign * r


def to_f32(x: Fraction) -> Fraction:
    return round_ieee(x, 23, -126, 127)


def to_f16(x: Fraction) -> Fraction:
    return round_ieee(x, 10, -14, 15)


def frac(v) -> Fraction:
    return Fraction(float(v))


# ---- code tables from bit-field definitions ---------------------------------

def e2m1_value(code: int) -> Fraction:
    """Unit-scale value of a 4-bit E2M1 code: sign bit 3, exponent bits 2..1
    (bias 1), mantissa bit 0; exponent 0 is subnormal (0 or 0.5)."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return -mag if s else mag


def nearest_code(w: Fraction, table: dict, prefer) -> int:
    """Code whose value in ``table`` (code -> Fraction) is nearest to w; among
    exact ties the code with the smallest ``prefer(code)`` key wins."""
    best = None
    for c, v in table.items():
        key = (abs(w - v), prefer(c))
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def int4_table(z: int, s: Fraction) -> dict:
    return {q: (q - z) * s for q in range(16)}


def int4_prefer(z: int):
    return lambda q: (q - z) % 2  # even (q - z) wins a tie


def e2m1_table(s: Fraction) -> dict:
    return {c: e2m1_value(c) * s for c in range(16)}


def e2m1_prefer(c: int):
    # even magnitude index (mantissa bit 0) first, then +0 over -0
    return ((c & 1), (c >> 3) & 1)


def razer_table(s: Fraction, v: Fraction) -> dict:
    t = {c: e2m1_value(c) * s for c in range(16) if c != 8}
    t[8] = v * s
    return t


def razer_prefer(c: int):
    return (1 if c == 8 else 0, c & 1, (c >> 3) & 1)


def afpq_table(sp: Fraction, sn: Fraction) -> dict:
    return {c: (e2m1_value(c) * (sn if c & 8 else sp)) for c in range(16)}


def bfp_table(mb: int, step: Fraction) -> dict:
    lim = (1 << mb) - 1
    return {m: m * step for m in range(-lim, lim + 1)}


def int8_table(s: Fraction) -> dict:
    return {q: q * s for q in range(-127, 128)}


def even_int_prefer(q: int):
    return q % 2


def sum_exact(values) -> Fraction:
    return sum((Fraction(float(v)) for v in values), Fraction(0))


def f16_array(vals) -> np.ndarray:
    return np.asarray(vals, dtype=np.float16)


# ---- 3-bit FP (E2M0) -----------------------------------------------------------

def fp3_value(code: int) -> Fraction:
    """Unit-scale value of a 3-bit FP code: sign bit 2, exponent bits 1..0
    (bias 1), no mantissa; exponent 0 is zero."""
    s = (code >> 2) & 1
    e = code & 3
    mag = Fraction(0) if e == 0 else Fraction(2) ** (e - 1)
    return -mag if s else mag


def fp3_prefer(c: int):
    # even index (exponent bit 0 clear) first, then +0 over -0
    return (c & 1, (c >> 2) & 1)


def razer3_table(s: Fraction, v: Fraction) -> dict:
    t = {c: fp3_value(c) * s for c in range(8) if c != 4}
    t[4] = v * s
    return t


def razer3_prefer(c: int):
    return (1 if c == 4 else 0, c & 1, (c >> 2) & 1)


def afpq3_table(sp: Fraction, sn: Fraction) -> dict:
    return {c: fp3_value(c) * (sn if c & 4 else sp) for c in range(8)}
