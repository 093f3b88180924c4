"""Logical RTN quantizers and decoders for every format (test infrastructure).

Each ``quantize_*`` takes fp16 weights ``w`` of shape [N, K] (row = output
channel, groups run along K) and returns a :class:`Quantized` holding the
logical codes and metadata; :func:`dequantize` maps them back to exact fp64
values.  Byte layout lives in ``layout.py``.

Arithmetic conventions (our reading; the pages print no formulas):

* fp16 inputs widen to fp32 exactly.  Every scale formula is evaluated in IEEE
  binary32 with one rounding per operation (numpy float32), then rounded once
  to binary16 with round-to-nearest-even.  Codes are chosen against the stored
  fp16 scale, so decoding the codes with the stored metadata gives back exactly
  the candidate set they were chosen from.
* Round-to-nearest ties go to the even neighbour: the even integer for the INT
  formats and the block mantissas, the even magnitude index (mantissa bit 0)
  for E2M1.  Under RaZeR the special value must be strictly nearer to win.
* An element whose magnitude rounds to zero gets the +0 code (sign bit 0).
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

FORMATS = ("int4_asym", "fp4_e2m1", "fp4_razer", "fp4_afpq", "bfp6", "bfp4", "int8", "fp3_razer", "fp3_afpq")

# E2M1 magnitudes by 3-bit index (2 exponent bits, bias 1, 1 mantissa bit;
# exponent field 0 is subnormal: 0 and 0.5).  Sign-magnitude gives 16 codes
# with both +0 (0b0000) and -0 (0b1000) -- the redundancy RaZeR reuses
# (Chen et al., "The Power of Negative Zero", abstract).
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0

# RaZeR candidate special values, in selector order 0..3.  The set {+-5, +-8}
# is the workload's stated candidate list; the page itself fixes only that
# the redundant negative-zero code takes a value picked per group from a
# fixed list.
RAZER_SPECIALS = (5.0, -5.0, 8.0, -8.0)

# FP3 magnitudes by 2-bit index: the E2M1 grid without its mantissa bit
# (2 exponent bits, bias 1, exponent field 0 is zero) -- E2M0.  Sign-magnitude
# gives 8 codes with +0 (0b000) and -0 (0b100).  "The Power of Negative Zero"
# (abstract) names 3-bit FP as the precision where the redundant zero costs
# most, and "AFPQ" (abstract) sub-4-bit FP; neither prints a 3-bit codebook,
# so this grid is the reading taken here: the plainest 3-bit member of the
# family whose 4-bit member (E2M1) the workloads fix.
FP3_MAGNITUDES = np.array([0.0, 1.0, 2.0, 4.0], dtype=np.float64)
FP3_MAX = 4.0

# 3-bit RaZeR candidate special values, selector order 0..3.  Reading: the
# rule that turns the E2M1 grid into the workload's 4-bit set {+-5, +-8} --
# the midpoint of the two largest magnitudes (4 and 6 -> 5) and the first
# value of the next binade above the grid (8) -- applied to the FP3 grid:
# (2 + 4) / 2 = 3 and 8.
RAZER3_SPECIALS = (3.0, -3.0, 8.0, -8.0)

# Block formats: block length along K and mantissa magnitude bits.
BFP_BLOCK = 16
BFP_MANT_BITS = {"bfp6": 5, "bfp4": 3}
BFP_EXP_BIAS = 127

INT4_QMAX = 15
INT8_QMAX = 127


@dataclass
class Quantized:
    """Logical result of RTN quantization of one [N, K] weight matrix."""

    fmt: str
    n: int
    k: int
    group: int
    codes: np.ndarray  # int64 [N, K]: 4-bit patterns (INT4, E2M1 family), 3-bit
    #                    patterns (FP3 family) or signed integers (block mantissas, INT8)
    scales: Optional[np.ndarray] = None  # float16: [N,K/g], AFPQ [N,K/64,2], INT8 [N]
    zeros: Optional[np.ndarray] = None  # int64 [N, K/g]   (INT4)
    selectors: Optional[np.ndarray] = None  # int64 [N, K/g] (RaZeR)
    exps: Optional[np.ndarray] = None  # uint8 [N, K/16] (block formats)


# ----------------------------------------------------------------- helpers --

def _f16_from_f32(x32: np.ndarray) -> np.ndarray:
    """Round binary32 values once to binary16 (round-to-nearest-even)."""
    assert x32.dtype == np.float32
    return x32.astype(np.float16)


def _grouped(w: np.ndarray, g: int) -> np.ndarray:
    n, k = w.shape
    return w.reshape(n, k // g, g)


def _nearest_magnitude_index(mag: np.ndarray, scale: np.ndarray, table: Optional[np.ndarray] = None) -> np.ndarray:
    """Index into ``table`` (E2M1_MAGNITUDES, or FP3_MAGNITUDES) of the value
    M[i]*scale nearest to ``mag``.

    ``mag`` >= 0 (fp64, exact fp16 values); ``scale`` broadcasts against ``mag``
    and holds exact fp16 scales.  Each distance |mag - M[i]*scale| is exact in
    fp64 (both terms are multiples of 2^-25 below 2^19).  On an exact tie
    between two neighbours the even index wins; when scale is 0 every
    candidate ties and index 0 (the zero code) wins.
    """
    if table is None:
        table = E2M1_MAGNITUDES
    cand = table * scale[..., None]
    dist = np.abs(mag[..., None] - cand)
    best = dist.min(axis=-1, keepdims=True)
    tied = dist == best
    even = (np.arange(table.size) % 2) == 0
    tied_even = tied & even
    return np.where(tied_even.any(axis=-1), tied_even.argmax(axis=-1), tied.argmax(axis=-1))


def _rne_quotient(w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """round-half-even(w / s) for w an fp16 (or binary32) value and s > 0 an
    fp16 value.

    The fp64 quotient lands on the same side of every half-integer as the exact
    quotient: h*s is exact, and when w/s is not itself a half-integer h, w - h*s
    is a non-zero multiple of the finer of the two values' last-bit units, so
    w/s lies at least 2^-26 from h, far more than the fp64 rounding error of a
    quotient below 2^5; when it is one the fp64 quotient is exact.  np.rint
    rounds halves to even.
    """
    return np.rint(w / s)


def _tree_sum_last_axis(a: np.ndarray) -> np.ndarray:
    """Sum over the last axis (power-of-two length) by repeated halving:
    a <- a[:h] + a[h:], fp64, until one element is left."""
    while a.shape[-1] > 1:
        h = a.shape[-1] // 2
        a = a[..., :h] + a[..., h:]
    return a[..., 0]


def _e2m1_codes(w64: np.ndarray, scale64: np.ndarray) -> np.ndarray:
    """Signed E2M1 codes (sign<<3 | index) of w against one scale per group."""
    idx = _nearest_magnitude_index(np.abs(w64), scale64)
    sign = (w64 < 0) & (idx > 0)
    return (sign.astype(np.int64) << 3) | idx


def _e2m1_values(codes: np.ndarray) -> np.ndarray:
    """Unit-scale E2M1 value of each code (code 8 -> -0.0, i.e. 0)."""
    mag = E2M1_MAGNITUDES[codes & 7]
    return np.where((codes & 8) != 0, -mag, mag)


# ------------------------------------------------------------- quantizers --

def _int4_asym_candidate(w16: np.ndarray, g: int, lo: np.ndarray, hi: np.ndarray):
    """INT4 codes of the groups of w16 for the range [lo, hi] (binary32 per
    group, lo <= 0 <= hi).  Returns (codes, stored fp16 scale, zero-points,
    fp64 dequantized values, fp64 SSE summed by repeated halving).
    s = f16((hi - lo) / 15); z = clamp(rne(-lo/s), 0, 15);
    q = clamp(z + rne(w/s), 0, 15); value = (q - z) * s; s = 0 gives z = q = 0."""
    s16 = _f16_from_f32((hi - lo) / np.float32(INT4_QMAX))
    s = s16.astype(np.float64)
    nz = s > 0
    safe = np.where(nz, s, 1.0)
    z = np.where(nz, np.clip(_rne_quotient(-lo.astype(np.float64), safe), 0, INT4_QMAX), 0)
    wg64 = _grouped(w16, g).astype(np.float64)
    j = _rne_quotient(wg64, safe[..., None])
    q = np.clip(z[..., None] + j, 0, INT4_QMAX)
    q = np.where(nz[..., None], q, 0).astype(np.int64)
    deq = (q - z[..., None]) * s[..., None]
    sse = _tree_sum_last_axis((wg64 - deq) ** 2)
    return q, s16, z.astype(np.int64), deq, sse


def quantize_int4_asym(w16: np.ndarray, g: int) -> Quantized:
    """Asymmetric INT4 RTN per group: fp16 scale and 4-bit integer zero-point.

    Asymmetric INT is the comparison format of "The Power of Negative Zero"
    (abstract) and the storage baseline of "AFPQ" (abstract); RTN per group is
    the method of "Is (Selective) Round-To-Nearest Quantization All You Need?".
    Reading: the range is [min(w,0), max(w,0)] so that 0 is on the grid and a
    constant group is handled; s = f16((hi - lo) / 15); z = clamp(rne(-lo/s),
    0, 15); q = clamp(z + rne(w/s), 0, 15); value = (q - z) * s.  If s is 0 the
    group is all zero: z = 0, q = 0.
    """
    n, k = w16.shape
    wg32 = _grouped(w16, g).astype(np.float32)
    lo = np.minimum(wg32.min(axis=-1), np.float32(0))
    hi = np.maximum(wg32.max(axis=-1), np.float32(0))
    q, s16, z, _, _ = _int4_asym_candidate(w16, g, lo, hi)
    return Quantized("int4_asym", n, k, g, q.reshape(n, k), scales=s16, zeros=z)


def _e2m1_candidate(w16: np.ndarray, g: int, absmax32: np.ndarray):
    """E2M1 codes of the groups of w16 for the range absmax (binary32 per
    group).  Returns (codes, stored fp16 scale, fp64 SSE summed by repeated
    halving).  s = f16(absmax / 6); each element takes the nearest of
    {+-M[i] s}, saturating at 6 s."""
    wg64 = _grouped(w16, g).astype(np.float64)
    s16 = _f16_from_f32(absmax32 / np.float32(E2M1_MAX))
    s = s16.astype(np.float64)[..., None]
    codes = _e2m1_codes(wg64, s)
    sse = _tree_sum_last_axis((wg64 - _e2m1_values(codes) * s) ** 2)
    return codes, s16, sse


def quantize_fp4_e2m1(w16: np.ndarray, g: int) -> Quantized:
    """FP4 E2M1 RTN per group with an fp16 absmax scale s = f16(absmax / 6).

    Each element takes the nearest of the 15 distinct values {+-M[i]*s}
    (ties to the even magnitude index, saturating at 6*s); the sign-magnitude
    form with two zeros is the FP4 datatype of "The Power of Negative Zero"
    (abstract).
    """
    n, k = w16.shape
    absmax32 = np.abs(_grouped(w16, g).astype(np.float32)).max(axis=-1)
    codes, s16, _ = _e2m1_candidate(w16, g, absmax32)
    return Quantized("fp4_e2m1", n, k, g, codes.reshape(n, k), scales=s16)


# --------------------------------------------------------- clipping search --

CLIP_DENOM = 20
CLIP_MAX_CANDIDATES = 10


def clip_bound(v32: np.ndarray, c: int) -> np.ndarray:
    """Range bound v scaled by the clip ratio (20 - c) / 20, in binary32:
    v * (20 - c) is exact (v is an fp16 value, 20 - c has 5 bits), then one
    correctly rounded division by 20.  c = 0 returns v itself."""
    v32 = np.asarray(v32, dtype=np.float32)
    return (v32 * np.float32(CLIP_DENOM - c)) / np.float32(CLIP_DENOM)


def quantize_clipped(fmt: str, w16: np.ndarray, g: int, candidates: int) -> Quantized:
    """RTN with a data-free per-group clipping search (INT4 asym, E2M1, AFPQ,
    RaZeR).

    "The Power of Negative Zero" (abstract) says its datatype can be combined
    with clipping but gives no procedure; the search below, including its
    grid of ratios, is this project's own reading, the plainest data-free
    one: for c = 0 .. candidates - 1 the group's
    range is shrunk by the ratio (20 - c) / 20 (:func:`clip_bound`), the group
    is quantized by RTN on the shrunk range exactly as the format's quantizer
    does (values beyond it saturate), and the candidate with the smallest fp64
    SSE against the fp16 weights is kept; on equal SSE the smaller c wins (less
    clipping).  AFPQ shrinks both one-sided ranges by the same ratio; RaZeR
    shrinks the absmax and tries its four special values under each ratio
    (ties: the smaller c, then the earlier special).  candidates = 1 is plain
    RTN.  The stored format is unchanged: only the scales (and INT4
    zero-points, RaZeR selectors) and codes differ.
    """
    if not 1 <= candidates <= CLIP_MAX_CANDIDATES:
        raise ValueError(f"candidates must be in 1..{CLIP_MAX_CANDIDATES}")
    w16 = np.asarray(w16, dtype=np.float16)
    n, k = w16.shape
    wg32 = _grouped(w16, g).astype(np.float32)
    if fmt == "int4_asym":
        lo = np.minimum(wg32.min(axis=-1), np.float32(0))
        hi = np.maximum(wg32.max(axis=-1), np.float32(0))
        res = [_int4_asym_candidate(w16, g, clip_bound(lo, c), clip_bound(hi, c)) for c in range(candidates)]
        sse = np.stack([r[4] for r in res], axis=-1)
        best = sse.argmin(axis=-1)  # first minimum: the least clipping
        q = np.choose(best[..., None], [r[0] for r in res])
        s16 = np.choose(best, [r[1] for r in res]).astype(np.float16)
        z = np.choose(best, [r[2] for r in res]).astype(np.int64)
        return Quantized("int4_asym", n, k, g, q.reshape(n, k), scales=s16, zeros=z)
    if fmt == "fp4_e2m1":
        absmax32 = np.abs(wg32).max(axis=-1)
        res = [_e2m1_candidate(w16, g, clip_bound(absmax32, c)) for c in range(candidates)]
        sse = np.stack([r[2] for r in res], axis=-1)
        best = sse.argmin(axis=-1)
        codes = np.choose(best[..., None], [r[0] for r in res])
        s16 = np.choose(best, [r[1] for r in res]).astype(np.float16)
        return Quantized("fp4_e2m1", n, k, g, codes.reshape(n, k), scales=s16)
    if fmt == "fp4_afpq":  # both one-sided ranges shrink by the same ratio
        pos32 = np.maximum(wg32.max(axis=-1), np.float32(0))
        neg32 = np.maximum(-wg32.min(axis=-1), np.float32(0))
        res = [_afpq_candidate(w16, g, clip_bound(pos32, c), clip_bound(neg32, c)) for c in range(candidates)]
        sse = np.stack([r[2] for r in res], axis=-1)
        best = sse.argmin(axis=-1)
        codes = np.choose(best[..., None], [r[0] for r in res])
        sp = np.choose(best, [r[1][..., 0] for r in res])
        sn = np.choose(best, [r[1][..., 1] for r in res])
        return Quantized("fp4_afpq", n, k, g, codes.reshape(n, k),
                         scales=np.stack([sp, sn], axis=-1).astype(np.float16))
    if fmt == "fp4_razer":  # the absmax shrinks, then every special value is tried under it
        wg64 = wg32.astype(np.float64)
        absmax32 = np.abs(wg32).max(axis=-1)
        res = [razer_candidate(wg64, clip_bound(absmax32, c), v) for c in range(candidates) for v in RAZER_SPECIALS]
        sse = np.stack([r[3] for r in res], axis=-1)  # candidate index = 4 c + selector
        best = sse.argmin(axis=-1)  # first minimum: the least clipping, then the earlier special
        codes = np.choose(best[..., None], [r[0] for r in res])
        s16 = np.choose(best, [r[1] for r in res]).astype(np.float16)
        return Quantized("fp4_razer", n, k, g, codes.reshape(n, k), scales=s16,
                         selectors=(best % len(RAZER_SPECIALS)).astype(np.int64))
    raise ValueError(f"no clipping search for format {fmt!r}")


def razer_candidate(wg64: np.ndarray, absmax32: np.ndarray, v: float):
    """Quantize groups under one RaZeR candidate special value ``v``.

    Returns (codes, stored fp16 scale, fp64 dequantized values, fp64 SSE).
    Scale reading: s_v = f16(absmax / max(6, |v|)), so the special value can
    reach the group's extreme (with absmax/6 a candidate of 8 could never win).
    An element takes code 0b1000 (decoding to v*s_v) only when v*s_v is
    strictly nearer than its nearest standard E2M1 value.  SSE is the fp64 sum
    of squared errors over the group, summed by repeated halving.
    """
    s16 = _f16_from_f32(absmax32 / np.float32(max(E2M1_MAX, abs(v))))
    s = s16.astype(np.float64)[..., None]
    std_codes = _e2m1_codes(wg64, s)
    std_vals = _e2m1_values(std_codes) * s
    spec_val = v * s
    use_spec = np.abs(wg64 - spec_val) < np.abs(wg64 - std_vals)
    codes = np.where(use_spec, 8, std_codes)
    deq = np.where(use_spec, spec_val, std_vals)
    sse = _tree_sum_last_axis((wg64 - deq) ** 2)
    return codes, s16, deq, sse


def quantize_fp4_razer(w16: np.ndarray, g: int) -> Quantized:
    """RaZeR: E2M1 whose -0 code is remapped to a per-group special value.

    "The Power of Negative Zero" (abstract, method section): the negative-zero
    encoding is remapped to a special value from a pre-defined set, chosen per
    group.  Reading: every candidate in RAZER_SPECIALS is tried (see
    :func:`razer_candidate`) and the one with the smallest fp64 SSE is kept;
    on equal SSE the earlier candidate wins.  The 2-bit selector stores its
    index.
    """
    n, k = w16.shape
    wg64 = _grouped(w16, g).astype(np.float64)
    absmax32 = np.abs(_grouped(w16, g).astype(np.float32)).max(axis=-1)
    results = [razer_candidate(wg64, absmax32, v) for v in RAZER_SPECIALS]
    sse = np.stack([r[3] for r in results], axis=-1)  # [n, G, 4]
    sel = sse.argmin(axis=-1)  # first minimum
    codes = np.choose(sel[..., None], [r[0] for r in results])
    scales = np.choose(sel, [r[1] for r in results]).astype(np.float16)
    return Quantized("fp4_razer", n, k, g, codes.reshape(n, k), scales=scales,
                     selectors=sel.astype(np.int64))


def _afpq_candidate(w16: np.ndarray, g: int, pos32: np.ndarray, neg32: np.ndarray):
    """AFPQ codes of the groups of w16 for the one-sided ranges pos, neg
    (binary32 per group).  Returns (codes, stored fp16 scale pairs [.., 2],
    fp64 SSE summed by repeated halving).  s+ = f16(pos / 6), s- = f16(neg / 6);
    w < 0 takes the nearest -M[i] s-, else the nearest +M[i] s+."""
    sp16 = _f16_from_f32(pos32 / np.float32(E2M1_MAX))
    sn16 = _f16_from_f32(neg32 / np.float32(E2M1_MAX))
    wg64 = _grouped(w16, g).astype(np.float64)
    scale = np.where(wg64 < 0, sn16.astype(np.float64)[..., None], sp16.astype(np.float64)[..., None])
    codes = _e2m1_codes(wg64, scale)
    sse = _tree_sum_last_axis((wg64 - _e2m1_values(codes) * scale) ** 2)
    return codes, np.stack([sp16, sn16], axis=-1), sse


def quantize_fp4_afpq(w16: np.ndarray, g: int) -> Quantized:
    """AFPQ: E2M1 with separate fp16 scales for positive and negative values.

    "AFPQ: Asymmetric Floating Point Quantization for LLMs" (abstract).
    Reading: s+ = f16(max(max w, 0) / 6), s- = f16(max(-min w, 0) / 6);
    w > 0 rounds to the nearest +M[i]*s+, w < 0 to the nearest -M[i]*s-
    (sign bit set unless the magnitude index is 0), w = 0 to +0.
    Stored as the pair (s+, s-) per group: 32 bits, the same as an asymmetric
    INT scale plus fp16 zero-point.
    """
    n, k = w16.shape
    wg32 = _grouped(w16, g).astype(np.float32)
    pos32 = np.maximum(wg32.max(axis=-1), np.float32(0))
    neg32 = np.maximum(-wg32.min(axis=-1), np.float32(0))
    codes, scales, _ = _afpq_candidate(w16, g, pos32, neg32)
    return Quantized("fp4_afpq", n, k, g, codes.reshape(n, k), scales=scales)


# ------------------------------------------------------------ 3-bit formats --

def _fp3_codes(w64: np.ndarray, scale64: np.ndarray) -> np.ndarray:
    """Signed FP3 codes (sign<<2 | index) of w against one scale per group:
    the nearest of {+-M3[i] s}, ties to the even index, saturating at 4 s;
    a value that rounds to magnitude 0 takes +0."""
    idx = _nearest_magnitude_index(np.abs(w64), scale64, FP3_MAGNITUDES)
    sign = (w64 < 0) & (idx > 0)
    return (sign.astype(np.int64) << 2) | idx


def _fp3_values(codes: np.ndarray) -> np.ndarray:
    """Unit-scale FP3 value of each code (code 4 -> -0.0, i.e. 0)."""
    mag = FP3_MAGNITUDES[codes & 3]
    return np.where((codes & 4) != 0, -mag, mag)


def razer3_candidate(wg64: np.ndarray, absmax32: np.ndarray, v: float):
    """Quantize groups under one 3-bit RaZeR candidate special value ``v``:
    :func:`razer_candidate` on the FP3 grid.  s_v = f16(absmax / max(4, |v|));
    an element takes code 0b100 (decoding to v*s_v) only when v*s_v is
    strictly nearer than its nearest standard FP3 value.  Returns (codes,
    stored fp16 scale, fp64 dequantized values, fp64 SSE by repeated
    halving)."""
    s16 = _f16_from_f32(absmax32 / np.float32(max(FP3_MAX, abs(v))))
    s = s16.astype(np.float64)[..., None]
    std_codes = _fp3_codes(wg64, s)
    std_vals = _fp3_values(std_codes) * s
    spec_val = v * s
    use_spec = np.abs(wg64 - spec_val) < np.abs(wg64 - std_vals)
    codes = np.where(use_spec, 4, std_codes)
    deq = np.where(use_spec, spec_val, std_vals)
    sse = _tree_sum_last_axis((wg64 - deq) ** 2)
    return codes, s16, deq, sse


def quantize_fp3_razer(w16: np.ndarray, g: int) -> Quantized:
    """3-bit RaZeR: FP3 (E2M0) whose -0 code is remapped to a per-group
    special value from RAZER3_SPECIALS ("The Power of Negative Zero",
    abstract: the remapping for 3- and 4-bit FP).  Every candidate is tried
    (:func:`razer3_candidate`) and the smallest fp64 SSE wins, the earlier
    candidate on equal SSE; the 2-bit selector stores its index."""
    n, k = w16.shape
    wg64 = _grouped(w16, g).astype(np.float64)
    absmax32 = np.abs(_grouped(w16, g).astype(np.float32)).max(axis=-1)
    results = [razer3_candidate(wg64, absmax32, v) for v in RAZER3_SPECIALS]
    sse = np.stack([r[3] for r in results], axis=-1)
    sel = sse.argmin(axis=-1)  # first minimum
    codes = np.choose(sel[..., None], [r[0] for r in results])
    scales = np.choose(sel, [r[1] for r in results]).astype(np.float16)
    return Quantized("fp3_razer", n, k, g, codes.reshape(n, k), scales=scales, selectors=sel.astype(np.int64))


def quantize_fp3_afpq(w16: np.ndarray, g: int) -> Quantized:
    """3-bit AFPQ: FP3 (E2M0) with separate fp16 scales for positive and
    negative values ("AFPQ", abstract: asymmetry matters most for small
    groups and sub-4 bits).  Reading, as for 4 bits with the FP3 grid:
    s+ = f16(max(max w, 0) / 4), s- = f16(max(-min w, 0) / 4); w > 0 rounds
    to the nearest +M3[i] s+, w < 0 to the nearest -M3[i] s- (sign bit set
    unless the index is 0), w = 0 to +0.  The -0 code is unused."""
    n, k = w16.shape
    wg32 = _grouped(w16, g).astype(np.float32)
    sp16 = _f16_from_f32(np.maximum(wg32.max(axis=-1), np.float32(0)) / np.float32(FP3_MAX))
    sn16 = _f16_from_f32(np.maximum(-wg32.min(axis=-1), np.float32(0)) / np.float32(FP3_MAX))
    wg64 = _grouped(w16, g).astype(np.float64)
    scale = np.where(wg64 < 0, sn16.astype(np.float64)[..., None], sp16.astype(np.float64)[..., None])
    codes = _fp3_codes(wg64, scale)
    return Quantized("fp3_afpq", n, k, g, codes.reshape(n, k), scales=np.stack([sp16, sn16], axis=-1))


def quantize_bfp(w16: np.ndarray, fmt: str) -> Quantized:
    """Block floating point: one shared 8-bit exponent per block of 16 along K.

    "Revisiting Block-based Quantisation" (abstract): block formats share a
    scaling factor across packed numbers.  Reading: each element keeps a signed
    mantissa of Mb magnitude bits (Mb = 5 for bfp6, 3 for bfp4), i.e. an
    integer in [-(2^Mb - 1), 2^Mb - 1].  With a = max|w| of the block,
    E = floor(log2 a) (exact from the fp16 value), the stored byte is E + 127,
    the step is 2^(E - Mb + 1), the magnitude is min(rne(|w| / step), 2^Mb - 1)
    and the value is mantissa * step.  An all-zero block stores byte 0 and zero
    mantissas.  Width check: 1 + 5 + 8/16 = 6.5 bits per element gives the
    page's 5x memory density over float32 and 1.2x over 8-bit.

    ``codes`` holds the signed mantissa (an int in the range above).
    """
    mb = BFP_MANT_BITS[fmt]
    n, k = w16.shape
    wb = _grouped(w16, BFP_BLOCK).astype(np.float64)
    a = np.abs(wb).max(axis=-1)
    nz = a > 0
    _, e = np.frexp(np.where(nz, a, 1.0))  # a = f * 2^e, f in [0.5, 1)
    E = (e - 1).astype(np.int64)
    step = np.ldexp(1.0, E - mb + 1)[..., None]
    m = np.minimum(np.rint(np.abs(wb) / step), (1 << mb) - 1).astype(np.int64)
    m = np.where(nz[..., None], m, 0)
    codes = np.where(wb < 0, -m, m)
    exps = np.where(nz, E + BFP_EXP_BIAS, 0).astype(np.uint8)
    return Quantized(fmt, n, k, BFP_BLOCK, codes.reshape(n, k), exps=exps)


def quantize_int8(w16: np.ndarray) -> Quantized:
    """Symmetric INT8 per output channel: s = f16(absmax_row / 127),
    q = clamp(rne(w / s), -127, 127).

    The up-precision format for selected layers in "Is (Selective)
    Round-To-Nearest Quantization All You Need?" (abstract; INT4 to INT8 in the
    method section).  Reading: symmetric, no zero-point, one scale per row.
    """
    n, k = w16.shape
    absmax32 = np.abs(w16.astype(np.float32)).max(axis=-1)
    s16 = _f16_from_f32(absmax32 / np.float32(INT8_QMAX))
    s = s16.astype(np.float64)
    nz = s > 0
    safe = np.where(nz, s, 1.0)
    q = np.clip(_rne_quotient(w16.astype(np.float64), safe[:, None]), -INT8_QMAX, INT8_QMAX)
    q = np.where(nz[:, None], q, 0).astype(np.int64)
    return Quantized("int8", n, k, k, q, scales=s16)


def quantize(fmt: str, w16: np.ndarray, group: int) -> Quantized:
    """Dispatch to the format's quantizer after checking the shape rules."""
    if fmt not in FORMATS:
        raise ValueError(f"unknown format {fmt!r}")
    w16 = np.ascontiguousarray(w16, dtype=np.float16)
    if w16.ndim != 2:
        raise ValueError("weights must be [N, K]")
    n, k = w16.shape
    if not np.all(np.isfinite(w16)):
        raise ValueError("weights must be finite")
    if fmt == "int8":
        if group != k:
            raise ValueError("int8 is per output channel: group must equal K")
        return quantize_int8(w16)
    if fmt in BFP_MANT_BITS:
        if group != BFP_BLOCK:
            raise ValueError("block formats use blocks of 16")
        if k % BFP_BLOCK:
            raise ValueError("K must be a multiple of 16")
        return quantize_bfp(w16, fmt)
    if group <= 0 or k % group or group & (group - 1):
        raise ValueError("group must be a power of two dividing K")
    return {
        "int4_asym": quantize_int4_asym,
        "fp4_e2m1": quantize_fp4_e2m1,
        "fp4_razer": quantize_fp4_razer,
        "fp4_afpq": quantize_fp4_afpq,
        "fp3_razer": quantize_fp3_razer,
        "fp3_afpq": quantize_fp3_afpq,
    }[fmt](w16, group)


# ----------------------------------------------------------------- decode --

def dequantize(q: Quantized) -> np.ndarray:
    """Exact fp64 values of the codes under the stored metadata, [N, K]."""
    n, k, g = q.n, q.k, q.group
    c = q.codes.reshape(n, k // g, g)
    if q.fmt == "int4_asym":
        s = q.scales.astype(np.float64)[..., None]
        out = (c - q.zeros[..., None]).astype(np.float64) * s
    elif q.fmt == "fp4_e2m1":
        out = _e2m1_values(c) * q.scales.astype(np.float64)[..., None]
    elif q.fmt == "fp4_razer":
        s = q.scales.astype(np.float64)[..., None]
        special = np.asarray(RAZER_SPECIALS)[q.selectors][..., None]
        out = np.where(c == 8, special, _e2m1_values(c)) * s
    elif q.fmt == "fp4_afpq":
        sp = q.scales[..., 0].astype(np.float64)[..., None]
        sn = q.scales[..., 1].astype(np.float64)[..., None]
        mag = E2M1_MAGNITUDES[c & 7]
        out = np.where((c & 8) != 0, -mag * sn, mag * sp)
    elif q.fmt == "fp3_razer":
        s = q.scales.astype(np.float64)[..., None]
        special = np.asarray(RAZER3_SPECIALS)[q.selectors][..., None]
        out = np.where(c == 4, special, _fp3_values(c)) * s
    elif q.fmt == "fp3_afpq":
        sp = q.scales[..., 0].astype(np.float64)[..., None]
        sn = q.scales[..., 1].astype(np.float64)[..., None]
        mag = FP3_MAGNITUDES[c & 3]
        out = np.where((c & 4) != 0, -mag * sn, mag * sp)
    elif q.fmt in BFP_MANT_BITS:
        mb = BFP_MANT_BITS[q.fmt]
        E = q.exps.astype(np.int64) - BFP_EXP_BIAS
        out = c.astype(np.float64) * np.ldexp(1.0, E - mb + 1)[..., None]
    elif q.fmt == "int8":
        out = c.astype(np.float64) * q.scales.astype(np.float64)[:, None, None]
    else:
        raise ValueError(q.fmt)
    return out.reshape(n, k)
