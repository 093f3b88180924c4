"""Byte layout of packed weights (test infrastructure).

The layout is ours (the pages fix none); the HIP packer emits the same bytes,
coded separately.  Everything is row-major along K so that consecutive lanes
read consecutive 16-byte pieces of a row:

* 4-bit fields (int4_asym, fp4_e2m1, fp4_razer, fp4_afpq, bfp4): uint32
  [N][K/8]; element k is field (k mod 8) of word k/8, bits 4j..4j+3 for
  field j (low nibble first).  int4_asym stores q in 0..15; the E2M1 family
  stores sign<<3 | magnitude index; bfp4 stores its signed mantissa as a 4-bit
  two's complement field (-7..7).
* bfp6: the signed mantissa as a 6-bit two's complement field (-31..31).  Its
  low 4 bits go to "codes" exactly like a 4-bit format; its top 2 bits go to
  "codes_hi", uint32 [N][K/16].  Word k/16 of codes_hi holds the 2-bit field of
  element e = k mod 16 at bit 16*((e mod 8) div 4) + 8*(e div 8) + 2*(e mod 4),
  which puts the fields of elements j and j+4 of one codes word exactly 16
  bits apart.
* int8: int8 [N][K] (two's complement).
* 3-bit fields (fp3_razer, fp3_afpq): 32 codes per 3 dwords, uint32
  [N][K/32][3].  Piece p of a row holds elements 32p .. 32p+31; element
  e = 8q + n of the piece (q = 0..3, n = 0..7) has magnitude index bits
  (i1, i0) and sign s (code = s<<2 | i1<<1 | i0):
    - index bits in word q div 2: for even q at bits 4n+1 (i0) and 4n+2 (i1),
      for odd q at bits 4n+3 (i0) and (4n+4) mod 32 (i1);
    - sign in word 2 at bit 4n + 3 - q.
  So word 0 masked with 0x66666666 (and the same word rotated right by 2 for
  odd q) plus the sign word shifted left by q and masked with 0x88888888 is
  the piece's q-th group of eight codes as 4-bit E2M1 codes with mantissa 0
  (sign<<3 | index<<1), the same magnitudes {0, 1, 2, 4}.
* scales: fp16 [N][K/g] (int4_asym, fp4_e2m1, fp4_razer); fp16 [N][K/g][2]
  as (s+, s-) for fp4_afpq; fp16 [N] for int8; none for block formats.
* aux: int4_asym zero-points, 4-bit, uint32 [N][ceil(G/8)] low nibble first
  (G = K/g groups per row, rows padded to whole words); fp4_razer selectors,
  2-bit, uint32 [N][ceil(G/16)] low bits first; block exponents uint8
  [N][K/16].

In device memory each buffer is these bytes followed by zero bytes up to the
next multiple of 16 (:func:`buffer_nbytes`, :func:`device_bytes`), so that
16-byte loads that start inside a buffer never end outside it.
"""

from __future__ import annotations

import numpy as np

from .formats import BFP_BLOCK, Quantized

FOUR_BIT_FORMATS = ("int4_asym", "fp4_e2m1", "fp4_razer", "fp4_afpq")
FP3_FORMATS = ("fp3_razer", "fp3_afpq")


def _fp3_positions(e: int):
    """(word, bit of i0, bit of i1, bit of the sign in word 2) of element e
    (0..31) of a 3-bit piece."""
    q, n = divmod(e, 8)
    word = q // 2
    if q % 2 == 0:
        b0, b1 = 4 * n + 1, 4 * n + 2
    else:
        b0, b1 = 4 * n + 3, (4 * n + 4) % 32
    return word, b0, b1, 4 * n + 3 - q


def _pack_fp3(codes: np.ndarray) -> np.ndarray:
    """3-bit codes [N, K] -> uint32 [N, K/32 * 3] (see the module doc)."""
    n, k = codes.shape
    c = codes.reshape(n, k // 32, 32).astype(np.uint64)
    words = np.zeros((n, k // 32, 3), dtype=np.uint64)
    for e in range(32):
        word, b0, b1, bs = _fp3_positions(e)
        ce = c[:, :, e]
        words[:, :, word] |= (ce & np.uint64(1)) << np.uint64(b0)
        words[:, :, word] |= ((ce >> np.uint64(1)) & np.uint64(1)) << np.uint64(b1)
        words[:, :, 2] |= ((ce >> np.uint64(2)) & np.uint64(1)) << np.uint64(bs)
    return words.reshape(n, -1).astype(np.uint32)


def _unpack_fp3(words: np.ndarray, k: int) -> np.ndarray:
    n = words.shape[0]
    w = words.reshape(n, k // 32, 3).astype(np.uint64)
    out = np.zeros((n, k // 32, 32), dtype=np.int64)
    for e in range(32):
        word, b0, b1, bs = _fp3_positions(e)
        i0 = (w[:, :, word] >> np.uint64(b0)) & np.uint64(1)
        i1 = (w[:, :, word] >> np.uint64(b1)) & np.uint64(1)
        sg = (w[:, :, 2] >> np.uint64(bs)) & np.uint64(1)
        out[:, :, e] = (sg << np.uint64(2) | i1 << np.uint64(1) | i0).astype(np.int64)
    return out.reshape(n, k)


def _bfp6_hi_position(e: np.ndarray) -> np.ndarray:
    """Bit offset in a codes_hi word of the 2-bit field of element e (0..15)."""
    return 16 * ((e % 8) // 4) + 8 * (e // 8) + 2 * (e % 4)


def _pack_bfp6_hi(hi2: np.ndarray) -> np.ndarray:
    n, k = hi2.shape
    v = hi2.reshape(n, k // 16, 16).astype(np.uint64)
    pos = _bfp6_hi_position(np.arange(16)).astype(np.uint64)
    return np.bitwise_or.reduce(v << pos, axis=-1).astype(np.uint32)


def _unpack_bfp6_hi(words: np.ndarray, k: int) -> np.ndarray:
    pos = _bfp6_hi_position(np.arange(16)).astype(np.uint64)
    w = words.astype(np.uint64)[..., None]
    return ((w >> pos) & np.uint64(3)).astype(np.int64).reshape(words.shape[0], k)


def _sign_extend(v: np.ndarray, bits: int) -> np.ndarray:
    return np.where(v >= (1 << (bits - 1)), v - (1 << bits), v)


def _pack_fields(values: np.ndarray, bits: int) -> np.ndarray:
    """Pack non-negative ints of ``bits`` width along the last axis into uint32
    words, field j of a word at bits [j*bits, (j+1)*bits).  The last axis is
    padded with zeros to a whole number of words."""
    per = 32 // bits
    n, m = values.shape
    words = -(-m // per)
    v = np.zeros((n, words * per), dtype=np.uint64)
    v[:, :m] = values.astype(np.uint64)
    assert int(v.max(initial=0)) < (1 << bits)
    v = v.reshape(n, words, per)
    out = np.zeros((n, words), dtype=np.uint64)
    for j in range(per):
        out |= v[:, :, j] << np.uint64(j * bits)
    return out.astype(np.uint32)


def _unpack_fields(words: np.ndarray, bits: int, m: int) -> np.ndarray:
    per = 32 // bits
    w = words.astype(np.uint64)
    n, nw = w.shape
    out = np.empty((n, nw, per), dtype=np.int64)
    mask = np.uint64((1 << bits) - 1)
    for j in range(per):
        out[:, :, j] = ((w >> np.uint64(j * bits)) & mask).astype(np.int64)
    return out.reshape(n, nw * per)[:, :m]


def pack(q: Quantized) -> dict:
    """Physical buffers {"codes", "codes_hi", "scales", "aux"} (absent ones
    are None) as numpy arrays with the dtypes listed in the module doc."""
    out = {"codes": None, "codes_hi": None, "scales": None, "aux": None}
    if q.fmt in FOUR_BIT_FORMATS:
        out["codes"] = _pack_fields(q.codes, 4)
    elif q.fmt in FP3_FORMATS:
        out["codes"] = _pack_fp3(q.codes)
    elif q.fmt == "bfp4":
        out["codes"] = _pack_fields(q.codes & 0xF, 4)
    elif q.fmt == "bfp6":
        field = q.codes & 0x3F
        out["codes"] = _pack_fields(field & 0xF, 4)
        out["codes_hi"] = _pack_bfp6_hi(field >> 4)
    elif q.fmt == "int8":
        out["codes"] = q.codes.astype(np.int8)
    else:
        raise ValueError(q.fmt)
    if q.scales is not None:
        out["scales"] = np.ascontiguousarray(q.scales.astype(np.float16))
    if q.fmt == "int4_asym":
        out["aux"] = _pack_fields(q.zeros, 4)
    elif q.fmt in ("fp4_razer", "fp3_razer"):
        out["aux"] = _pack_fields(q.selectors, 2)
    elif q.fmt in ("bfp6", "bfp4"):
        out["aux"] = np.ascontiguousarray(q.exps.astype(np.uint8))
    return out


def unpack(fmt: str, n: int, k: int, group: int, buf: dict) -> Quantized:
    """Inverse of :func:`pack`."""
    if fmt in FOUR_BIT_FORMATS:
        codes = _unpack_fields(buf["codes"], 4, k)
    elif fmt in FP3_FORMATS:
        codes = _unpack_fp3(buf["codes"], k)
    elif fmt == "bfp4":
        codes = _sign_extend(_unpack_fields(buf["codes"], 4, k), 4)
    elif fmt == "bfp6":
        field = _unpack_fields(buf["codes"], 4, k) | (_unpack_bfp6_hi(buf["codes_hi"], k) << 4)
        codes = _sign_extend(field, 6)
    elif fmt == "int8":
        codes = buf["codes"].astype(np.int64)
    else:
        raise ValueError(fmt)
    q = Quantized(fmt, n, k, group, codes)
    if buf.get("scales") is not None:
        q.scales = buf["scales"].astype(np.float16)
    G = k // group
    if fmt == "int4_asym":
        q.zeros = _unpack_fields(buf["aux"], 4, G)
    elif fmt in ("fp4_razer", "fp3_razer"):
        q.selectors = _unpack_fields(buf["aux"], 2, G)
    elif fmt in ("bfp6", "bfp4"):
        q.exps = buf["aux"].astype(np.uint8)
    return q


PAD = 16


def buffer_nbytes(fmt: str, n: int, k: int, group: int) -> dict:
    """Allocated byte size of each buffer: the packed bytes rounded up to a
    multiple of PAD (0 when the format has no such buffer)."""
    return {name: -(-v // PAD) * PAD for name, v in packed_nbytes(fmt, n, k, group).items()}


def device_bytes(fmt: str, n: int, k: int, group: int, buf: dict) -> dict:
    """The buffers of :func:`pack` as they sit in device memory: flat uint8,
    zero-padded to :func:`buffer_nbytes`."""
    sizes = buffer_nbytes(fmt, n, k, group)
    out = {}
    for name, arr in buf.items():
        if arr is None:
            out[name] = None
            continue
        raw = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        padded = np.zeros(sizes[name], dtype=np.uint8)
        padded[: raw.size] = raw
        out[name] = padded
    return out


def packed_nbytes(fmt: str, n: int, k: int, group: int) -> dict:
    """Byte size of the packed contents of each buffer (0 when the format
    has none), before padding."""
    G = k // group
    sizes = {"codes": 0, "codes_hi": 0, "scales": 0, "aux": 0}
    if fmt == "int8":
        sizes["codes"] = n * k
        sizes["scales"] = 2 * n
        return sizes
    sizes["codes"] = n * (k // 32) * 12 if fmt in FP3_FORMATS else n * (k // 8) * 4
    if fmt == "bfp6":
        sizes["codes_hi"] = n * (k // 16) * 4
    if fmt in ("bfp6", "bfp4"):
        sizes["aux"] = n * (k // BFP_BLOCK)
        return sizes
    sizes["scales"] = n * G * 2 * (2 if fmt in ("fp4_afpq", "fp3_afpq") else 1)
    if fmt == "int4_asym":
        sizes["aux"] = n * (-(-G // 8)) * 4
    elif fmt in ("fp4_razer", "fp3_razer"):
        sizes["aux"] = n * (-(-G // 16)) * 4
    return sizes
