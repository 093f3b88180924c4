"""fp64 decode attention over a quantized KV cache (test infrastructure).

RaZeR is applied to the KV cache as well as to weights ("The Power of
Negative Zero: Datatype Customization for Quantized Large Language Models",
abstract: the datatype plugs into quantization of both weights and the KV
cache).  The page gives no cache layout; the reading taken here:

* every cached key and value vector -- one token of one KV head, head_dim
  long -- is quantized like one weight row (RTN onto the format, groups along
  head_dim), so the cache of one layer is the matrix [B * Hkv * L, head_dim]
  and ``formats.quantize`` / ``formats.dequantize`` apply unchanged;
* decoding one new token per sequence is then the plain definition of
  attention on the dequantized cache: for query head h of sequence b, which
  reads KV head h // (Hq / Hkv) (grouped-query sharing),
      s_t = scale * <q[b, h], K_deq[b, kv, t]>   for t < len_b,
      p = softmax(s),   o[b, h] = sum_t p_t V_deq[b, kv, t];
* a sequence of length 0 has no keys to attend to: its output is 0.

Every product is exact in fp64 (fp16 query times an exactly representable
dequantized value); the sums, the exponential and the division carry fp64
rounding only.
"""

from __future__ import annotations

import numpy as np


def attn_decode_f64(q16: np.ndarray, k_deq: np.ndarray, v_deq: np.ndarray, seq_lens, scale: float) -> np.ndarray:
    """``q16`` fp16 [B, Hq, D]; ``k_deq``, ``v_deq`` [B, Hkv, L, D] (any float
    dtype, taken as fp64); ``seq_lens`` ints [B] in [0, L]; ``scale`` the
    factor on every score.  Returns fp64 [B, Hq, D]."""
    q = np.asarray(q16, dtype=np.float16).astype(np.float64)
    k = np.asarray(k_deq, dtype=np.float64)
    v = np.asarray(v_deq, dtype=np.float64)
    B, Hq, D = q.shape
    Bk, Hkv, L, Dk = k.shape
    if (Bk, Dk) != (B, D) or v.shape != k.shape or Hq % Hkv:
        raise ValueError("shape mismatch")
    gq = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        if not 0 <= n <= L:
            raise ValueError("sequence length outside [0, L]")
        if n == 0:
            continue
        for h in range(Hq):
            kv = h // gq
            s = float(scale) * (k[b, kv, :n] @ q[b, h])
            e = np.exp(s - s.max())
            out[b, h] = (e @ v[b, kv, :n]) / e.sum()
    return out


def kv_rows(cache: np.ndarray) -> np.ndarray:
    """[B, Hkv, L, D] -> the [B * Hkv * L, D] matrix whose rows are quantized
    one by one (row index ((b * Hkv) + kv) * L + t)."""
    c = np.asarray(cache)
    return c.reshape(-1, c.shape[-1])
