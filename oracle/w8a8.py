"""W8A8 product (test infrastructure): INT8 activations per token times INT8
weights per output channel, integer products, one rescale at the end.

"A Method for Layer Bit-Width Allocation in LLM Quantization via Performance
Maximization Under a Quality-Degradation Constraint" (abstract) measures W8A8
variants and finds that for the FFN and lm_head layers the cost of
quantizing and dequantizing is paid back by integer arithmetic; it names a
manual SmoothQuant implementation.  The page gives no formulas, so the steps
below are the reading taken here, the plainest W8A8 scheme:

* smoothing (optional): per-input-channel factors m[k] > 0 move activation
  outliers into the weights, x' = x / m and W' = W * m.  They come from
  calibration data, which is outside this path; the caller supplies m and
  folds it into the weights before quantizing them;
* activations, per token (row b), symmetric INT8: every step in IEEE
  binary32 with round-to-nearest-even, in this order:
      a[k] = f32(x[k]) / f32(m[k])            (a = f32(x) without m)
      s    = max_k |a[k]| / 127
      q[k] = clamp(rne(a[k] / s), -127, 127)  (q = 0 when s = 0)
  The reading is that the quantizer is a binary32 computation throughout:
  its input is fp16 widened exactly, its scale is a binary32 number, and
  each step is one binary32 operation, so the code is the nearest integer
  to the rounded binary32 quotient, not to the exact one (the two can
  differ: tests/golden/w8a8_examples.json holds a smoothed row where they
  do);
* weights: the library's INT8 format, symmetric per output channel with an
  fp16 scale (``formats.quantize_int8``);
* product: acc[b, n] = sum_k q_x[b, k] * q_w[n, k], exact (|acc| < 2^31 for
  k <= 16384);
* output: y[b, n] = f16((f32(s_x[b]) * f32(s_w[n])) * f32(acc[b, n])), two
  binary32 multiplies, each rounded, then one rounding to fp16; f32(acc)
  itself rounds once |acc| > 2^24.  Reading: the rescale stays in the
  precision the activation scale is defined in.

Every step is exact integer arithmetic or one IEEE operation, so the library
must match this bit for bit.
"""

from __future__ import annotations

import numpy as np

QMAX = 127


def quantize_activations(x16: np.ndarray, smooth=None):
    """x16: fp16 [B, K]; smooth: positive float32 [K] or None.  Returns
    (q int8 [B, K], s float32 [B])."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float32)
    if x.ndim != 2:
        raise ValueError("x must be [B, K]")
    if smooth is not None:
        m = np.asarray(smooth, dtype=np.float32)
        if m.shape != (x.shape[1],) or not np.all(m > 0):
            raise ValueError("smoothing factors must be positive, one per input channel")
        a = x / m[None, :]
    else:
        a = x
    absmax = np.abs(a).max(axis=1)
    s = (absmax / np.float32(QMAX)).astype(np.float32)
    q = np.zeros(a.shape, dtype=np.int8)
    nz = s > 0
    quot = a[nz] / s[nz][:, None]  # binary32 quotient
    q[nz] = np.clip(np.rint(quot), -QMAX, QMAX).astype(np.int8)
    return q, s


def integer_product(qx: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """acc[b, n] = sum_k qx[b, k] * qw[n, k], exact in int64."""
    return np.asarray(qx, dtype=np.int64) @ np.asarray(qw, dtype=np.int64).T


def gemm_w8a8(x16: np.ndarray, qw: np.ndarray, sw16: np.ndarray, smooth=None):
    """y fp16 [B, N] of the W8A8 product; qw int8 [N, K] and sw16 fp16 [N]
    are the INT8 weight codes and scales.  Also returns the integer
    accumulators and the activation codes and scales."""
    qx, sx = quantize_activations(x16, smooth)
    acc = integer_product(qx, qw)
    scale = sx[:, None].astype(np.float32) * np.asarray(sw16, dtype=np.float16).astype(np.float32)[None, :]
    with np.errstate(over="ignore"):  # fp16 overflow rounds to +-inf, as IEEE fixes
        y = (scale * acc.astype(np.float32)).astype(np.float16)
    return y, acc, qx, sx
