"""fp64 matrix-vector / skinny matrix product on dequantized weights (test
infrastructure).

y[b, n] = sum_k W_deq[n, k] * x[b, k]: the product every page's kernel
computes with dequantization fused in ("The Power of Negative Zero", abstract:
a GEMV with fused dequantization; "Is (Selective) Round-To-Nearest
Quantization All You Need?", abstract: RTN on Marlin kernels).  W_deq and the
fp16 activations are exact in fp64 and each product is exact; the sum is
numpy's fp64 matmul (rounding error ~1e-16 relative).
"""

from __future__ import annotations

import numpy as np


def gemv_f64(w_deq: np.ndarray, x16: np.ndarray) -> np.ndarray:
    """``w_deq`` fp64 [N, K], ``x16`` fp16 [B, K] (or [K]) -> fp64 [B, N]."""
    x = np.atleast_2d(np.asarray(x16, dtype=np.float16)).astype(np.float64)
    if x.shape[1] != w_deq.shape[1]:
        raise ValueError("K mismatch")
    return x @ np.asarray(w_deq, dtype=np.float64).T
