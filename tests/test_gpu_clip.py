"""GPU parity of q_pack_clip (the per-group clipping search) against the
oracle's quantize_clipped: packed buffers bit for bit.  Every decision is an
fp32 formula rounded once, an exact comparison, or an fp64 SSE summed in the
same pairwise order on both sides, so the bytes must agree exactly.

Cases: the four grouped 4-bit formats, every group size, 1 (plain RTN), 2 and 10 candidates,
heavy-tailed rows (clipping chosen often), all-zero and constant rows
(awkward_rows), and the product over clipped weights against the oracle's
W_deq at the usual tolerance."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from dequant_gemv_rtn_amd import binding
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _weights(n, k, seed):
    rng = np.random.default_rng(seed)
    w = rng.standard_t(3, size=(n, k)) * 0.02
    return U.awkward_rows(w.astype(np.float16), rng)


@pytest.mark.parametrize("fmt", ["int4_asym", "fp4_e2m1", "fp4_afpq", "fp4_razer"])
@pytest.mark.parametrize("g", [32, 64, 128, 256])
@pytest.mark.parametrize("cands", [1, 2, 10])
def test_pack_clip_bit_exact(fmt, g, cands):
    n, k = 23, 2048 + 4 * g
    w = _weights(n, k, 31 * g + cands)
    qw = binding.pack_clip(torch.from_numpy(w).to(U.device()), fmt, g, cands)
    torch.cuda.synchronize()
    q = oracle.quantize_clipped(fmt, w, g, cands)
    ref = oracle.device_bytes(fmt, n, k, g, oracle.pack(q))
    U.assert_packed_equal(U.gpu_buffers(qw), ref, f"clip {fmt} g{g} c{cands}")
    if cands == 1:  # the plain pack, bit for bit
        plain = binding.pack(torch.from_numpy(w).to(U.device()), fmt, g)
        U.assert_packed_equal(U.gpu_buffers(qw), U.gpu_buffers(plain), f"clip=1 vs pack {fmt} g{g}")


@pytest.mark.parametrize("fmt", ["int4_asym", "fp4_e2m1", "fp4_afpq", "fp4_razer"])
def test_products_over_clipped_weights(fmt):
    n, k, g = 300, 4096, 128
    w = (np.random.default_rng(5).standard_t(3, size=(n, k)) * 0.02).astype(np.float16)  # no fp16-extreme rows
    qw = binding.pack_clip(torch.from_numpy(w).to(U.device()), fmt, g, 10)
    deq = oracle.dequantize(oracle.quantize_clipped(fmt, w, g, 10))
    rng = np.random.default_rng(9)
    for b in (1, 8, 33):
        x = rng.standard_normal((b, k)).astype(np.float16)
        y = binding.gemm_skinny(qw, torch.from_numpy(x).to(U.device())).cpu().numpy()
        U.check_tolerance(y, oracle.gemv_f64(deq, x), deq, x, f"clipped {fmt} b={b}")
