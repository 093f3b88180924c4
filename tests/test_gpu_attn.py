"""GPU parity of decode attention over a quantized KV cache (q_attn_decode)
against the CPU oracle.

The caches are packed on the device with q_pack (one row per cached vector),
and the oracle dequantizes its own quantization of the same fp16 caches --
bit-identical to the device packing, which the packing tests establish and
one case here re-checks.  The output must satisfy, per element,
    |out - ref| <= 1e-3 * max|V_deq| over the sequence + 2^-11 * |ref|
(fp32 scores, exponentials and sums against fp64, then one fp16 rounding).

Cases: grouped-query heads 2, 3 and 4 per KV head (one workgroup head group)
and 8 (two head groups), one query head per KV head; ragged lengths, length 1
and 0, a NULL length array; groups 128, 64 and 32; both forms of the scores
at group 128 (MFMA and v_dot2); RaZeR and plain E2M1; sequence ranges from 64
to 1024 tokens (one and many ranges per sequence); a long sequence;
repeatability.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from dequant_gemv_rtn_amd import binding
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

D = 128


def _cache(rng, B, H, L, scale=0.5):
    c = rng.standard_normal((B, H, L, D)) * scale
    c[rng.random(c.shape) < 0.002] *= 8  # a few outliers per group
    return c.astype(np.float16)


def _ref_deq(fmt, cache16, g):
    B, H, L, _ = cache16.shape
    return oracle.dequantize(oracle.quantize(fmt, oracle.kv_rows(cache16), g)).reshape(B, H, L, D)


def _check(out, ref, v_deq, lens, kv_of, what, floor=1e-7):
    out = out.astype(np.float64)
    for b in range(out.shape[0]):
        for h in range(out.shape[1]):
            n = lens[b]
            vmax = np.abs(v_deq[b, kv_of(h), :n]).max() if n else 0.0
            err = np.abs(out[b, h] - ref[b, h])
            tol = 1e-3 * vmax + 2.0 ** -11 * np.abs(ref[b, h]) + floor
            if not np.all(err <= tol):
                i = int(np.argmax(err - tol))
                raise AssertionError(f"{what}: b={b} h={h} d={i}: {out[b, h, i]} vs {ref[b, h, i]} (tol {tol[i]:.3g})")


def _run(fmt, g, B, Hq, Hkv, L, lens, seed, scale=None, null_lens=False):
    rng = np.random.default_rng(seed)
    dev = U.device()
    k16, v16 = _cache(rng, B, Hkv, L), _cache(rng, B, Hkv, L)
    q16 = (rng.standard_normal((B, Hq, D)) * 0.5).astype(np.float16)
    kq = binding.pack_kv(torch.from_numpy(k16).to(dev), fmt, g)
    vq = binding.pack_kv(torch.from_numpy(v16).to(dev), fmt, g)
    lens_t = None if null_lens else torch.tensor(lens, dtype=torch.int32, device=dev)
    out = binding.attn_decode(kq, vq, torch.from_numpy(q16).to(dev), Hkv, L, lens_t, scale)
    torch.cuda.synchronize()
    k_deq, v_deq = _ref_deq(fmt, k16, g), _ref_deq(fmt, v16, g)
    sc = D ** -0.5 if scale is None else scale
    ref = oracle.attn_decode_f64(q16, k_deq, v_deq, lens, sc)
    gq = Hq // Hkv
    _check(out.cpu().numpy(), ref, v_deq, lens, lambda h: h // gq, f"{fmt} g{g} B={B} Hq={Hq} Hkv={Hkv} L={L}")
    return kq, vq, q16, out, k16


@pytest.mark.parametrize("fmt", ["fp4_razer", "fp4_e2m1"])
@pytest.mark.parametrize("g", [128, 64, 32])
def test_attention_matches_oracle_grouped_heads(fmt, g):
    """4 query heads per KV head, ragged lengths in one batch (including a
    single token), a few 64-token ranges per sequence."""
    _run(fmt, g, B=3, Hq=16, Hkv=4, L=300, lens=[300, 1, 173], seed=11 + g)


def test_attention_eight_heads_per_kv_and_mha():
    _run("fp4_razer", 128, B=2, Hq=16, Hkv=2, L=777, lens=[777, 640], seed=21)   # two head groups
    _run("fp4_razer", 128, B=2, Hq=6, Hkv=6, L=129, lens=[129, 64], seed=22)     # one head per KV head
    _run("fp4_razer", 64, B=1, Hq=6, Hkv=2, L=200, lens=[200], seed=23)          # 3 heads per KV head


@pytest.mark.parametrize("mfma", ["1", "0"])
def test_attention_score_forms_and_two_heads_per_kv(mfma, tune):
    """Both forms of the scores at group 128: on the MFMAs (the default, one
    scale per key row) and v_dot2 (QGEMV_ATTN_MFMA=0, the form groups of 32
    and 64 always take); two query heads per KV head (2 heads per workgroup),
    four, and one."""
    tune.set("QGEMV_ATTN_MFMA", mfma)
    _run("fp4_razer", 128, B=2, Hq=8, Hkv=4, L=300, lens=[300, 77], seed=71)
    _run("fp4_e2m1", 128, B=1, Hq=4, Hkv=1, L=500, lens=[433], seed=72)
    _run("fp4_razer", 128, B=2, Hq=3, Hkv=3, L=130, lens=[1, 130], seed=73)


@pytest.mark.parametrize("mfma", ["1", "0"])
def test_attention_tiny_values_peaked_weights(mfma, tune):
    """A value cache of tiny magnitude (its group scales in fp16's subnormal
    range) under a peaked softmax (large query norm), over 2000 tokens:
    most weights times scales are far below fp16's normal range, which the
    matrix-core form of the value sum must not lose (it shifts them by a
    power of two).  The absolute floor of the bound is 2^-25, half the
    smallest fp16 step."""
    tune.set("QGEMV_ATTN_MFMA", mfma)
    rng = np.random.default_rng(81)
    dev = U.device()
    B, Hq, Hkv, L = 2, 8, 2, 2000
    lens = [2000, 1234]
    k16, v16 = _cache(rng, B, Hkv, L), _cache(rng, B, Hkv, L, scale=2e-6)
    q16 = (rng.standard_normal((B, Hq, D)) * 8).astype(np.float16)
    kq = binding.pack_kv(torch.from_numpy(k16).to(dev))
    vq = binding.pack_kv(torch.from_numpy(v16).to(dev))
    out = binding.attn_decode(kq, vq, torch.from_numpy(q16).to(dev), Hkv, L,
                              torch.tensor(lens, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    k_deq, v_deq = _ref_deq("fp4_razer", k16, 128), _ref_deq("fp4_razer", v16, 128)
    ref = oracle.attn_decode_f64(q16, k_deq, v_deq, lens, D ** -0.5)
    assert np.abs(ref).max() < 2.0 ** -10  # tiny outputs, many of them fp16 subnormals
    _check(out.cpu().numpy(), ref, v_deq, lens, lambda h: h // (Hq // Hkv), f"tiny values mfma={mfma}",
           floor=2.0 ** -25)


def test_attention_maximum_lengths():
    """max_len at the limit the header states (2^20: 1024 ranges of 1024
    tokens, the combine kernel's largest count, nearly all of them empty)
    with a 3000-token sequence; and a 262139-token sequence (256 ranges, the
    last one ragged).  Rows are quantized one by one, so the oracle only needs
    the rows inside each sequence."""
    rng = np.random.default_rng(91)
    dev = U.device()
    for B, Hq, Hkv, L, lens in ((1, 4, 1, 1 << 20, [3000]), (1, 4, 1, 1 << 18, [(1 << 18) - 5])):
        n = max(lens)
        k16 = np.zeros((B, Hkv, L, D), dtype=np.float16)
        v16 = np.zeros((B, Hkv, L, D), dtype=np.float16)
        k16[:, :, :n], v16[:, :, :n] = _cache(rng, B, Hkv, n), _cache(rng, B, Hkv, n)
        q16 = (rng.standard_normal((B, Hq, D)) * 0.5).astype(np.float16)
        kq = binding.pack_kv(torch.from_numpy(k16).to(dev))
        vq = binding.pack_kv(torch.from_numpy(v16).to(dev))
        out = binding.attn_decode(kq, vq, torch.from_numpy(q16).to(dev), Hkv, L,
                                  torch.tensor(lens, dtype=torch.int32, device=dev))
        torch.cuda.synchronize()
        del kq, vq
        k_deq, v_deq = _ref_deq("fp4_razer", k16[:, :, :n], 128), _ref_deq("fp4_razer", v16[:, :, :n], 128)
        ref = oracle.attn_decode_f64(q16, k_deq, v_deq, lens, D ** -0.5)
        _check(out.cpu().numpy(), ref, v_deq, lens, lambda h: h // (Hq // Hkv), f"B={B} max_len={L} lens={lens}")
        del k16, v16, k_deq, v_deq
        torch.cuda.empty_cache()


def test_attention_empty_and_null_lengths():
    kq, vq, q16, out, _ = _run("fp4_razer", 128, B=3, Hq=8, Hkv=2, L=96, lens=[0, 96, 5], seed=31)
    assert torch.all(out[0] == 0)
    _run("fp4_razer", 128, B=2, Hq=8, Hkv=2, L=96, lens=[96, 96], seed=32, null_lens=True)


def test_attention_long_sequence_and_large_ranges():
    """B = 1 with 2 KV heads gives 1024-token ranges; 5000 tokens is a ragged
    last range.  Also a custom scale."""
    _run("fp4_razer", 128, B=1, Hq=8, Hkv=2, L=5000, lens=[5000], seed=41)
    _run("fp4_razer", 128, B=1, Hq=8, Hkv=2, L=5000, lens=[4097], seed=42, scale=0.05)


def test_attention_llama3_8b_shape_sampled():
    """Llama-3-8B decode shape (32 query heads, 8 KV heads, head_dim 128), four
    sequences of up to 2048 tokens; the cache packing is compared bit for bit
    with the oracle's on the first sequence's rows."""
    kq, vq, q16, out, k16 = _run("fp4_razer", 128, B=4, Hq=32, Hkv=8, L=2048, lens=[2048, 1500, 17, 1024], seed=51)
    rows = np.arange(8 * 2048)
    _, ref = U.oracle_buffers("fp4_razer", oracle.kv_rows(k16)[rows], 128)
    ref = {name: (None if v is None else v[: oracle.packed_nbytes("fp4_razer", len(rows), 128, 128)[name]])
           for name, v in ref.items()}
    U.assert_packed_equal(U.gpu_buffers(kq, rows), ref, "K cache rows of sequence 0")


def test_attention_repeatable():
    rng = np.random.default_rng(61)
    dev = U.device()
    B, Hq, Hkv, L = 2, 32, 8, 1000
    k = binding.pack_kv(torch.from_numpy(_cache(rng, B, Hkv, L)).to(dev))
    v = binding.pack_kv(torch.from_numpy(_cache(rng, B, Hkv, L)).to(dev))
    q = torch.from_numpy((rng.standard_normal((B, Hq, D)) * 0.5).astype(np.float16)).to(dev)
    lens = torch.tensor([1000, 999], dtype=torch.int32, device=dev)
    a = binding.attn_decode(k, v, q, Hkv, L, lens)
    b = binding.attn_decode(k, v, q, Hkv, L, lens)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
