"""Pins of the decode-attention oracle (CPU only).

Each check fixes the oracle to something it does not compute itself:

* one key: softmax of a single score is 1, so the output is that value row;
* equal keys (or scale 0): uniform weights, the output is the mean of the
  value rows (closed form);
* two keys: the weight of the first is the logistic function of the score
  difference, 1 / (1 + e^(s2 - s1));
* a large score gap: the output tends to the winning value row, with the
  weight of the others bounded by e^-gap;
* invariance under a permutation of the tokens and under adding a constant to
  every score (a key component along a direction orthogonal to q);
* grouped-query sharing: query head h reads KV head h // (Hq / Hkv);
* random cases against scipy's softmax and a matrix product;
* a length-0 sequence outputs 0; planted mistakes (a dropped scale, the wrong
  KV head, an unnormalized sum) fail the checks above.
"""

from __future__ import annotations

import numpy as np
import pytest
from scipy.special import softmax

import oracle


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def test_single_key_returns_its_value():
    rng = np.random.default_rng(1)
    q = _rand(rng, 1, 2, 8).astype(np.float16)
    k = _rand(rng, 1, 1, 5, 8)
    v = _rand(rng, 1, 1, 5, 8)
    out = oracle.attn_decode_f64(q, k, v, [1], 0.7)
    assert np.array_equal(out[0, 0], v[0, 0, 0]) and np.array_equal(out[0, 1], v[0, 0, 0])


def test_equal_keys_and_zero_scale_give_the_mean():
    rng = np.random.default_rng(2)
    q = _rand(rng, 2, 4, 16).astype(np.float16)
    k = np.repeat(_rand(rng, 2, 2, 1, 16), 7, axis=2)
    v = _rand(rng, 2, 2, 7, 16)
    out = oracle.attn_decode_f64(q, k, v, [7, 5], 0.3)
    for b, n in ((0, 7), (1, 5)):
        for h in range(4):
            assert np.allclose(out[b, h], v[b, h // 2, :n].mean(axis=0), rtol=0, atol=1e-14)
    k2 = _rand(rng, 2, 2, 7, 16)
    out0 = oracle.attn_decode_f64(q, k2, v, [7, 7], 0.0)
    assert np.allclose(out0[1, 3], v[1, 1].mean(axis=0), rtol=0, atol=1e-14)


def test_two_keys_follow_the_logistic_weight():
    q = np.array([[[1.0, 2.0, -1.0, 0.5]]], dtype=np.float16)
    k = np.array([[[[0.5, 0.25, 1.0, 2.0], [-1.0, 0.75, 0.5, -0.5]]]])
    v = np.array([[[[1.0, 0.0, 3.0, -2.0], [0.0, 4.0, -1.0, 1.0]]]])
    scale = 0.5
    s1 = scale * (0.5 * 1 + 0.25 * 2 + 1.0 * -1 + 2.0 * 0.5)    # 0.5
    s2 = scale * (-1.0 * 1 + 0.75 * 2 + 0.5 * -1 + -0.5 * 0.5)  # -0.125
    w1 = 1.0 / (1.0 + np.exp(s2 - s1))
    want = w1 * v[0, 0, 0] + (1 - w1) * v[0, 0, 1]
    got = oracle.attn_decode_f64(q, k, v, [2], scale)[0, 0]
    assert np.allclose(got, want, rtol=0, atol=1e-15)


def test_large_gap_selects_the_winner():
    rng = np.random.default_rng(3)
    D = 8
    q = np.zeros((1, 1, D), dtype=np.float16)
    q[0, 0, 0] = 1
    k = _rand(rng, 1, 1, 6, D) * 0.01
    k[0, 0, 4, 0] = 40.0  # score gap about 40 at scale 1
    v = _rand(rng, 1, 1, 6, D)
    out = oracle.attn_decode_f64(q, k, v, [6], 1.0)[0, 0]
    assert np.max(np.abs(out - v[0, 0, 4])) < 5 * np.exp(-39) * np.abs(v).max()


def test_permutation_and_shift_invariance():
    rng = np.random.default_rng(4)
    D = 16
    q = _rand(rng, 1, 2, D).astype(np.float16)
    k = _rand(rng, 1, 1, 9, D)
    v = _rand(rng, 1, 1, 9, D)
    base = oracle.attn_decode_f64(q, k, v, [9], 0.25)
    perm = rng.permutation(9)
    assert np.allclose(oracle.attn_decode_f64(q, k[:, :, perm], v[:, :, perm], [9], 0.25), base, rtol=0, atol=1e-13)
    # a key component orthogonal to both queries changes no score
    qq = q[0].astype(np.float64)
    u = rng.standard_normal(D)
    u -= np.linalg.lstsq(qq.T, u, rcond=None)[0] @ qq
    assert np.allclose(qq @ u, 0, atol=1e-12)
    shifted = k + 3.0 * u
    assert np.allclose(oracle.attn_decode_f64(q, shifted, v, [9], 0.25), base, rtol=0, atol=1e-12)


def test_grouped_query_heads_read_their_kv_head():
    D, L = 4, 3
    q = np.ones((1, 8, D), dtype=np.float16)
    k = np.zeros((1, 2, L, D))
    v = np.zeros((1, 2, L, D))
    v[0, 0] = 1.0
    v[0, 1] = 2.0
    out = oracle.attn_decode_f64(q, k, v, [L], 1.0)
    assert np.all(out[0, :4] == 1.0) and np.all(out[0, 4:] == 2.0)


def test_against_scipy_softmax():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, L, D = 3, 8, 2, 37, 32
    q = _rand(rng, B, Hq, D).astype(np.float16)
    k = _rand(rng, B, Hkv, L, D)
    v = _rand(rng, B, Hkv, L, D)
    lens = [37, 1, 20]
    scale = D ** -0.5
    out = oracle.attn_decode_f64(q, k, v, lens, scale)
    for b in range(B):
        for h in range(Hq):
            n, kv = lens[b], h // (Hq // Hkv)
            p = softmax(scale * (k[b, kv, :n] @ q[b, h].astype(np.float64)))
            assert np.allclose(out[b, h], p @ v[b, kv, :n], rtol=1e-12, atol=1e-12)


def test_empty_sequence_outputs_zero_and_bad_lengths_raise():
    q = np.ones((2, 1, 4), dtype=np.float16)
    k = np.ones((2, 1, 3, 4))
    out = oracle.attn_decode_f64(q, k, k, [0, 3], 1.0)
    assert np.all(out[0] == 0) and np.all(out[1] == 1)
    with pytest.raises(ValueError):
        oracle.attn_decode_f64(q, k, k, [4, 1], 1.0)


def test_kv_rows_order():
    c = np.arange(2 * 3 * 4 * 5).reshape(2, 3, 4, 5)
    rows = oracle.kv_rows(c)
    assert rows.shape == (24, 5)
    b, kv, t = 1, 2, 3
    assert np.array_equal(rows[(b * 3 + kv) * 4 + t], c[b, kv, t])


# ----------------------------------------------------- planted mistakes --

def _mutants():
    from oracle.attn import attn_decode_f64 as orig  # the unpatched function

    def no_scale(q, k, v, lens, scale):
        return orig(q, k, v, lens, 1.0)

    def wrong_head(q, k, v, lens, scale):
        out = np.zeros(q.shape)
        Hq, Hkv = q.shape[1], k.shape[1]
        for h in range(Hq):
            kv = h % Hkv  # interleaved instead of grouped
            out[:, h] = orig(q[:, h:h + 1], k[:, kv:kv + 1], v[:, kv:kv + 1], lens, scale)[:, 0]
        return out

    def unnormalized(q, k, v, lens, scale):
        out = np.zeros(q.shape)
        for b in range(q.shape[0]):
            for h in range(q.shape[1]):
                kv = h // (q.shape[1] // k.shape[1])
                n = lens[b]
                s = scale * (k[b, kv, :n] @ q[b, h].astype(np.float64))
                out[b, h] = np.exp(s - s.max()) @ v[b, kv, :n]
        return out

    return [no_scale, wrong_head, unnormalized]


@pytest.mark.parametrize("mutant", _mutants(), ids=["no_scale", "wrong_head", "unnormalized"])
def test_planted_mistakes_are_caught(mutant, monkeypatch):
    monkeypatch.setattr(oracle, "attn_decode_f64", mutant)
    failed = 0
    for check in (test_two_keys_follow_the_logistic_weight, test_grouped_query_heads_read_their_kv_head,
                  test_against_scipy_softmax, test_equal_keys_and_zero_scale_give_the_mean):
        try:
            check()
        except AssertionError:
            failed += 1
    assert failed >= 1
