"""Pins of the oracle's KV-cache quantizers and decode attention.

The KV cache is held in 4 or 8 bits per value ("12G 的账本要这么算": KV at Q4
or Q8) and decode attention reads it with the KV heads grouped, six query heads
per KV head ("把非标准格式塞进 llama.cpp，难在哪").  The pins check the oracle
against exact rational arithmetic (the quantizers), the activation Q8 it shares
its rule with, closed forms of attention, an independent numpy/scipy
implementation, invariances, and an fp32 computation in another order against
the oracle's error allowance.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from tests.golden.q8_exact import f32_bits, from_bits, rint_even, round_f32


def q4_exact(v):
    """Q4 of one 32-block in exact arithmetic: (nibble codes, fp32 d)."""
    fv = [from_bits(f32_bits(x)) for x in np.asarray(v, np.float32)]
    amax = max(abs(x) for x in fv)
    d = round_f32(amax / 7)
    if d == 0:
        return [8] * 32, d
    r = round_f32(1 / d)
    codes = []
    for x in fv:
        t = rint_even(round_f32(x * r))
        codes.append(min(7, max(-7, t)) + 8)
    return codes, d


def test_q4_matches_exact_arithmetic():
    rng = np.random.default_rng(3)
    blocks = [rng.standard_normal(32).astype(np.float32) * s for s in (1.0, 1e-3, 37.0)]
    blocks.append((np.arange(32, dtype=np.float32) - 15.5) * 0.25)   # ties at the half levels
    for b in blocks:
        codes, scales = oracle.kv_quant(oracle.KV_Q4, b[None, :])
        want, d = q4_exact(b)
        got = [(int(codes[0, i // 2]) >> (4 * (i % 2))) & 15 for i in range(32)]
        assert got == want
        assert scales[0, 0] == np.float16(float(d)).view(np.uint16) if d != 0 else scales[0, 0] == 0


def test_q4_hand_worked_block():
    """amax = 7 gives d = 1 and id = 1 exactly, so x * id = x: the half-integer
    inputs are ties and go to the even level (0.5 -> 0, 1.5 -> 2, 2.5 -> 2,
    -0.5 -> 0, 6.5 -> 6), 0.25 -> 0, -0.75 -> -1; the scale is fp16 1.0."""
    x = np.zeros(32, np.float32)
    x[:15] = [7, 0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5, -0.5, -1.5, -2.5, -3.5, -4.5, -5.5, -6.5]
    x[30:] = [0.25, -0.75]
    codes, scales = oracle.kv_quant(oracle.KV_Q4, x[None, :])
    got = [((int(codes[0, i // 2]) >> (4 * (i % 2))) & 15) - 8 for i in range(32)]
    want = [7, 0, 2, 2, 4, 4, 6, 6, 0, -2, -2, -4, -4, -6, -6] + [0] * 15 + [0, -1]
    assert got == want
    assert scales[0, 0] == 0x3C00
    # byte layout: value 0 in the low nibble of byte 0, value 1 in its high nibble
    assert codes[0, 0] == (7 + 8) | ((0 + 8) << 4)


def test_q8_cache_is_the_activation_q8_with_fp16_scales():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((5, 256)) * rng.uniform(1e-3, 1e2, (5, 1))).astype(np.float32)
    codes, scales = oracle.kv_quant(oracle.KV_Q8, x)
    q, d, _ = oracle.act_quant(x, 32)
    assert (codes.view(np.int8) == q).all()
    assert (scales == d.astype(np.float16).view(np.uint16)).all()
    back = oracle.kv_dequant(oracle.KV_Q8, codes, scales, 256)
    assert (back == q.astype(np.float64) * np.repeat(d.astype(np.float16).astype(np.float64), 32, axis=1)).all()


def _cache(fmt, rng, n_kv, t_cap, D, scale=1.0):
    K = (rng.standard_normal((n_kv, t_cap, D)) * scale).astype(np.float32)
    V = rng.standard_normal((n_kv, t_cap, D)).astype(np.float32)
    kc, ks = oracle.kv_quant(fmt, K)
    vc, vs = oracle.kv_quant(fmt, V)
    return kc, ks, vc, vs


def _numpy_attention(fmt, q, kc, ks, vc, vs, T, dtype=np.float64):
    n_kv, D = kc.shape[0], q.shape[1]
    G = q.shape[0] // n_kv
    out = np.empty(q.shape, np.float64)
    for h in range(n_kv):
        K = oracle.kv_dequant(fmt, kc[h, :T], ks[h, :T], D).astype(dtype)
        V = oracle.kv_dequant(fmt, vc[h, :T], vs[h, :T], D).astype(dtype)
        for g in range(G):
            s = (K @ q[h * G + g].astype(dtype)) / dtype(np.sqrt(D))
            p = softmax(s.astype(np.float64)).astype(dtype)
            out[h * G + g] = (p @ V).astype(np.float64)
    return out


@pytest.mark.parametrize("fmt", [oracle.KV_Q4, oracle.KV_Q8])
def test_attention_matches_numpy_softmax(fmt):
    rng = np.random.default_rng(fmt)
    n_kv, G, D, T, t_cap = 2, 6, 256, 77, 96
    kc, ks, vc, vs = _cache(fmt, rng, n_kv, t_cap, D)
    q = rng.standard_normal((n_kv * G, D)).astype(np.float32)
    out, bound = oracle.attn_decode(fmt, q, kc, ks, vc, vs, T)
    want = _numpy_attention(fmt, q, kc, ks, vc, vs, T)
    assert np.abs(out - want).max() <= 1e-12 * (1 + np.abs(want).max())
    # an fp32 computation in another order stays inside the allowance
    got32 = _numpy_attention(fmt, q, kc, ks, vc, vs, T, np.float32)
    assert (np.abs(got32 - out) <= bound).all()


def test_attention_closed_forms():
    rng = np.random.default_rng(9)
    fmt, n_kv, G, D = oracle.KV_Q8, 1, 6, 256
    kc, ks, vc, vs = _cache(fmt, rng, n_kv, 40, D)
    q = rng.standard_normal((G, D)).astype(np.float32)
    V = oracle.kv_dequant(fmt, vc[0], vs[0], D)
    # one cached token: the output is its value row
    out, _ = oracle.attn_decode(fmt, q, kc, ks, vc, vs, 1)
    assert (out == V[0]).all()
    # a zero query weighs every token equally
    out, _ = oracle.attn_decode(fmt, np.zeros_like(q), kc, ks, vc, vs, 40)
    assert np.allclose(out, V.mean(axis=0), rtol=0, atol=1e-13)
    # identical keys: the same
    kc2, ks2 = kc.copy(), ks.copy()
    kc2[0, :] = kc[0, 3]
    ks2[0, :] = ks[0, 3]
    out, _ = oracle.attn_decode(fmt, q, kc2, ks2, vc, vs, 40)
    assert np.allclose(out, V.mean(axis=0), rtol=0, atol=1e-13)


def test_attention_dominant_token_and_permutation():
    rng = np.random.default_rng(10)
    fmt, n_kv, G, D, T = oracle.KV_Q4, 1, 6, 256, 50
    kc, ks, vc, vs = _cache(fmt, rng, n_kv, T, D, scale=0.05)
    q = rng.standard_normal((G, D)).astype(np.float32)
    # token 17's key aligned with query row 2, scaled up: its weight is ~1 for that row
    K = rng.standard_normal((1, T, D)).astype(np.float32) * 0.05
    K[0, 17] = q[2] * 4.0
    kc, ks = oracle.kv_quant(fmt, K)
    out, _ = oracle.attn_decode(fmt, q, kc, ks, vc, vs, T)
    V = oracle.kv_dequant(fmt, vc[0], vs[0], D)
    assert np.abs(out[2] - V[17]).max() < 1e-6
    # permuting the cached tokens (keys with their values) changes nothing
    perm = rng.permutation(T)
    out2, _ = oracle.attn_decode(fmt, q, kc[:, perm], ks[:, perm], vc[:, perm], vs[:, perm], T)
    assert np.abs(out2 - out).max() <= 1e-12
    # the query rows of a group are independent of one another
    q2 = q.copy()
    q2[4] = -q2[4]
    out3, _ = oracle.attn_decode(fmt, q2, kc, ks, vc, vs, T)
    assert (out3[[0, 1, 2, 3, 5]] == out[[0, 1, 2, 3, 5]]).all() and np.abs(out3[4] - out[4]).max() > 1e-3
