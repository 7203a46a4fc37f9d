"""Pins of the oracle's trellis encoder (Viterbi over the bit-shift trellis).

The trellis codes of the pages' 2-3 bit format are chosen jointly for a row
("12 GB 装下 27B，靠的是什么取舍": QTIP-style trellis coding in groups of 4
weights): the encoder returns the symbol path whose decoded values are closest
to the weights in squared error.  Each pin below checks the oracle against
something other than itself: exhaustive search with exact rational arithmetic,
the fully connected special case (a scalar quantizer), exact recovery of a
sequence the trellis can produce, the decoder, and the Gaussian
rate-distortion bounds.
"""
from __future__ import annotations

import itertools
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.golden.q8_exact import round_f32

HERE = os.path.dirname(os.path.abspath(__file__))


def fmaf_exact(a, b, c) -> Fraction:
    """fp32 fused multiply-add, rounded once, in exact rational arithmetic."""
    return round_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def brute_force(L, val, w, sc):
    """Minimum over every state path of the fp32 cost fold
    c <- fma(d, d, c), d = fma(-sc, val[s], w) (both rounded once), and the
    set of paths attaining it."""
    S, K = 1 << L, len(w)
    best, arg = None, []

    def d_of(i, s):
        return float(fmaf_exact(-np.float32(sc[i]), np.float32(val[s]), np.float32(w[i])))

    def walk(i, s, c, path):
        nonlocal best, arg
        c = fmaf_exact(d_of(i, s), d_of(i, s), c)
        path = path + [s]
        if i == K - 1:
            if best is None or c < best:
                best, arg = c, [path]
            elif c == best:
                arg.append(path)
            return
        for sym in range(4):
            walk(i + 1, ((s << 2) | sym) & (S - 1), c, path)

    for s0 in range(S):
        walk(0, s0, Fraction(0), [])
    return best, arg


@pytest.mark.parametrize("L,K,seed", [(4, 5, 1), (4, 5, 2), (6, 4, 3), (2, 6, 4)])
def test_viterbi_equals_exhaustive_search(L, K, seed):
    rng = np.random.default_rng(seed)
    val = rng.standard_normal(1 << L).astype(np.float32)
    w = rng.standard_normal(K).astype(np.float32)
    sc = rng.uniform(0.5, 1.5, K).astype(np.float32)
    st, cost = oracle.viterbi(L, val, w, sc)
    best, paths = brute_force(L, val, w, sc)
    assert Fraction(float(cost)) == best
    assert [int(s) for s in st] in paths
    # the path is a trellis path: each state shifts the previous one by one symbol
    for i in range(1, K):
        assert (int(st[i]) >> 2) == (int(st[i - 1]) & ((1 << (L - 2)) - 1))


def test_viterbi_fully_connected_is_a_scalar_quantizer():
    """With 2-bit states every state follows every state, so the best path picks
    the nearest value at each step on its own."""
    rng = np.random.default_rng(7)
    val = np.array([-1.5, -0.5, 0.5, 1.5], np.float32)
    w = rng.standard_normal(200).astype(np.float32)
    sc = np.full(200, 0.75, np.float32)
    st, cost = oracle.viterbi(2, val, w, sc)
    err = (w[:, None].astype(np.float64) - sc[:, None].astype(np.float64) * val[None, :]) ** 2
    assert (st == np.argmin(err, axis=1)).all()
    assert abs(float(cost) - err.min(axis=1).sum()) <= 1e-5 * err.min(axis=1).sum()


def test_viterbi_ties_take_the_smallest_choices():
    """All values zero: every path costs the same; the rules (smallest last
    state, smallest predecessor choice) give the all-zero path."""
    st, cost = oracle.viterbi(8, np.zeros(256, np.float32), np.ones(9, np.float32), np.ones(9, np.float32))
    assert (st == 0).all() and float(cost) == 9.0
    # one value stands out at state 5 = 0b101: the last state is 5; its
    # predecessors are 5 >> 2 = 1 plus a << 6, the smallest being 1; those of 1
    # are 0 plus a << 6, the smallest being 0
    val = np.zeros(256, np.float32)
    val[5] = 1.0
    st, cost = oracle.viterbi(8, val, np.array([0, 0, 1], np.float32), np.ones(3, np.float32))
    assert [int(s) for s in st] == [0, 1, 5] and float(cost) == 0.0


def test_viterbi_16_bit_states_exhaustive_short_rows():
    """The 2^16-state trellis against an exhaustive search over all 2^16 x 4^2
    paths of 3 steps, in fp64 (the fp32 recursion can only pick a path whose
    exact cost is within rounding of the optimum)."""
    rng = np.random.default_rng(11)
    v16 = oracle.codebook_v16().astype(np.float16).astype(np.float64)
    h = np.array([oracle.trellis_hash(s) for s in range(65536)])
    val = v16[h]
    for trial in range(3):
        w = rng.standard_normal(3).astype(np.float32)
        sc = np.full(3, np.float32(np.float16(rng.uniform(0.5, 1.5))), np.float32)
        st, cost = oracle.viterbi(16, val.astype(np.float32), w, sc)
        s0 = np.arange(65536)[:, None, None]
        s1 = ((s0 << 2) | np.arange(4)[None, :, None]) & 0xFFFF
        s2 = ((s1 << 2) | np.arange(4)[None, None, :]) & 0xFFFF
        tot = ((w[0] - sc[0] * val[s0]) ** 2 + (w[1] - sc[1] * val[s1]) ** 2 + (w[2] - sc[2] * val[s2]) ** 2)
        got = sum((float(w[i]) - float(sc[i]) * val[int(st[i])]) ** 2 for i in range(3))
        assert got <= tot.min() + 1e-6 * (1 + tot.min())
        assert abs(float(cost) - got) <= 1e-6 * (1 + got)


def test_rms_scale_hand_worked():
    want = {}
    for line in open(os.path.join(HERE, "golden", "trellis_rms_scale.txt")):
        if line.strip() and not line.startswith("#"):
            k, v = line.split()
            want[k] = int(v, 16)
    blocks = {
        "all2": np.full(64, 2.0), "alt34": np.tile([3.0, 4.0], 32), "zero": np.zeros(64),
        "spike8": np.r_[8.0, np.zeros(63)], "all300": np.full(64, 300.0), "allm05": np.full(64, -0.5),
    }
    for k, b in blocks.items():
        assert oracle.trellis_rms_scale(b.astype(np.float32)) == want[k], k


def _codebook_row(rng, K, scales_f16):
    """A row the trellis produces exactly: random seed and symbols, decoded."""
    seed = int(rng.integers(0, 65536))
    codes = rng.integers(0, 4, K).astype(np.int8)
    packed = oracle.pack(oracle.TRELLIS2, codes[None, :])
    w = oracle.trellis_decode_f32(packed, np.array([seed], np.uint16), scales_f16[None, :], K)[0]
    return w


@pytest.mark.parametrize("K", [64, 192])
def test_encoder_recovers_a_trellis_sequence_exactly(K):
    rng = np.random.default_rng(K)
    sc = np.array([np.float16(v) for v in rng.uniform(0.25, 2.0, K // 64)], np.float16).view(np.uint16)
    w = _codebook_row(rng, K, sc)
    packed, seeds, scales, cost = oracle.trellis_encode(w[None, :], scales_in=sc[None, :])
    assert float(cost[0]) == 0.0 and (scales[0] == sc).all()
    back = oracle.trellis_decode_f32(packed, seeds, scales, K)[0]
    assert (back == w).all()


def test_encoder_cost_is_the_reconstruction_error():
    rng = np.random.default_rng(21)
    w = (0.02 * rng.standard_normal((3, 320))).astype(np.float32)
    packed, seeds, scales, cost = oracle.trellis_encode(w)
    back = oracle.trellis_decode_f32(packed, seeds, scales, 320)
    err = ((w.astype(np.float64) - back) ** 2).sum(axis=1)
    assert np.allclose(cost, err, rtol=2e-5, atol=0)
    # and the scales are the RMS rule of each block
    for n in range(3):
        for b in range(5):
            assert scales[n, b] == oracle.trellis_rms_scale(w[n, 64 * b:64 * b + 64])
    # each seed is the first state's top 14 bits
    st = oracle.trellis_states(packed, seeds, 320)
    assert (st[:, 0] >> 2 == seeds).all()


def test_encoder_gaussian_distortion_between_bounds():
    """Unit-variance Gaussian rows at 2 bits per weight: the distortion of any
    code is above the rate-distortion bound 2^-4 = 0.0625, and a trellis code
    beats the best 4-level scalar quantizer (Lloyd-Max, 0.1175)."""
    rng = np.random.default_rng(5)
    w = rng.standard_normal((2, 1024)).astype(np.float32)
    packed, seeds, scales, cost = oracle.trellis_encode(w)
    back = oracle.trellis_decode_f32(packed, seeds, scales, 1024)
    nmse = ((w.astype(np.float64) - back) ** 2).sum() / (w.astype(np.float64) ** 2).sum()
    assert 0.0625 < nmse < 0.1175, nmse


def test_encoder_zero_rows():
    packed, seeds, scales, cost = oracle.trellis_encode(np.zeros((2, 128), np.float32))
    assert (packed == 0).all() and (seeds == 0).all() and (scales == 0).all() and (cost == 0).all()


def _viterbi_rule_reference(L, val, w, sc):
    """The documented recursion and tie rules written out again in Python with
    exact rational fused operations (each rounded once to fp32)."""
    S, top, K = 1 << L, L - 2, len(w)
    f32 = lambda x: round_f32(Fraction(float(np.float32(x))))  # noqa: E731
    C = [None] * S
    IN = [Fraction(0)] * S
    dec = []
    for i in range(K):
        nC, nIN, di = [None] * S, [None] * S, [0] * S
        for s in range(S):
            if i == 0:
                m, best = Fraction(0), 0
            else:
                p = [(s >> 2) | (a << top) for a in range(4)]
                win = []
                for a in range(2):
                    x, y = p[a], p[a + 2]
                    take_y = C[y] < C[x] or (C[y] == C[x] and IN[y] < IN[x])
                    win.append(a + 2 if take_y else a)
                best = win[1] if C[p[win[1]]] < C[p[win[0]]] else win[0]
                m = C[p[best]]
            di[s] = best
            nIN[s] = m
            d = round_f32(f32(w[i]) - f32(sc[i]) * f32(val[s]))
            nC[s] = round_f32(d * d + m)
        C, IN = nC, nIN
        dec.append(di)
    last = min(range(S), key=lambda s: (C[s], s))
    st = [last]
    for i in range(K - 1, 0, -1):
        s = st[-1]
        st.append((s >> 2) | (dec[i][s] << top))
    return st[::-1], C[last]


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_viterbi_tie_rules_against_a_written_out_reference(seed):
    """Cases built to tie: the values ignore the top state bit (as the trellis
    hash ignores bit 15), few distinct values, and a large step that rounds
    different incoming costs to the same cost.  The path must be the one the
    documented rules pick."""
    rng = np.random.default_rng(seed)
    L = 4
    base = rng.integers(-2, 3, 8).astype(np.float32) * np.float32(0.5)
    val = np.concatenate([base, base])          # val[s] = val[s ^ 8]
    w = rng.integers(-3, 4, 5).astype(np.float32) * np.float32(0.25)
    w[2] = np.float32(3000.0)                    # d^2 ~ 1e7: costs that differ a little round together
    sc = np.ones(5, np.float32)
    st, cost = oracle.viterbi(L, val, w, sc)
    want, wcost = _viterbi_rule_reference(L, val, w, sc)
    assert [int(x) for x in st] == want
    assert Fraction(float(cost)) == wcost
