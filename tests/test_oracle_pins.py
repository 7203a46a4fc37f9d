"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what pins it: a number a page prints, a value worked out by hand
from a format definition (tests/golden/), a closed form, a library routine that
covers a special case, or brute force on tiny inputs.  The pins are chosen so a
plausible mistake (a dropped term, a swapped digit order, a wrong sign, an
off-by-one window) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.special

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLD, name), encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip() if not line.lstrip().startswith("#") else ""
            if line:
                yield line.split()


# ----------------------------------------------------------------------------------
# Byte accounting against the pages' printed numbers
# ----------------------------------------------------------------------------------

def test_page_numbers_byte_accounting(qref):
    g = {row[0]: float(row[1]) for row in _golden_lines("page_numbers.txt")}
    tol = {row[0]: float(row[2]) for row in _golden_lines("page_numbers.txt")}
    assert abs(math.log2(3) - g["ternary_floor_bits"]) <= tol["ternary_floor_bits"]
    assert abs(27e9 * 1.585 / 8 / 1e9 - g["ternary_27b_floor_gb"]) <= tol["ternary_27b_floor_gb"]
    assert abs(27e9 * 1.58 / 8 / 1e9 - g["ternary_27b_158_gb"]) <= tol["ternary_27b_158_gb"]
    # Scale overhead: a 64-weight block with one fp16 scale (the trellis format's block).
    blk = qref.scale_block(qref.TRELLIS2)
    assert blk == 64
    assert abs(27e9 / blk * 2 / 1e9 - g["scales_block64_gb"]) <= tol["scales_block64_gb"]
    # Ternary packing: 52 bytes per 256 weights is above the log2(3) floor and,
    # with its fp16 scale, within the ~1.7 bits per weight the pages observed.
    bpw = qref.packed_row_bytes(qref.TERN_B3, 256) * 8 / 256
    assert math.log2(3) <= bpw
    assert bpw + 16 / 256 <= g["observed_ternary_bpw_max"]
    # Level counts.
    assert 2 ** 4 == g["levels_4bit"] and 2 ** 2 == g["levels_2bit"] and 2 ** 1 == g["levels_1bit"]
    c, _ = qref.quantize(qref.INT4, synth.gauss([9, 1], (1, 4096)))
    assert len(np.unique(c)) == g["levels_4bit"]
    c, _ = qref.quantize(qref.INT2, synth.gauss([9, 2], (1, 4096)))
    assert len(np.unique(c)) == g["levels_2bit"]
    c, _ = qref.quantize(qref.SIGN1, synth.gauss([9, 3], (1, 4096)))
    assert len(np.unique(c)) == g["levels_1bit"]


def test_layer_byte_totals(qref):
    """Per-layer and per-stack byte totals from the row-stride function."""
    def layer_bytes(fmt_of):
        tot = 0
        for name, N, K in synth.LAYER_SHAPES:
            fmt = fmt_of(name)
            tot += N * qref.row_stride(fmt, K) + N * (K // qref.scale_block(fmt)) * 2
        return tot

    # Closed forms: bits per weight incl. fp16 scales x 340,787,200 weights / 8.
    W = sum(N * K for _, N, K in synth.LAYER_SHAPES)
    assert W == 340_787_200
    assert layer_bytes(lambda n: qref.INT2) == W * (2 + 16 / 32) / 8 == 106_496_000
    assert layer_bytes(lambda n: qref.SIGN1) == W * (1 + 16 / 128) / 8 == 47_923_200
    mixed = layer_bytes(lambda n: qref.INT4 if n in synth.ATTN else qref.TERN_B3)
    attn = sum(N * K for n, N, K in synth.LAYER_SHAPES if n in synth.ATTN)
    assert mixed == attn * (4 + 0.5) / 8 + (W - attn) * (1.625 + 16 / 256) / 8
    assert 64 * layer_bytes(lambda n: qref.SIGN1) == 3_067_084_800
    assert 64 * mixed == 6_252_134_400


# ----------------------------------------------------------------------------------
# fp16 conversion: numpy's float16 cast is the special-case library routine
# ----------------------------------------------------------------------------------

def test_f16_conversion_matches_numpy(qref):
    r = synth.rng(7, 7)
    vals = np.concatenate([
        r.standard_normal(4000) * 10.0 ** r.integers(-9, 5, 4000),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11, 0.1, 0.2, 1.5, -7.5]),
    ])
    for v in vals:
        with np.errstate(over="ignore"):
            want = int(np.array([v], np.float64).astype(np.float16).view(np.uint16)[0])
        assert qref.f64_to_f16_bits(v) == want, v
    for h in [0, 1, 0x3C00, 0x7BFF, 0x8001, 0x03FF, 0x0400, 0xC1C5]:
        assert qref.f16_bits_to_f64(h) == float(np.array([h], np.uint16).view(np.float16)[0])


# ----------------------------------------------------------------------------------
# Activation Q8
# ----------------------------------------------------------------------------------

def test_q8_hand_worked_ties(qref):
    rows = {r[0]: r[1:] for r in _golden_lines("q8_ties.txt")}
    x = np.zeros(32, np.float32)
    x[:8] = [float(v) for v in rows["x"]]
    q, d, s = qref.q8_block(x)
    assert list(q[:8]) == [int(v) for v in rows["q"]] and not q[8:].any()
    assert d == float(rows["d"][0]) and s == int(rows["qsum"][0])
    x = np.zeros(32, np.float32)
    x[:4] = [float(v) for v in rows["x2"]]
    q, d, s = qref.q8_block(x)
    assert list(q[:4]) == [int(v) for v in rows["q2"]] and d == float(rows["d2"][0])


def _tiny_cases():
    cases = {}
    for r in _golden_lines("q8_tiny.txt"):
        cases.setdefault(r[0], {})[r[1]] = r[2:]
    return cases


def test_q8_tiny_blocks_hand_worked(qref):
    """Blocks whose amax is tiny (tests/golden/q8_tiny.txt): a reciprocal 1/d that
    overflows makes a zero block, a subnormal d that does not is quantized
    normally; the boundary pair E/F sits one fp32 step apart.  The golden lines
    are re-derived here in exact rational arithmetic as well."""
    import golden.q8_exact as qe

    for name, c in _tiny_cases().items():
        xb = [int(h, 16) for h in c["x"]]
        x = np.zeros(32, np.uint32)
        x[:len(xb)] = xb
        q, d, s = qref.q8_block(x.view(np.float32))
        want_q = [int(v) for v in c["q"]]
        assert list(q[:len(want_q)]) == want_q and not q[len(want_q):].any(), name
        assert np.float32(d).view(np.uint32) == int(c["d"][0], 16), name
        assert s == int(c["qsum"][0]), name
        eq, ed, es = qe.q8_exact([qe.from_bits(b) for b in xb])
        assert eq == want_q and qe.f32_bits(ed) == int(c["d"][0], 16) and es == s, name


def test_q8_matches_exact_arithmetic(qref):
    """Random blocks with amax from the smallest subnormal up to 1e6 (dense
    around the 2^-128 reciprocal-overflow boundary): the oracle's fp32 Q8 equals
    the same definition carried out in exact rational arithmetic."""
    import golden.q8_exact as qe

    rng = np.random.default_rng(31)
    exps = np.concatenate([np.arange(-149, -100), rng.integers(-100, 20, 40)])
    for e in exps:
        for rep in range(3):
            mant = rng.integers(1, 1 << 24, 32).astype(np.float64)
            v = (mant * 2.0 ** (int(e) - 23) * rng.choice([-1.0, 1.0], 32)).astype(np.float32)
            v[rng.integers(0, 32, 4)] = 0.0
            q, d, s = qref.q8_block(v)
            eq, ed, es = qe.q8_exact([qe.from_bits(int(b)) for b in v.view(np.uint32)])
            assert list(q) == eq and np.float32(d).view(np.uint32) == qe.f32_bits(ed) and s == es, (e, rep)


def test_q8_properties(qref):
    x = synth.gauss([11], (64, 1024)) * synth.uniform([12], (64, 1), 0.01, 100.0)
    x[3, :32] = 0.0  # an all-zero block
    q, d, s = qref.act_quant(x, 32)
    assert (np.abs(q.astype(np.int32)) <= 127).all() and (q != -128).all()
    assert d[3, 0] == 0 and not q[3, :32].any() and s[3, 0] == 0
    xb = x.reshape(64, -1, 32)
    qb = q.reshape(64, -1, 32).astype(np.int64)
    am = np.abs(xb).max(-1)
    # the absmax element maps to +-127; reconstruction error within half a step
    i = np.abs(xb).argmax(-1)
    assert (np.abs(np.take_along_axis(qb, i[..., None], -1)[..., 0])[am > 0] == 127).all()
    err = np.abs(xb - qb * d[..., None])
    # half a step, plus fp32 rounding of x * (1/d) (relative 2^-23 of |x| <= 127 d)
    assert (err <= d[..., None] * (0.5 + 127 * 2.0 ** -22)).all()
    assert (qb.sum(-1) == s).all()


# ----------------------------------------------------------------------------------
# Weight quantizers
# ----------------------------------------------------------------------------------

def test_ternary_quantizer_hand_example(qref):
    # [P3] §5.1: scale = mean|W| + 1e-8, code = clamp(round(W/scale), -1, 1).
    w = np.zeros((1, 256), np.float32)
    w[0, :5] = [3.0, -3.0, 1.0, -1.0, 0.01]
    t, s = qref.quantize(qref.TERN_B3, w)
    # mean|w| = 8.01/256 = 0.03129; 3/0.03129 -> 1 (clamped), 1/0.03129 = 32 -> 1,
    # 0.01/0.03129 = 0.32 -> 0
    assert list(t[0, :5]) == [1, -1, 1, -1, 0] and not t[0, 5:].any()
    assert s[0, 0] == int(np.array([8.01 / 256 + 1e-8]).astype(np.float16).view(np.uint16)[0])
    # equal magnitudes: round(1 - 1e-8*...) = 1
    w = np.full((1, 256), -0.5, np.float32)
    t, _ = qref.quantize(qref.TERN_B3, w)
    assert (t == -1).all()


@pytest.mark.parametrize("fmt,L", [("INT2", 4), ("INT4", 16)])
def test_level_quantizer_is_nearest_level(qref, fmt, L):
    """Brute force: the code's level is a nearest level to w (ties allowed)."""
    f = getattr(qref, fmt)
    w = synth.gauss([13, L], (8, 256), 0.02)
    c, s = qref.quantize(f, w)
    sc = s.view(np.float16).astype(np.float64)
    levels = (np.arange(L) - (L - 1) / 2.0)
    for n in range(8):
        for k in range(256):
            sb = sc[n, k // 32]
            u = w[n, k] / sb
            dist = np.abs(levels - u)
            assert dist[c[n, k]] <= dist.min() + 1e-12
    # the scale is fp16(amax / ((L-1)/2))
    am = np.abs(w.astype(np.float64)).reshape(8, -1, 32).max(-1)
    assert (s == (am / ((L - 1) / 2)).astype(np.float16).view(np.uint16)).all()


def test_level_quantizer_hand_example(qref):
    w = np.zeros((1, 32), np.float32)
    w[0, :5] = [0.3, -0.3, 0.1, 0.0, -0.1]
    c, s = qref.quantize(qref.INT2, w)
    # s = fp16(0.3/1.5 = 0.2) = 0.19995; u = 1.5004 -> 3, -1.5004 -> 0,
    # 0.5001 -> 2, 0 -> 2 (tie toward the upper level), -0.5001 -> 1
    assert s[0, 0] == 0x3266
    assert list(c[0, :5]) == [3, 0, 2, 2, 1]


def test_sign_quantizer(qref):
    w = synth.gauss([14], (4, 512))
    w[0, 0] = 0.0
    b, s = qref.quantize(qref.SIGN1, w)
    assert (b == (w >= 0)).all() and b[0, 0] == 1
    m = np.abs(w.astype(np.float64)).reshape(4, -1, 128).mean(-1)
    assert (s == m.astype(np.float16).view(np.uint16)).all()


def test_sign_quantizer_hand_worked_scales(qref):
    """tests/golden/sign1_scales.txt: the fp16 scale (mean |w|, ties to even) and
    the sign bits of hand-built blocks."""
    for r in _golden_lines("sign1_scales.txt"):
        vals = []
        for run in r[1:-2]:
            n, v = run.split("x")
            vals += [float(v)] * int(n)
        w = np.array([vals], np.float32)
        assert w.shape == (1, 128), r[0]
        b, s = qref.quantize(qref.SIGN1, w)
        assert s[0, 0] == int(r[-2], 16), (r[0], hex(s[0, 0]))
        assert int(b.sum()) == int(r[-1]), r[0]


# ----------------------------------------------------------------------------------
# Packed layouts
# ----------------------------------------------------------------------------------

def test_ternary_bytes_hand_worked(qref):
    for r in _golden_lines("tern_bytes.txt"):
        t = [int(v) for v in r[:5]]
        byte = int(r[6])
        # Put the five trits in word 0, byte 0 (weights 0, 4, 8, 12, 16).
        codes = np.zeros((1, 256), np.int8)
        for i in range(5):
            codes[0, 4 * i] = t[i]
        p = qref.pack(qref.TERN_B3, codes)
        assert p[0, 0] == byte, (t, p[0, 0], byte)
        assert (qref.unpack(qref.TERN_B3, p, 256) == codes).all()


def test_ternary_all_bytes_and_fixed_point_digits(qref):
    """All 243 trit tuples are distinct bytes; digits come back both by integer
    division of b = floor(243 q / 256) (the oracle) and by repeated x3 of the
    fixed-point fraction (an independent formula)."""
    seen = set()
    for b in range(243):
        dig = [(b // 3 ** (4 - i)) % 3 for i in range(5)]
        codes = np.zeros((1, 256), np.int8)
        for i in range(5):
            codes[0, 4 * i + 1] = dig[i] - 1   # word 0, byte 1
        p = qref.pack(qref.TERN_B3, codes)
        q = int(p[0, 1])
        assert q == -(-256 * b // 243)
        seen.add(q)
        r, got = q, []
        for _ in range(5):
            r *= 3
            got.append(r >> 8)
            r &= 0xFF
        assert got == dig
        assert (qref.unpack(qref.TERN_B3, p, 256) == codes).all()
    assert len(seen) == 243 and max(seen) == 255


def test_ternary_position_map(qref):
    """One nonzero weight changes exactly one byte, at word k//20 (tail: 12),
    byte k%4, digit (k%20)//4 (tail: (k-240)//4); the tail's 5th digit is 1."""
    zero = qref.pack(qref.TERN_B3, np.zeros((1, 256), np.int8))
    assert (zero[0, :52] == 128).all()       # b = 121 (all digits 1)
    for k in range(256):
        codes = np.zeros((1, 256), np.int8)
        codes[0, k] = 1
        p = qref.pack(qref.TERN_B3, codes)
        diff = np.nonzero(p[0] != zero[0])[0]
        if k < 240:
            word, digit = k // 20, (k % 20) // 4
        else:
            word, digit = 12, (k - 240) // 4
        assert list(diff) == [4 * word + k % 4], k
        b = 121 + 3 ** (4 - digit)
        assert p[0, diff[0]] == -(-256 * b // 243)


def _plane_bit(k, bits):
    """Bit of weight k of a little-endian 32-bit word: 1- and 2-bit codes
    nibble-lane (weight 8j+n in nibble n at offset j*bits), 4-bit codes
    byte-lane (weight 4j+b in byte b at offset 4j)."""
    if bits == 4:
        return 8 * (k % 4) + 4 * (k // 4)
    return 4 * (k % 8) + (k // 8) * bits


@pytest.mark.parametrize("name,bits", [("INT2", 2), ("SIGN1", 1), ("INT4", 4)])
def test_plane_position_map(qref, name, bits):
    """A single set code lands at the bit the layout names and nowhere else."""
    fmt = getattr(qref, name)
    per_word = 32 // bits
    K = 256
    for k in range(0, K, 7):
        codes = np.zeros((1, K), np.int8)
        codes[0, k] = (1 << bits) - 1 if bits > 1 else 1
        p = qref.pack(fmt, codes)
        word = int.from_bytes(bytes(p[0, 4 * (k // per_word): 4 * (k // per_word) + 4]), "little")
        want = ((1 << bits) - 1) << _plane_bit(k % per_word, bits)
        assert word == want, (name, k)
        # nothing else in the row is set
        rest = p[0].copy()
        rest[4 * (k // per_word): 4 * (k // per_word) + 4] = 0
        assert not rest.any()


def test_plane_masks_select_eight_consecutive_weights(qref):
    """(word >> j*bits) & 0x11111111 (1-bit) / 0x33333333 (2-bit) holds the codes of
    weights 8j .. 8j+7 of the word, weight 8j+n in nibble n."""
    rng = np.random.default_rng(3)
    for name, bits, mask in (("SIGN1", 1, 0x11111111), ("INT2", 2, 0x33333333)):
        fmt = getattr(qref, name)
        per_word = 32 // bits
        codes = rng.integers(0, 1 << bits, (1, 256)).astype(np.int8)
        p = qref.pack(fmt, codes)
        for w in range(256 // per_word):
            word = int.from_bytes(bytes(p[0, 4 * w: 4 * w + 4]), "little")
            for j in range(4 // bits):
                plane = (word >> (j * bits)) & mask
                got = [(plane >> (4 * n)) & 15 for n in range(8)]
                assert got == list(codes[0, w * per_word + 8 * j: w * per_word + 8 * j + 8]), (name, w, j)


def test_act_planes_reconstruct_every_byte(qref):
    """Every int8 value v comes back as 16 * sext4(hi) + lo with lo in [0, 15]."""
    v = np.arange(-128, 128, dtype=np.int16)
    q = np.zeros((1, 256 * 32), np.int8)
    q[0, ::32] = v  # value v at position 0 of block v+128, the rest zero
    pl = qref.act_planes(q)
    assert pl.shape == (1, 256, 8) and pl.dtype == np.uint32
    lo = pl[0, :, 0] & 15
    hi = pl[0, :, 4] & 15
    hi_s = np.where(hi >= 8, hi.astype(np.int64) - 16, hi)
    assert (16 * hi_s + lo == v).all()
    # nothing else set: the other positions are zero
    rest = pl[0].copy()
    rest[:, 0] &= ~np.uint32(15)
    rest[:, 4] &= ~np.uint32(15)
    assert not rest.any()


def test_act_planes_positions(qref):
    """Value i of a 32-block lands in nibble i%8 of word i//8 (lo) and 4 + i//8 (hi)."""
    for i in range(32):
        q = np.zeros((1, 64), np.int8)
        q[0, 32 + i] = -17  # lo 15, hi -2 (nibble 14)
        pl = qref.act_planes(q)
        assert not pl[0, 0].any()
        want = np.zeros(8, np.uint32)
        want[i // 8] = 15 << (4 * (i % 8))
        want[4 + i // 8] = 14 << (4 * (i % 8))
        assert (pl[0, 1] == want).all(), i


@pytest.mark.parametrize("name,bits", [("SIGN1", 1), ("INT2", 2)])
def test_nibble_dots_equal_block_dots(qref, name, bits):
    """Brute force: multiplying code planes and activation planes nibble by nibble
    (lo unsigned, hi signed) gives the integer dot sum(code * q) of every 32-block."""
    rng = np.random.default_rng(11)
    fmt = getattr(qref, name)
    K = 512
    codes = rng.integers(0, 1 << bits, (3, K)).astype(np.int8)
    q = rng.integers(-127, 128, (1, K)).astype(np.int8)
    p = qref.pack(fmt, codes)
    pl = qref.act_planes(q)
    words = p[:, : K * bits // 8].view("<u4").astype(np.int64)
    mask = 0x11111111 if bits == 1 else 0x33333333
    nib = lambda x, n: (x >> (4 * n)) & 15
    for r in range(3):
        for kb in range(K // 32):
            acc = 0
            for g in range(4):
                # group g of the block: word and plane index inside the block's words
                wi, j = divmod(g, 4 // bits)
                word = int(words[r, kb * bits + wi])
                cp = (word >> (j * bits)) & mask
                lo, hi = int(pl[0, kb, g]), int(pl[0, kb, 4 + g])
                for n in range(8):
                    h = nib(hi, n)
                    acc += nib(cp, n) * (16 * (h - 16 if h >= 8 else h) + nib(lo, n))
            want = int((codes[r, kb * 32: kb * 32 + 32].astype(np.int64) * q[0, kb * 32: kb * 32 + 32]).sum())
            assert acc == want, (name, r, kb)


@pytest.mark.parametrize("name", ["TERN_B3", "INT2", "SIGN1", "INT4", "TRELLIS2"])
def test_pack_roundtrip(qref, name):
    fmt = getattr(qref, name)
    lo, n = {"TERN_B3": (-1, 3), "INT2": (0, 4), "SIGN1": (0, 2), "INT4": (0, 16), "TRELLIS2": (0, 4)}[name]
    for K in (256, 512, 1280):
        codes = (synth.symbols([15, K, fmt], (5, K), n) + lo).astype(np.int8)
        p = qref.pack(fmt, codes)
        assert p.shape == (5, qref.row_stride(fmt, K)) and p.shape[1] % 16 == 0
        assert not p[:, qref.packed_row_bytes(fmt, K):].any()
        assert (qref.unpack(fmt, p, K) == codes).all()


# ----------------------------------------------------------------------------------
# Trellis: hash, states, codebook
# ----------------------------------------------------------------------------------

def test_hash_hand_values_and_balance(qref):
    for st, h in _golden_lines("hash_values.txt"):
        assert qref.trellis_hash(int(st, 16)) == int(h)
    hs = np.array([qref.trellis_hash(s) for s in range(1 << 16)])
    assert (np.bincount(hs, minlength=256) == 256).all()
    # bit 15 of the state never reaches the low 8 bits
    assert (hs[:1 << 15] == hs[1 << 15:]).all()


def test_trellis_states_hand_and_window(qref):
    g = {r[0]: r[1:] for r in _golden_lines("trellis_states.txt")}
    seed = int(g["seed"][0], 16)
    sym = [int(v) for v in g["symbols"]]
    codes = np.zeros((1, 64), np.int8)
    codes[0, :4] = sym
    p = qref.pack(qref.TRELLIS2, codes)
    assert p[0, 0] == int(g["byte"][0], 16)
    st = qref.trellis_states(p, np.array([seed], np.uint16), 64)
    assert [int(v) for v in st[0, :4]] == [int(v, 16) for v in g["states"]]
    # Window form: the state after symbol 4g+j is the last 16 bits of seed||bytes.
    K = 1024
    codes = synth.symbols([16], (6, K), 4)
    seeds = synth.u16([17], 6)
    p = qref.pack(qref.TRELLIS2, codes)
    st = qref.trellis_states(p, seeds, K)
    for n in range(6):
        by = [int(seeds[n]) >> 8, int(seeds[n]) & 0xFF] + [int(v) for v in p[n, :K // 4]]
        for i in range(0, K, 13):
            gi, j = divmod(i, 4)
            win = ((by[gi] << 16) | (by[gi + 1] << 8) | by[gi + 2]) >> (6 - 2 * j)
            assert st[n, i] == win & 0xFFFF


def test_codebook_is_nearest_fp16_quantile(qref):
    """Phi at the fp16 midpoints around V16[k] brackets (k+0.5)/256 (forward
    CDF through scipy's ndtr, not the oracle's inverse)."""
    v16 = qref.codebook_v16()
    f = v16.view(np.float16).astype(np.float64)
    for k in range(256):
        p = (k + 0.5) / 256
        h = int(v16[k])
        up = float(np.array([h + (1 if f[k] >= 0 else -1)], np.uint16).view(np.float16)[0]) if h not in (0, 0x8000) else None
        dn = float(np.array([h - (1 if f[k] >= 0 else -1)], np.uint16).view(np.float16)[0])
        lo_mid, hi_mid = sorted([(f[k] + dn) / 2, (f[k] + up) / 2])
        assert scipy.special.ndtr(lo_mid) <= p <= scipy.special.ndtr(hi_mid), k
    assert (v16.view(np.float16)[::-1].astype(np.float64) == -f).all()    # antisymmetric
    assert f.sum() == 0 and (np.diff(f) > 0).all()
    assert abs(qref.norm_ppf(0.975) - 1.959963984540054) < 1e-12


def test_codebook_v8(qref):
    v8, g = qref.codebook_v8()
    f = qref.codebook_v16().view(np.float16).astype(np.float64)
    assert v8[0] == -127 and v8[255] == 127 and (np.diff(v8.astype(int)) >= 0).all()
    assert abs(g - f[255] / 127) < 1e-15
    assert (np.abs(v8 * g - f) <= g / 2 + 1e-12).all()


def test_trellis_decode_values(qref):
    K = 512
    codes = synth.symbols([18], (3, K), 4)
    seeds = synth.u16([19], 3)
    scales = synth.uniform_f16([20], (3, K // 64), 0.01, 0.03)
    p = qref.pack(qref.TRELLIS2, codes)
    w = qref.trellis_decode_f32(p, seeds, scales, K)
    st = qref.trellis_states(p, seeds, K)
    v16 = qref.codebook_v16().view(np.float16).astype(np.float64)
    h = np.array([[qref.trellis_hash(int(s)) for s in row] for row in st])
    want = v16[h] * np.repeat(scales.view(np.float16).astype(np.float64), 64, axis=1)
    assert (w.astype(np.float64) == want).all()       # the fp32 product is exact
    wq, dw = qref.trellis_decode_i8(p, seeds, scales, K, 256)
    q2, d2, _ = qref.act_quant(w, 256)
    assert (wq == q2).all() and (dw == d2).all()


# ----------------------------------------------------------------------------------
# Walsh-Hadamard rotation
# ----------------------------------------------------------------------------------

def test_fwht_matches_sylvester_matrix(qref):
    H = scipy.linalg.hadamard(256).astype(np.float64)      # Sylvester order
    for seed in range(4):
        x = synth.gauss([21, seed], 256)
        got = qref.fwht256(x).astype(np.float64)
        want = H @ x.astype(np.float64) / 16
        assert np.abs(got - want).max() <= 1e-5 * np.abs(x).sum() / 16
        # orthonormal: applying it twice returns the input, norm preserved
        back = qref.fwht256(qref.fwht256(x))
        assert np.abs(back - x).max() < 1e-5
        assert abs(np.linalg.norm(got) - np.linalg.norm(x)) < 1e-4 * np.linalg.norm(x)
    e = np.zeros(256, np.float32)
    e[37] = 1.0
    assert (np.abs(qref.fwht256(e)) == 0.0625).all()
    xi = synth.symbols([22], 256, 100).astype(np.float32)
    assert (qref.fwht256(xi).astype(np.float64) == H @ xi.astype(np.float64) / 16).all()


def test_hadamard_quant_signs(qref):
    K = 512
    x = synth.gauss([23], (3, K))
    zero = np.zeros(K // 32, np.uint32)
    q0, d0, s0 = qref.hadamard_quant(x, zero, 256)
    # no signs: FWHT then Q8 of each block
    for b in range(3):
        for blk in range(2):
            u = qref.fwht256(x[b, blk * 256:(blk + 1) * 256])
            q, d, s = qref.q8_block(u)
            assert (q0[b, blk * 256:(blk + 1) * 256] == q).all() and d0[b, blk] == d
    # flipping every sign negates every output
    ones = np.full(K // 32, 0xFFFFFFFF, np.uint32)
    q1, d1, _ = qref.hadamard_quant(x, ones, 256)
    assert (q1 == -q0).all() and (d1 == d0).all()
    # one sign bit = negating that input
    sb = zero.copy()
    sb[1] = 1 << 5                      # input 37
    xm = x.copy()
    xm[:, 37] *= -1
    qa, da, _ = qref.hadamard_quant(x, sb, 32)
    qb, db, _ = qref.hadamard_quant(xm, zero, 32)
    assert (qa == qb).all() and (da == db).all()
    # outliers: the rotation spreads a x20 spike over its block
    xo = synth.with_outliers(synth.gauss([24], (16, 5120)), [25])
    _, dr, _ = qref.hadamard_quant(xo, synth.sign_bits([26], 5120), 256)
    _, dp, _ = qref.act_quant(xo, 256)
    assert dr.max() < dp.max()


# ----------------------------------------------------------------------------------
# GEMV: identities, brute force and the dense dequantized product
# ----------------------------------------------------------------------------------

def _gemv_case(qref, name, N, K, B, seed):
    fmt = getattr(qref, name)
    x = synth.gauss([30, seed], (B, K))
    q, d, s = qref.act_quant(x, 32)
    if name == "TERN_B3":
        codes = synth.trits([31, seed], (N, K))
        sc = synth.uniform_f16([32, seed], (N, K // 256), 0.01, 0.1)
    elif name == "TRELLIS2":
        codes = synth.symbols([31, seed], (N, K), 4)
        sc = synth.uniform_f16([32, seed], (N, K // 64), 0.01, 0.03)
    else:
        codes, sc = qref.quantize(fmt, synth.gauss([31, seed], (N, K), 0.02))
    seeds = synth.u16([33, seed], N) if name == "TRELLIS2" else None
    p = qref.pack(fmt, codes)
    y, a, I = qref.gemv(fmt, p, sc, seeds, K, q, d, want_I=True)
    return fmt, codes, sc, seeds, p, q, d, s, y, a, I


def test_ternary_identity(qref):
    """W.x = sum(x where +1) - sum(x where -1), per 32-block ([P3] §1.2, [P4] §2.2)."""
    _, t, _, _, _, q, _, _, _, _, I = _gemv_case(qref, "TERN_B3", 37, 1024, 2, 1)
    qq = q.astype(np.int64).reshape(2, 1, -1, 32)
    tt = t.reshape(1, 37, -1, 32)
    want = np.where(tt == 1, qq, 0).sum(-1) - np.where(tt == -1, qq, 0).sum(-1)
    assert (I == want).all()


def test_sign_and_2bit_identities(qref):
    _, b, _, _, _, q, _, s, _, _, I = _gemv_case(qref, "SIGN1", 19, 512, 1, 2)
    S1 = np.where(b.reshape(19, -1, 32) == 1, q.astype(np.int64).reshape(1, -1, 32), 0).sum(-1)
    assert (I[0] == 2 * S1 - s[0][None, :]).all()
    _, c, _, _, _, q, _, s, _, _, I = _gemv_case(qref, "INT2", 19, 512, 1, 3)
    Sc = (c.reshape(19, -1, 32).astype(np.int64) * q.astype(np.int64).reshape(1, -1, 32)).sum(-1)
    assert (I[0] == 2 * Sc - 3 * s[0][None, :]).all()


@pytest.mark.parametrize("name", ["TERN_B3", "INT2", "SIGN1", "INT4", "TRELLIS2"])
def test_gemv_brute_force_and_dense(qref, name):
    N, K, B = 21, 512, 3
    fmt, codes, sc, seeds, p, q, d, s, y, a, I = _gemv_case(qref, name, N, K, B, 4)
    if name == "TRELLIS2":
        # levels from the window form of the state, not the oracle's recurrence
        v8, g = qref.codebook_v8()
        lev = np.empty((N, K), np.int64)
        for n in range(N):
            by = [int(seeds[n]) >> 8, int(seeds[n]) & 0xFF] + [int(v) for v in p[n, :K // 4]]
            for i in range(K):
                gi, j = divmod(i, 4)
                st = (((by[gi] << 16) | (by[gi + 1] << 8) | by[gi + 2]) >> (6 - 2 * j)) & 0xFFFF
                lev[n, i] = v8[qref.trellis_hash(st)]
        factor = np.repeat(sc.view(np.float16).astype(np.float64) * g, 64, axis=1)
    else:
        c = codes.astype(np.int64)
        lev = {"TERN_B3": c, "INT2": 2 * c - 3, "SIGN1": 2 * c - 1, "INT4": 2 * c - 15}[name]
        blk = {"TERN_B3": 256, "INT2": 32, "SIGN1": 128, "INT4": 32}[name]
        half = 0.5 if name in ("INT2", "INT4") else 1.0
        factor = np.repeat(sc.view(np.float16).astype(np.float64) * half, blk, axis=1)
    # brute-force integer block dots
    want_I = (lev.reshape(1, N, -1, 32) * q.astype(np.int64).reshape(B, 1, -1, 32)).sum(-1)
    assert (I == want_I).all()
    # dense dequantized product in fp64 (a different summation order)
    Wd = lev * factor
    Xd = q.astype(np.float64) * np.repeat(d.astype(np.float64), 32, axis=1)
    yd = Xd @ Wd.T
    assert np.abs(y - yd).max() <= 1e-12 * a.max()
    assert (a >= np.abs(y)).all()


def test_gemv_zero_activation(qref):
    *_, y, a, I = _gemv_case(qref, "INT4", 8, 256, 1, 5)
    fmt = qref.INT4
    codes, sc = qref.quantize(fmt, synth.gauss([5], (8, 256), 0.02))
    p = qref.pack(fmt, codes)
    q = np.zeros((1, 256), np.int8)
    d = np.zeros((1, 8), np.float32)
    y, a, I = qref.gemv(fmt, p, sc, None, 256, q, d, want_I=True)
    assert not y.any() and not a.any() and not I.any()


# ----------------------------------------------------------------------------------
# GEMM
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("kblock", [256, 32, 512])
def test_gemm_brute_force(qref, kblock):
    M, N, K = 13, 9, 512
    xq = synth.integers([40], (M, K), -127, 127)
    wq = synth.integers([41], (N, K), -127, 127)
    dx = synth.uniform([42], (M, K // kblock), 0.001, 0.1)
    dw = synth.uniform([43], (N, K // kblock), 0.001, 0.1)
    y, a = qref.gemm_i8(xq.astype(np.int8), dx, wq.astype(np.int8), dw, kblock)
    Ib = np.einsum("mbk,nbk->mnb", xq.astype(np.int64).reshape(M, -1, kblock),
                   wq.astype(np.int64).reshape(N, -1, kblock))
    assert np.abs(Ib).max() < 2 ** 24
    T = dx.astype(np.float64)[:, None, :] * dw.astype(np.float64)[None, :, :] * Ib
    assert np.abs(y - T.sum(-1)).max() <= 1e-12 * a.max()
    assert np.allclose(a, np.abs(T).sum(-1), rtol=1e-14, atol=0)


def test_per_row_scales(qref):
    """One scale per row (the block is the whole row): the rotation + Q8 per token
    and the trellis decode + Q8 per weight row follow the Q8 rule with amax over
    the row (the amax element maps to +-127, reconstruction within half a step
    of the rotated / decoded values, Sigma q), pinned against the rotation and the
    decoded values themselves (each pinned above); the GEMM is the exact integer
    matmul times the outer product of the scales."""
    import scipy.linalg

    B, K = 5, 1280
    x = synth.with_outliers(synth.gauss([50], (B, K)), [51])
    sb = synth.sign_bits([52, K], K)
    q, d, s = qref.hadamard_quant(x, sb, K)
    assert q.shape == (B, K) and d.shape == (B, 1) and s.shape == (B, 1)
    sign = 1.0 - 2.0 * ((sb[np.arange(K) // 32] >> (np.arange(K) % 32)) & 1)
    H = scipy.linalg.hadamard(256).astype(np.float64)
    rot = ((x.astype(np.float64) * sign).reshape(B, -1, 256) @ H.T / 16.0).reshape(B, K)
    am = np.abs(rot).max(1)
    assert np.allclose(d[:, 0], am / 127.0, rtol=1e-6)
    qi = q.astype(np.int64)
    assert (np.abs(qi) <= 127).all() and (np.abs(qi).max(1) == 127).all()
    assert (np.abs(rot - qi * d) <= d * 0.5 + am[:, None] * 1e-5).all()
    assert (qi.sum(1) == s[:, 0]).all()
    # trellis decode with one scale per row, against the exact decoded values
    N = 4
    codes = synth.symbols([53], (N, K), 4)
    sc = synth.uniform_f16([54], (N, K // 64), 0.01, 0.03)
    seeds = synth.u16([55], N)
    p = qref.pack(qref.TRELLIS2, codes)
    w = qref.trellis_decode_f32(p, seeds, sc, K).astype(np.float64)
    wq, dw = qref.trellis_decode_i8(p, seeds, sc, K, K)
    assert dw.shape == (N, 1)
    amw = np.abs(w).max(1)
    assert (dw[:, 0] == (amw.astype(np.float32) / np.float32(127.0))).all()
    wi = wq.astype(np.int64)
    assert (np.abs(wi).max(1) == 127).all()
    assert (np.abs(w - wi * dw) <= dw * 0.5 * (1 + 1e-5)).all()
    # GEMM, kblock = K: y = dx dw (xq . wq), the sum of absolute terms |y|
    M, Nn, Kk = 7, 6, 320
    xq = synth.integers([56], (M, Kk), -127, 127).astype(np.int8)
    wq2 = synth.integers([57], (Nn, Kk), -127, 127).astype(np.int8)
    dx = synth.uniform([58], (M, 1), 0.001, 0.1)
    dw2 = synth.uniform([59], (Nn, 1), 0.001, 0.1)
    y, a = qref.gemm_i8(xq, dx, wq2, dw2, Kk)
    I = xq.astype(np.int64) @ wq2.astype(np.int64).T
    ref = dx.astype(np.float64) * dw2.astype(np.float64).T * I
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()
    assert np.allclose(a, np.abs(ref), rtol=1e-14, atol=0)
