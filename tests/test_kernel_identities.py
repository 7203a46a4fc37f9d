"""CPU checks of the arithmetic identities the HIP kernels rely on where they
compute a defined quantity by a shorter route (not a check of the oracle):
the trellis hash read straight as a byte offset into an fp32 table, Q8
rounding through the fp32 sum 1.5 * 2^23 + v * (1 / d) without a clamp, and
the one-token ternary kernel's telescoped digits and sparse matrix-core
operand layout against the oracle's block dots."""
import numpy as np

MAGIC = np.float32(12582912.0)  # 1.5 * 2^23


def test_trellis_hash_byte_offset():
    """For every 24-bit window w and shift s in {0, 2, 4, 6}, with the state
    st = (w >> s) & 0xFFFF and the page's hash h = ((st * 0x9E37) ^ (st >> 7))
    & 0xFF: ((220 a) ^ (a >> 5)) & 0x3FC == 4 h for a = w >> s (a multiply that
    sees only the low 24 bits of a, bits above the state masked off)."""
    w = np.arange(1 << 24, dtype=np.uint64)
    for s in (0, 2, 4, 6):
        a = w >> np.uint64(s)
        st = a & np.uint64(0xFFFF)
        h = ((st * np.uint64(0x9E37)) ^ (st >> np.uint64(7))) & np.uint64(0xFF)
        off = (((a & np.uint64(0xFFFFFF)) * np.uint64(220)) ^ (a >> np.uint64(5))) & np.uint64(0x3FC)
        assert np.array_equal(off, h * np.uint64(4)), s


def _q8_reference(v, am):
    dd = np.float32(am) / np.float32(127.0)
    with np.errstate(divide="ignore", over="ignore"):
        r = np.float32(1.0) / dd
    inv = r if np.isfinite(r) else np.float32(0.0)   # 1/d overflows for d <= 2^-128: a zero block
    t = (v * inv).astype(np.float32)
    return np.clip(np.rint(t), -127, 127).astype(np.int64), t


def test_q8_magic_sum_rounding():
    """The low byte of fp32(1.5 * 2^23 + t), t = fp32(v * (1 / d)), is rint(t)
    (ties to even) in two's complement, and |rint(t)| <= 127 for every |v| <=
    amax, so the clamp never acts: checked on blocks with amax spread over many
    binades down to the smallest subnormal (blocks whose 1/d overflows have
    id = 0 and every t = 0), including v = +-amax, ties and values next to them."""
    rng = np.random.default_rng(7)
    tiny = [1.4e-45, 1e-44, 1e-42, 1e-40, 1e-38, 3.0e-37, 3.73e-37, 3.8e-37, 1e-36, 1e-35, 2.0 ** -118]
    for am in np.concatenate([tiny, [1e-30, 1e-7, 0.37, 1.0, 126.99, 127.0, 3.3e7],
                              rng.uniform(1e-6, 1e6, 200)]).astype(np.float32):
        dd = np.float32(am) / np.float32(127.0)
        with np.errstate(divide="ignore", over="ignore"):
            inv = np.float32(1.0) / dd
        step = inv if np.isfinite(inv) else np.float32(1.0)
        v = np.concatenate([rng.uniform(-am, am, 4000).astype(np.float32), [am, -am, 0.0],
                            ((np.arange(-127, 128) + 0.5) / step).astype(np.float32)]).astype(np.float32)
        v = v[np.abs(v) <= am]
        q, t = _q8_reference(v, am)
        assert np.abs(np.rint(t)).max() <= 127          # no clamp needed
        bits = (t + MAGIC).astype(np.float32).view(np.uint32)
        low = (bits & 0xFF).astype(np.int64)
        assert np.array_equal(np.where(low > 127, low - 256, low), q)
        # the sum of 16 biased words minus 16 x 0x4B400000 (mod 2^32) is the sum of the codes
        k = (len(q) // 16) * 16
        b16 = bits[:k].astype(np.uint64).reshape(-1, 16).sum(1) - np.uint64(16 * 0x4B400000)
        assert np.array_equal((b16 & np.uint64(0xFFFFFFFF)).astype(np.int64).astype(np.int32),
                              q[:k].reshape(-1, 16).sum(1).astype(np.int32))


# ---- one-token ternary GEMV on the sparse matrix cores -------------------------------------------

def test_telescoped_ternary_digits():
    """For every byte x and j = 0..4, the digit the x3 recursion yields equals
    h_{j+1} - 3 h_j with h_j = floor(3^j x / 256); h_1..h_4 are at most 80 (a
    signed byte), and 3^4 x fits a 16-bit lane (no carry into the next lane)."""
    x = np.arange(256, dtype=np.int64)
    r = x.copy()
    h = [np.zeros_like(x)] + [(3 ** j * x) >> 8 for j in range(1, 6)]
    for j in range(5):
        y = 3 * r
        dig = y >> 8
        r = y & 0xFF
        assert np.array_equal(dig, h[j + 1] - 3 * h[j]), j
    assert max(int(h[j].max()) for j in range(1, 5)) <= 80
    assert int((81 * x).max()) < 1 << 16


def _s8(v):
    v = np.asarray(v, np.int64) & 0xFF
    return np.where(v >= 128, v - 256, v)


def _perm0(w, sel):
    """v_perm_b32(0, w, sel): byte k = byte sel_k of w (sel_k < 4), else 0 (0x0C)."""
    out = np.zeros_like(w)
    for k in range(4):
        s = (sel >> (8 * k)) & 0xFF
        if s < 4:
            out |= ((w >> (8 * s)) & 0xFF) << (8 * k)
    return out


def _tern1_block_dots(words, act):
    """The one-token ternary kernel's arithmetic for 16 rows and one 256-weight
    sub-chunk, written out: words [16][13] code words, act [256] int8.
    Returns I [16][8] (block dots of the trits with the activations).

    B operand, lane l = (row l % 16, quarter q = l / 16): words 3q..3q+2 as
    [Y1..Y4 of bytes 0,2 / 1,3 (Yj = 3^j x in 16-bit lanes), the last digit
    ((Y4 & 0x00FF00FF) * 3)] and 3^(q+1) x of word 12.  Compressed A, lane l =
    (A-row 2b + c = l % 16, j = l / 16), dword i = 4 t + cA: the activation
    dword of slot pair kappa = 4 t + 2 (j >> 1) + (cA & 1) of quarter
    qB = 2 (j & 1) + (cA >> 1), bytes 0, 2, 1, 3, kept in block b where the
    coefficient exists.  Sparse 16x16x128 product with B dwords 0-3 at
    k-groups 4 j + d and 4-7 at 16 + 4 j + d, compressed A at k-groups 8 j + g,
    positions 1 and 3 of each group; the accumulator starts at -qsum, and
    I_b = C[2b] - 3 C[2b + 1]."""
    M = 0x00FF00FF
    ab = [int(v) & 0xFF for v in act]
    adw = np.array([ab[4 * g] | (ab[4 * g + 1] << 8) | (ab[4 * g + 2] << 16) | (ab[4 * g + 3] << 24)
                    for g in range(64)], np.int64)
    qs = [int(act[32 * b:32 * b + 32].sum()) for b in range(8)]
    Bl = np.zeros((64, 32), np.int64)
    for l in range(64):
        r, q = l & 15, l >> 4
        out = []
        for mm in range(3):
            w = int(words[r, 3 * q + mm])
            xl, xh = w & M, ((w >> 8) & 0xFF) | (((w >> 24) & 0xFF) << 16)
            for m in (3, 9, 27, 81):
                out += [xl * m, xh * m]
            out += [((xl * 81) & M) * 3, ((xh * 81) & M) * 3]
        w = int(words[r, 12])
        xl, xh = w & M, ((w >> 8) & 0xFF) | (((w >> 24) & 0xFF) << 16)
        out += [xl * 3 ** (q + 1), xh * 3 ** (q + 1)]
        Bl[l] = out
    Al = np.zeros((64, 16), np.int64)
    for l in range(64):
        j, c, b = l >> 4, l & 1, (l & 15) >> 1
        for i in range(16):
            t, cA = i >> 2, i & 3
            qB, kap = 2 * (j & 1) + (cA >> 1), 4 * t + 2 * (j >> 1) + (cA & 1)
            if kap < 15:
                g = 15 * qB + c + kap
                on = (g >> 3) == b and not (c == 1 and kap % 5 >= 3)
            else:
                g = 60 + min(qB + c, 3)
                on = b == 7 and not (c == 1 and qB == 3)
            Al[l, i] = int(_perm0(np.int64(adw[g]), 0x03010200)) if on else 0
    C = np.zeros((16, 16), np.int64)
    for l in range(64):
        C[4 * (l >> 4), l & 15] = -qs[2 * (l >> 4)]
        C[4 * (l >> 4) + 2, l & 15] = -qs[2 * (l >> 4) + 1]
    for t in range(4):
        Bd = np.zeros((128, 16), np.int64)
        Ad = np.zeros((16, 128), np.int64)
        for l in range(64):
            j = l >> 4
            for d in range(8):
                for byte in range(4):
                    kk = 4 * d + byte
                    Bd[16 * j + (kk & 15) + 64 * (kk >> 4), l & 15] = _s8(int(Bl[l, 8 * t + d]) >> (8 * byte))
            for e in range(16):
                v = _s8(int(Al[l, 4 * t + e // 4]) >> (8 * (e % 4)))
                pos = 1 if e % 2 == 0 else 3                     # index 0xD per group of four
                Ad[l & 15, 32 * j + 4 * (e >> 1) + pos] += v
        C += Ad @ Bd
    assert np.abs(C).max() < 1 << 23                             # the 24-bit multiply-adds of the epilogue
    I = np.zeros((16, 8), np.int64)
    for l in range(64):
        jq, r = l >> 4, l & 15
        I[r, 2 * jq] = C[4 * jq, r] - 3 * C[4 * jq + 1, r]
        I[r, 2 * jq + 1] = C[4 * jq + 2, r] - 3 * C[4 * jq + 3, r]
    return I


def test_ternary_one_token_matrix_core_arithmetic():
    """The one-token ternary kernel's block dots, restated from its operand
    layout on the host, equal the oracle's exact block dots: random trits,
    all +1, all -1, and activations at +-127."""
    import oracle

    rng = np.random.default_rng(11)
    for trial in range(6):
        trits = rng.integers(-1, 2, size=(16, 256)).astype(np.int8)
        if trial == 1:
            trits[:] = 1
        if trial == 2:
            trits[:] = -1
        act = rng.integers(-127, 128, size=256).astype(np.int8)
        if trial == 3:
            act[:] = 127
        if trial == 4:
            act[:] = -127
        packed = oracle.pack(oracle.TERN_B3, trits)
        words = np.ascontiguousarray(packed[:, :52]).view("<u4").astype(np.int64).reshape(16, 13)
        scales = np.full((16, 1), 0x3C00, np.uint16)             # fp16 1.0
        _, _, I = oracle.gemv(oracle.TERN_B3, packed, scales, None, 256, act[None, :],
                              np.ones((1, 8), np.float32), want_I=True)
        assert np.array_equal(_tern1_block_dots(words, act), I[0]), trial
