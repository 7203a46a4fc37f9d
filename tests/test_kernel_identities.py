"""CPU checks of the arithmetic identities the HIP kernels rely on where they
compute a defined quantity by a shorter route (not a check of the oracle):
the trellis hash read straight as a byte offset into an fp32 table, and Q8
rounding through the fp32 sum 1.5 * 2^23 + v * (1 / d) without a clamp."""
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
