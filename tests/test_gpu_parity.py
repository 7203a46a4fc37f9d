"""GPU parity of every kernel against the CPU oracle, at sizes the oracle runs
in seconds (several 64-row tiles, ragged row counts, K with and without a tail
segment) and on edge cases.  All calls go through the C ABI."""
import os

import numpy as np
import pytest

import oracle
import synth
from gpu_common import (INT2, INT4, NAMES, SIGN1, TERN, TRELLIS, assert_close_terms, dev, gpu_act, gpu_act_planes,
                        gpu_scales_rowmajor, gpu_weight, host, oracle_weight, raw_weight)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import extreme_bit_quantized_amd as ebq  # noqa: E402

ebq.load()
ALL = [TERN, INT2, SIGN1, INT4, TRELLIS]
SHAPES = [(1, 1024), (70, 1280), (200, 1024), (130, 5120), (64, 2304), (37, 512), (90, 2048)]


def _sync():
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------------------------
# activation quantization and the Hadamard rotation (bit-exact)
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("B,K,qblock", [(1, 32, 32), (3, 1024, 32), (5, 5120, 32), (64, 17408, 32),
                                        (2, 512, 256), (7, 6144, 256)])
def test_act_quant_bit_exact(B, K, qblock):
    x = synth.gauss([100, B, K], (B, K)) * synth.uniform([101, B], (B, 1), 1e-3, 1e3)
    x[0, :qblock] = 0.0                                   # zero block
    if K >= 2 * qblock:
        x[0, qblock:2 * qblock] = np.linspace(-127, 127, qblock, dtype=np.float32) / 2   # half-way ties
    q, d, s = gpu_act(x, qblock)
    _sync()
    rq, rd, rs = oracle.act_quant(x, qblock)
    assert (host(q) == rq).all()
    assert (host(d).view(np.uint32) == rd.view(np.uint32)).all()
    assert (host(s) == rs).all()


@pytest.mark.parametrize("B,K", [(1, 32), (3, 1024), (5, 17408), (64, 5120)])
def test_act_planes_bit_exact(B, K):
    x = synth.gauss([105, B, K], (B, K))
    n = min(K, 64)
    x[0, :n] = np.linspace(-127, 127, n, dtype=np.float32)      # the whole int8 range
    q, pl, d, s = gpu_act_planes(x)
    _sync()
    assert (host(pl).view(np.uint32) == oracle.act_planes(host(q))).all()


def test_act_quant_batch_bit_exact():
    """One batched launch over inputs of every width (q only, planes only, both,
    and an empty one): the oracle's Q8 per 32 and planes, bit for bit."""
    shapes = [(1, 32, "both"), (3, 1024, "planes"), (64, 5120, "both"), (2, 6144, "q"), (0, 512, "both"),
              (5, 17408, "planes"), (7, 96, "q")]
    jobs, ref = [], []
    for i, (B, K, kind) in enumerate(shapes):
        x = synth.gauss([115, i, K], (B, K)) * synth.uniform([116, i], (B, 1), 1e-3, 1e3)
        if B:
            x[0, :32] = 0.0                                            # zero block
            n = min(K - 32, 64)
            if n > 0:
                x[0, 32:32 + n] = np.linspace(-127, 127, n, dtype=np.float32) / 2   # ties
        q = torch.full((B, K), 99, dtype=torch.int8, device="cuda") if kind in ("q", "both") else None
        pl = torch.zeros((B, K // 32, 8), dtype=torch.int32, device="cuda") if kind in ("planes", "both") else None
        d = torch.full((B, K // 32), -1.0, dtype=torch.float32, device="cuda")
        sm = torch.full((B, K // 32), 7, dtype=torch.int32, device="cuda")
        jobs.append((dev(x), q, pl, d, sm))
        ref.append((x, q, pl, d, sm))
    ebq.qact_quant_batch(jobs)
    _sync()
    for x, q, pl, d, sm in ref:
        rq, rd, rs = oracle.act_quant(x, 32)
        assert (host(d).view(np.uint32) == rd.view(np.uint32)).all()
        assert (host(sm) == rs).all()
        if q is not None:
            assert (host(q) == rq).all()
        if pl is not None:
            assert (host(pl).view(np.uint32) == oracle.act_planes(rq)).all()


def _tiny_rows(seed, B, K):
    """Rows whose blocks have amax around the Q8 reciprocal-overflow boundary
    (d <= 2^-128 gives a zero block) and subnormal values: per 32 values a
    random binade from 2^-149 to 2^-100, plus the hand-worked blocks of
    tests/golden/q8_tiny.txt at the start of row 0."""
    rng = np.random.default_rng(synth.seed64(seed, B, K))
    mant = rng.integers(1, 1 << 24, (B, K)).astype(np.float64)
    e = np.repeat(rng.integers(-149, -99, (B, K // 32)), 32, axis=1)
    x = (mant * 2.0 ** (e - 23) * rng.choice([-1.0, 1.0], (B, K))).astype(np.float32)
    x[rng.random((B, K)) < 0.1] = 0.0
    golden = os.path.join(os.path.dirname(__file__), "golden", "q8_tiny.txt")
    blocks = {}
    with open(golden) as f:
        for line in f:
            r = line.split()
            if len(r) > 2 and not line.startswith("#") and r[1] == "x":
                blocks[r[0]] = np.array([int(h, 16) for h in r[2:]], np.uint32).view(np.float32)
    for i, v in enumerate(blocks.values()):
        if 32 * (i + 1) <= K:
            x[0, 32 * i:32 * (i + 1)] = 0.0
            x[0, 32 * i:32 * i + len(v)] = v
    return x


@pytest.mark.parametrize("B,K,qblock", [(3, 1024, 32), (2, 5120, 256)])
def test_act_quant_tiny_blocks_bit_exact(B, K, qblock):
    """Q8 where 1/d overflows (zero blocks), where d is subnormal but 1/d is finite,
    and on subnormal inputs: the per-launch kernel and the batched one."""
    x = _tiny_rows(102, B, K)
    q, d, s = gpu_act(x, qblock)
    _sync()
    rq, rd, rs = oracle.act_quant(x, qblock)
    assert (host(q) == rq).all()
    assert (host(d).view(np.uint32) == rd.view(np.uint32)).all()
    assert (host(s) == rs).all()
    if qblock == 32:
        qb = torch.zeros((B, K), dtype=torch.int8, device="cuda")
        pl = torch.zeros((B, K // 32, 8), dtype=torch.int32, device="cuda")
        db = torch.zeros((B, K // 32), dtype=torch.float32, device="cuda")
        sb = torch.zeros((B, K // 32), dtype=torch.int32, device="cuda")
        ebq.qact_quant_batch([(dev(x), qb, pl, db, sb)])
        _sync()
        assert (host(qb) == rq).all()
        assert (host(db).view(np.uint32) == rd.view(np.uint32)).all()
        assert (host(sb) == rs).all()
        assert (host(pl).view(np.uint32) == oracle.act_planes(rq)).all()


def test_act_quant_empty_batch():
    x = torch.zeros((0, 64), dtype=torch.float32, device="cuda")
    q = torch.zeros((0, 64), dtype=torch.int8, device="cuda")
    d = torch.zeros((0, 2), dtype=torch.float32, device="cuda")
    ebq.qact_quant_i8(x, 32, q, d, d)                     # no-op, no error


@pytest.mark.parametrize("B,K,qblock", [(1, 256, 256), (3, 5120, 256), (4, 17408, 256), (2, 1024, 32)])
def test_hadamard_quant_bit_exact(B, K, qblock):
    x = synth.with_outliers(synth.gauss([110, B, K], (B, K)), [111, B, K])
    sb = synth.sign_bits([112, K], K)
    xt = dev(x)
    q = torch.empty((B, K), dtype=torch.int8, device="cuda")
    d = torch.empty((B, K // qblock), dtype=torch.float32, device="cuda")
    s = torch.empty((B, K // qblock), dtype=torch.int32, device="cuda")
    ebq.qact_hadamard_quant_i8(xt, dev(sb), qblock, q, d, s)
    _sync()
    rq, rd, rs = oracle.hadamard_quant(x, sb, qblock)
    assert (host(q) == rq).all()
    assert (host(d).view(np.uint32) == rd.view(np.uint32)).all()
    assert (host(s) == rs).all()


@pytest.mark.parametrize("qblock", [256, 32])
def test_hadamard_quant_tiny_bit_exact(qblock):
    """Rotation + Q8 on rows scaled into the subnormal range: after the 1/16 the
    rotated values are subnormal (rounded by that multiply) and the blocks' amax
    straddles the 2^-128 reciprocal-overflow boundary of d."""
    K = 1024
    scales = [2.0 ** -e for e in (110, 114, 116, 117, 118, 119, 120, 121, 122, 124, 126, 130, 135, 140, 149)]
    x = synth.with_outliers(synth.gauss([113], (len(scales), K)), [114])
    x = (x.astype(np.float64) * np.array(scales)[:, None]).astype(np.float32)
    sb = synth.sign_bits([115, K], K)
    q = torch.empty((len(scales), K), dtype=torch.int8, device="cuda")
    d = torch.empty((len(scales), K // qblock), dtype=torch.float32, device="cuda")
    s = torch.empty((len(scales), K // qblock), dtype=torch.int32, device="cuda")
    ebq.qact_hadamard_quant_i8(dev(x), dev(sb), qblock, q, d, s)
    _sync()
    rq, rd, rs = oracle.hadamard_quant(x, sb, qblock)
    nz = rq.reshape(len(scales), -1, qblock).any(-1)
    assert ((rd > 0) & ~nz).any()                               # 1/d overflowed: zero blocks with d > 0
    assert ((rd > 0) & (rd < 2.0 ** -126) & nz).any()           # subnormal d, quantized normally
    assert (host(q) == rq).all()
    assert (host(d).view(np.uint32) == rd.view(np.uint32)).all()
    assert (host(s) == rs).all()


# ---------------------------------------------------------------------------------------------
# weight preparation (bit-exact bytes and scales)
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [TERN, INT2, SIGN1, INT4])
@pytest.mark.parametrize("N,K", [(1, 256), (37, 1024), (100, 5120)])
def test_quantize_pack_bit_exact(fmt, N, K):
    raw = raw_weight(fmt, N, K, 120 + fmt)
    raw["w"][0, :32] = 0.0                               # an all-zero block
    pw = gpu_weight(fmt, raw, N, K)
    _sync()
    rp, rs, _ = oracle_weight(fmt, raw)
    assert (host(pw.codes) == rp).all(), NAMES[fmt]
    assert (gpu_scales_rowmajor(pw) == rs).all(), NAMES[fmt]


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("N,K", [(64, 1024), (70, 1280), (1, 256), (130, 4352)])
def test_scale_storage_layout(fmt, N, K):
    """Tiled scale storage: every slot where the header's index formula puts it,
    padding zero, and the row-major round trip exact."""
    if K % oracle.scale_block(fmt):
        pytest.skip("K not a multiple of the scale block")
    nsb = K // oracle.scale_block(fmt)
    G = ebq.qfmt_scale_group(fmt)
    NG = -(-nsb // G)
    rm = synth.uniform_f16([185, fmt, N, K], (N, nsb), 0.01, 0.1)
    pw = ebq.PackedWeight.empty(fmt, N, K)
    pw.scales.fill_(-1)                                      # padding must be rewritten
    ebq.qweight_set_scales(pw, dev(rm))
    _sync()
    tiled = host(pw.scales).view(np.uint16)
    assert tiled.size * 2 == ebq.qfmt_scales_bytes(fmt, N, K) == -(-N // 64) * NG * 64 * G * 2
    want = np.zeros_like(tiled)
    for r in range(N):
        for b in range(nsb):
            want[((r // 64 * NG + b // G) * 64 + r % 64) * G + b % G] = rm[r, b]
    assert (tiled == want).all(), NAMES[fmt]
    assert (gpu_scales_rowmajor(pw) == rm).all(), NAMES[fmt]


@pytest.mark.parametrize("fmt", ALL)
def test_pack_levels_bit_exact(fmt):
    N, K = 45, 1280 if fmt != TERN else 1536
    lo, n = {TERN: (-1, 3), INT2: (0, 4), SIGN1: (0, 2), INT4: (0, 16), TRELLIS: (0, 4)}[fmt]
    codes = (synth.symbols([130, fmt], (N, K), n) + lo).astype(np.int8)
    pw = ebq.PackedWeight.empty(fmt, N, K)
    ebq.qweight_pack(fmt, dev(codes), pw)
    _sync()
    assert (host(pw.codes) == oracle.pack(fmt, codes)).all()


# ---------------------------------------------------------------------------------------------
# GEMV: exact block dots, fp32 outputs within tolerance, batches 1..64
# ---------------------------------------------------------------------------------------------

def _prep(fmt, N, K, seed, B=1):
    raw = raw_weight(fmt, N, K, seed)
    pw = gpu_weight(fmt, raw, N, K)
    rp, rs, rseeds = oracle_weight(fmt, raw)
    x = synth.gauss([seed, 9], (B, K))
    return raw, pw, (rp, rs, rseeds), x


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("N,K", SHAPES)
def test_blockdots_bit_exact(fmt, N, K):
    raw, pw, (rp, rs, rseeds), x = _prep(fmt, N, K, 140 + fmt)
    q, pl, d, s = gpu_act_planes(x)
    out = torch.full((N, K // 32), -7, dtype=torch.int32, device="cuda")
    ebq.qgemv_blockdots(pw, q, pl, s, out)
    _sync()
    rq, rd, _ = oracle.act_quant(x)
    _, _, I = oracle.gemv(fmt, rp, rs, rseeds, K, rq, rd, want_I=True)
    assert (host(out) == I[0]).all(), NAMES[fmt]


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("B", [1, 3, 6])
def test_gemv_parity(fmt, N, K, B):
    raw, pw, (rp, rs, rseeds), x = _prep(fmt, N, K, 150 + fmt + B, B)
    q, pl, d, s = gpu_act_planes(x)
    y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    ebq.qgemv(pw, q, pl, d, s, B, y)
    _sync()
    rq, rd, _ = oracle.act_quant(x)
    yr, absT, _ = oracle.gemv(fmt, rp, rs, rseeds, K, rq, rd)
    assert_close_terms(host(y), yr, absT, what="%s N=%d K=%d B=%d" % (NAMES[fmt], N, K, B))


@pytest.mark.parametrize("B", [2, 4, 5, 6, 7])
def test_gemv_every_batch_size(B):
    fmt, N, K = SIGN1, 96, 2048
    raw, pw, (rp, rs, rseeds), x = _prep(fmt, N, K, 160 + B, B)
    q, pl, d, s = gpu_act_planes(x)
    y = torch.empty((B, N), dtype=torch.float32, device="cuda")
    ebq.qgemv(pw, q, pl, d, s, B, y)
    _sync()
    rq, rd, _ = oracle.act_quant(x)
    yr, absT, _ = oracle.gemv(fmt, rp, rs, rseeds, K, rq, rd)
    assert_close_terms(host(y), yr, absT, what="B=%d" % B)


@pytest.mark.parametrize("fmt,K", [(TERN, 1024), (TERN, 2048), (INT4, 256), (INT4, 512), (SIGN1, 1024),
                                   (SIGN1, 2048), (INT2, 512), (INT2, 1024), (INT2, 2560), (TRELLIS, 512)])
@pytest.mark.parametrize("B", [1, 2])
def test_gemv_one_or_two_segment_rows(fmt, K, B):
    """Rows of one or two whole segments, where the single-matrix launch has the
    waves of a tile split a segment's sub-chunks between them (batch 1 and 2),
    and the 2-bit scalar-operand pipeline at batch 2."""
    N = 130
    raw, pw, (rp, rs, rseeds), x = _prep(fmt, N, K, 165 + fmt + 3 * B, B)
    q, pl, d, s = gpu_act_planes(x)
    y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    ebq.qgemv(pw, q, pl, d, s, B, y)
    _sync()
    rq, rd, _ = oracle.act_quant(x)
    yr, absT, _ = oracle.gemv(fmt, rp, rs, rseeds, K, rq, rd)
    assert_close_terms(host(y), yr, absT, what="%s K=%d B=%d" % (NAMES[fmt], K, B))


PARTIAL = [(INT2, 96), (INT2, 288), (INT4, 96), (INT4, 288), (SIGN1, 384), (TRELLIS, 320), (TERN, 768)]


@pytest.mark.parametrize("fmt,K", PARTIAL)
@pytest.mark.parametrize("B", [1, 2, 3])
def test_gemv_partial_sub_chunk(fmt, K, B):
    """K that ends inside a 256-weight sub-chunk (or a segment): the clamped
    activation loads, the masked blocks past K and the bounded test-hook copy,
    single matrix and grouped, and the block dots at batch 1."""
    N = 70
    raw, pw, (rp, rs, rseeds), x = _prep(fmt, N, K, 175 + fmt + 7 * B, B)
    q, pl, d, s = gpu_act_planes(x)
    rq, rd, _ = oracle.act_quant(x)
    yr, absT, I = oracle.gemv(fmt, rp, rs, rseeds, K, rq, rd, want_I=True)
    y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    ebq.qgemv(pw, q, pl, d, s, B, y)
    yg = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    plan = ebq.GroupedPlan([(pw, q, pl, d, s, yg)], B)
    plan.run()
    _sync()
    assert_close_terms(host(y), yr, absT, what="%s K=%d B=%d" % (NAMES[fmt], K, B))
    assert_close_terms(host(yg), yr, absT, what="grouped %s K=%d B=%d" % (NAMES[fmt], K, B))
    if B == 1:
        o2 = torch.full((N, K // 32), -7, dtype=torch.int32, device="cuda")
        ebq.qgemv_blockdots(pw, q[:1], pl[:1], s[:1], o2)
        _sync()
        assert (host(o2) == I[0]).all(), NAMES[fmt]


def test_gemv_trellis_edge_cases():
    """Trellis rows with all-0 and all-3 symbols, seeds 0 and 0xFFFF, a row with
    zero scales, zero activations and every q = 127."""
    N, K = 66, 1024
    codes = synth.symbols([184], (N, K), 4)
    codes[0] = 0
    codes[1] = 3
    seeds = synth.u16([185], N)
    seeds[0] = 0
    seeds[1] = 0xFFFF
    scales = synth.uniform_f16([186], (N, K // 64), 0.01, 0.03)
    scales[5] = 0
    raw = {"codes": codes, "scales": scales, "seeds": seeds}
    pw = gpu_weight(TRELLIS, raw, N, K)
    rp, rs, rseeds = oracle_weight(TRELLIS, raw)
    x = synth.gauss([187], (3, K))
    x[1] = 0.0
    x[2, :] = 127.0
    q, pl, d, s = gpu_act_planes(x)
    y = torch.empty((3, N), dtype=torch.float32, device="cuda")
    ebq.qgemv(pw, q, pl, d, s, 3, y)
    _sync()
    rq, rd, _ = oracle.act_quant(x)
    yr, absT, _ = oracle.gemv(TRELLIS, rp, rs, rseeds, K, rq, rd)
    assert_close_terms(host(y), yr, absT, what="trellis edge")
    assert not host(y)[1].any() and not host(y)[:, 5].any()


# ---- 9 to 64 tokens: the matrix-core GEMV ------------------------------------------------------

@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("B", [7, 9, 16, 33, 64])
def test_gemv_mfma_parity(fmt, N, K, B):
    """Batches above 6 run on the matrix cores (qgemv, single matrix, four waves
    splitting K): every format and shape at 7, 9, 16, 33 and 64 tokens."""
    raw, pw, (rp, rs, rseeds), x = _prep(fmt, N, K, 700 + fmt + B, B)
    q, pl, d, s = gpu_act_planes(x)
    y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    ebq.qgemv(pw, q, pl, d, s, B, y)
    _sync()
    rq, rd, _ = oracle.act_quant(x)
    yr, absT, _ = oracle.gemv(fmt, rp, rs, rseeds, K, rq, rd)
    assert_close_terms(host(y), yr, absT, what="%s N=%d K=%d B=%d" % (NAMES[fmt], N, K, B))


@pytest.mark.parametrize("B", [7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17, 31, 32, 47, 48, 49, 63, 64])
def test_gemv_mfma_every_token_count(B):
    """Every token count a 16-token group can end on, all five formats in one
    grouped plan (run twice) and as single-matrix launches."""
    specs = [(SIGN1, 200, 2048), (TERN, 130, 1280), (INT4, 70, 1024), (INT2, 90, 2560), (TRELLIS, 65, 1536)]
    entries, refs, singles = [], [], []
    for i, (fmt, N, K) in enumerate(specs):
        raw, pw, (rp, rs, rseeds), x = _prep(fmt, N, K, 720 + 10 * B + i, B)
        q, pl, d, s = gpu_act_planes(x)
        y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
        ys = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
        ebq.qgemv(pw, q, pl, d, s, B, ys)
        singles.append(ys)
        entries.append((pw, q, pl, d, s, y))
        rq, rd, _ = oracle.act_quant(x)
        refs.append(oracle.gemv(fmt, rp, rs, rseeds, K, rq, rd))
    plan = ebq.GroupedPlan(entries, B)
    for rep in range(2):
        for e in entries:
            e[5].fill_(float("nan"))
        plan.run()
        _sync()
        for (fmt, N, K), e, ys, (yr, absT, _) in zip(specs, entries, singles, refs):
            assert_close_terms(host(e[5]), yr, absT, what="grouped %s B=%d rep %d" % (NAMES[fmt], B, rep))
            assert_close_terms(host(ys), yr, absT, what="single %s B=%d" % (NAMES[fmt], B))


@pytest.mark.parametrize("fmt,K", PARTIAL)
def test_gemv_mfma_partial_sub_chunk(fmt, K):
    """K ending inside a 256-weight sub-chunk on the matrix-core path (blocks past
    K are skipped), single and grouped, 20 tokens."""
    B, N = 20, 70
    raw, pw, (rp, rs, rseeds), x = _prep(fmt, N, K, 760 + fmt, B)
    q, pl, d, s = gpu_act_planes(x)
    rq, rd, _ = oracle.act_quant(x)
    yr, absT, _ = oracle.gemv(fmt, rp, rs, rseeds, K, rq, rd)
    y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    ebq.qgemv(pw, q, pl, d, s, B, y)
    yg = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    plan = ebq.GroupedPlan([(pw, q, pl, d, s, yg)], B)
    plan.run()
    _sync()
    assert_close_terms(host(y), yr, absT, what="%s K=%d" % (NAMES[fmt], K))
    assert_close_terms(host(yg), yr, absT, what="grouped %s K=%d" % (NAMES[fmt], K))


@pytest.mark.parametrize("fmt", [TERN, INT2, SIGN1, INT4, TRELLIS])
def test_gemv_mfma_edge_cases(fmt):
    """All-max / all-min codes, a row of zero scales, zero activations for one
    token, every q = 127 for another, at 24 tokens; exact zeros where every term
    is zero."""
    N, K, B = 66, 1024, 24
    if fmt == TRELLIS:
        codes = synth.symbols([770], (N, K), 4)
        codes[0] = 0
        codes[1] = 3
        seeds = synth.u16([771], N)
        seeds[0], seeds[1] = 0, 0xFFFF
        scales = synth.uniform_f16([772], (N, K // 64), 0.01, 0.03)
        raw = {"codes": codes, "scales": scales, "seeds": seeds}
    else:
        lo, hi = {TERN: (-1, 1), INT2: (0, 3), SIGN1: (0, 1), INT4: (0, 15)}[fmt]
        codes = np.zeros((N, K), np.int8)
        codes[0::3] = hi
        codes[1::3] = lo
        codes[2::3] = synth.symbols([773, fmt], (N // 3, K), hi - lo + 1) + lo
        scales = synth.uniform_f16([774, fmt], (N, K // oracle.scale_block(fmt)), 0.01, 0.1)
        raw = {"codes": codes, "scales": scales}
    raw["scales"][5] = 0
    pw = gpu_weight(fmt, raw, N, K)
    rp, rs, rseeds = oracle_weight(fmt, raw)
    x = synth.gauss([775, fmt], (B, K))
    x[1] = 0.0
    x[2, :] = 127.0
    x[23, :] = -127.0
    q, pl, d, s = gpu_act_planes(x)
    y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    ebq.qgemv(pw, q, pl, d, s, B, y)
    _sync()
    rq, rd, _ = oracle.act_quant(x)
    yr, absT, _ = oracle.gemv(fmt, rp, rs, rseeds, K, rq, rd)
    assert_close_terms(host(y), yr, absT, what=NAMES[fmt])
    assert not host(y)[1].any() and not host(y)[:, 5].any()


def test_gemv_mfma_deterministic():
    fmt, N, K, B = TERN, 300, 5120, 40
    raw, pw, _, x = _prep(fmt, N, K, 780, B)
    q, pl, d, s = gpu_act_planes(x)
    y1 = torch.empty((B, N), dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y1)
    ebq.qgemv(pw, q, pl, d, s, B, y1)
    ebq.qgemv(pw, q, pl, d, s, B, y2)
    _sync()
    assert (host(y1).view(np.uint32) == host(y2).view(np.uint32)).all()


def test_gemv_deterministic():
    fmt, N, K = TERN, 300, 5120
    raw, pw, _, x = _prep(fmt, N, K, 170)
    q, pl, d, s = gpu_act_planes(x)
    y1 = torch.empty((1, N), dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y1)
    ebq.qgemv(pw, q, pl, d, s, 1, y1)
    ebq.qgemv(pw, q, pl, d, s, 1, y2)
    _sync()
    assert (host(y1).view(np.uint32) == host(y2).view(np.uint32)).all()


@pytest.mark.parametrize("fmt", [TERN, INT2, SIGN1, INT4])
def test_gemv_edge_cases(fmt):
    """All-max / all-min codes, zero activations, and exact zeros where every
    term is zero."""
    N, K = 66, 1024
    lo, hi = {TERN: (-1, 1), INT2: (0, 3), SIGN1: (0, 1), INT4: (0, 15)}[fmt]
    codes = np.zeros((N, K), np.int8)
    codes[0::3] = hi
    codes[1::3] = lo
    codes[2::3] = synth.symbols([180, fmt], (N // 3, K), hi - lo + 1) + lo
    scales = synth.uniform_f16([181, fmt], (N, K // oracle.scale_block(fmt)), 0.01, 0.1)
    scales[5] = 0                                           # a row with zero scales
    raw = {"codes": codes, "scales": scales}
    pw = gpu_weight(fmt, raw, N, K)
    rp, rs, _ = oracle_weight(fmt, raw)
    x = synth.gauss([182], (3, K))
    x[1] = 0.0                                              # zero activations
    x[2, :] = 127.0                                         # every q = 127
    q, pl, d, s = gpu_act_planes(x)
    y = torch.empty((3, N), dtype=torch.float32, device="cuda")
    ebq.qgemv(pw, q, pl, d, s, 3, y)
    _sync()
    rq, rd, _ = oracle.act_quant(x)
    yr, absT, _ = oracle.gemv(fmt, rp, rs, None, K, rq, rd)
    assert_close_terms(host(y), yr, absT, what=NAMES[fmt])
    assert not host(y)[1].any() and not host(y)[:, 5].any()


def test_sign_balanced_rows_give_exact_zero():
    """1-bit rows with as many +1 as -1 against constant activations: every
    block dot is 0, so y must be exactly 0."""
    N, K = 64, 512
    codes = np.zeros((N, K), np.int8)
    codes[:, 0::2] = 1
    scales = synth.uniform_f16([183], (N, K // 128), 0.5, 1.0)
    pw = gpu_weight(SIGN1, {"codes": codes, "scales": scales}, N, K)
    x = np.full((1, K), 3.0, np.float32)
    q, pl, d, s = gpu_act_planes(x)
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    ebq.qgemv(pw, q, pl, d, s, 1, y)
    _sync()
    assert (host(y) == 0).all()


# ---------------------------------------------------------------------------------------------
# grouped launch
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("B", [1, 8])
def test_grouped_parity_and_reuse(B):
    specs = [(SIGN1, 130, 5120), (TERN, 64, 1024), (INT4, 200, 1280), (INT2, 1, 2048), (TRELLIS, 70, 1280),
             (TERN, 300, 2304), (SIGN1, 65, 17408)]
    entries, refs = [], []
    for i, (fmt, N, K) in enumerate(specs):
        raw, pw, (rp, rs, rseeds), x = _prep(fmt, N, K, 190 + i, B)
        q, pl, d, s = gpu_act_planes(x)
        y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
        entries.append((pw, q, pl, d, s, y))
        rq, rd, _ = oracle.act_quant(x)
        refs.append(oracle.gemv(fmt, rp, rs, rseeds, K, rq, rd))
    plan = ebq.GroupedPlan(entries, B)
    first = None
    for rep in range(3):                                      # a plan runs any number of times
        for e in entries:
            e[5].fill_(float("nan"))
        plan.run()
        _sync()
        outs = [host(e[5]).copy() for e in entries]
        for (fmt, N, K), o, (yr, absT, _) in zip(specs, outs, refs):
            assert_close_terms(o, yr, absT, what="grouped %s rep %d" % (NAMES[fmt], rep))
        if first is None:
            first = outs
        else:                                                 # fixed tile order: bit-identical runs
            for a, b in zip(first, outs):
                assert (a.view(np.uint32) == b.view(np.uint32)).all()


def test_grouped_ternary_one_token_matrix_cores():
    """The one-token ternary grouped launch (telescoped digits on the matrix
    cores): row counts around the 16-row groups and 64-row tiles, K of only a
    tail (256, 768), of whole 1024-weight segments and of segments plus a
    tail; codes all +1, all -1, all 0 and random in one matrix; activations
    with saturated blocks (every q = +-127) and zero blocks; a 4-bit matrix in
    the same plan; three runs, bit-identical."""
    specs = [(1, 256), (15, 768), (16, 1024), (17, 1280), (63, 3072), (64, 5120), (65, 6912), (130, 2560)]
    entries, refs = [], []
    for i, (N, K) in enumerate(specs):
        codes = synth.symbols([610, i], (N, K), 3).astype(np.int8) - 1
        codes[0::7] = 1
        codes[1::7] = -1
        codes[2::7] = 0
        scales = synth.uniform_f16([611, i], (N, K // 256), 0.01, 0.1)
        raw = {"codes": codes, "scales": scales}
        pw = gpu_weight(TERN, raw, N, K)
        rp, rs, _ = oracle_weight(TERN, raw)
        x = synth.gauss([612, i], (1, K))
        x[0, 32:64] = 50.0                                  # a block of q = +127
        x[0, 64:96] = -50.0                                 # a block of q = -127
        x[0, 96:128] = 0.0                                  # a zero block
        x[0, K - 32:] = np.where(np.arange(32) % 2 == 0, 9.0, -9.0)  # alternating saturated block
        q, pl, d, s = gpu_act_planes(x)
        y = torch.full((1, N), float("nan"), dtype=torch.float32, device="cuda")
        entries.append((pw, q, pl, d, s, y))
        rq, rd, _ = oracle.act_quant(x)
        refs.append((TERN, N, K) + oracle.gemv(TERN, rp, rs, None, K, rq, rd)[:2])
    raw, pw, (rp, rs, rseeds), x = _prep(INT4, 70, 2048, 613)
    q, pl, d, s = gpu_act_planes(x)
    y = torch.full((1, 70), float("nan"), dtype=torch.float32, device="cuda")
    entries.append((pw, q, pl, d, s, y))
    rq, rd, _ = oracle.act_quant(x)
    refs.append((INT4, 70, 2048) + oracle.gemv(INT4, rp, rs, rseeds, 2048, rq, rd)[:2])
    plan = ebq.GroupedPlan(entries, 1)
    first = None
    for rep in range(3):
        for e in entries:
            e[5].fill_(float("nan"))
        plan.run()
        _sync()
        outs = [host(e[5]).copy() for e in entries]
        for (fmt, N, K, yr, absT), o in zip(refs, outs):
            assert_close_terms(o, yr, absT, what="grouped %s %dx%d rep %d" % (NAMES[fmt], N, K, rep))
        if first is None:
            first = outs
        else:
            for a, b in zip(first, outs):
                assert (a.view(np.uint32) == b.view(np.uint32)).all()


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("N,K", [(17408, 5120), (5120, 17408)])
@pytest.mark.parametrize("B", [1, 8, 16, 64])
def test_gemv_full_size_sampled(fmt, N, K, B):
    """Every format at the 27B FFN shapes (gate / up 17408 x 5120, down
    5120 x 17408), batch 1, 8, 16 and 64, run as a grouped plan (the launch the stack
    benchmarks time), checked against the oracle on sampled rows: the first
    and last tiles and 62 rows between.  Quantization and packing are per row,
    so the oracle builds only the sampled rows from the same draws."""
    seed = [500, fmt, N, B]
    rng = np.random.default_rng(synth.seed64(*seed))
    rows = np.sort(np.concatenate([np.arange(64), rng.choice(np.arange(64, N - 64), 62, replace=False),
                                   np.arange(N - 64, N)]))
    if fmt == TRELLIS:
        raw = {"codes": synth.symbols(seed + [1], (N, K), 4),
               "scales": synth.uniform_f16(seed + [2], (N, K // 64), 0.01, 0.03),
               "seeds": synth.u16(seed + [3], N)}
        pw = gpu_weight(fmt, raw, N, K)
        sub = {"codes": raw["codes"][rows], "scales": raw["scales"][rows], "seeds": raw["seeds"][rows]}
        del raw
    else:
        w = synth.gauss_torch(seed, (N, K), 0.02)
        pw = ebq.PackedWeight.empty(fmt, N, K)
        ebq.qweight_quantize(fmt, w, pw)
        sub = {"w": host(w[torch.from_numpy(rows).cuda()])}
        del w
    rp, rs, rseeds = oracle_weight(fmt, sub)
    x = synth.gauss(seed + [9], (B, K))
    q, pl, d, s = gpu_act_planes(x)
    y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    plan = ebq.GroupedPlan([(pw, q, pl, d, s, y)], B)
    plan.run()
    _sync()
    rq, rd, _ = oracle.act_quant(x)
    yr, absT, _ = oracle.gemv(fmt, rp, rs, rseeds, K, rq, rd)
    assert_close_terms(host(y)[:, rows], yr, absT, what="%s %dx%d B=%d" % (NAMES[fmt], N, K, B))


@pytest.mark.parametrize("B", [2, 3, 4, 5, 6, 7])
def test_grouped_every_batch_size(B):
    """The grouped launch at every batch size between 1 and 8 (each batch size and
    format has its own workgroup size), all five formats in one plan."""
    specs = [(SIGN1, 200, 2048), (TERN, 130, 1280), (INT4, 70, 1024), (INT2, 90, 2560), (TRELLIS, 65, 1536)]
    entries, refs = [], []
    for i, (fmt, N, K) in enumerate(specs):
        raw, pw, (rp, rs, rseeds), x = _prep(fmt, N, K, 400 + 10 * B + i, B)
        q, pl, d, s = gpu_act_planes(x)
        y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
        entries.append((pw, q, pl, d, s, y))
        rq, rd, _ = oracle.act_quant(x)
        refs.append(oracle.gemv(fmt, rp, rs, rseeds, K, rq, rd))
    plan = ebq.GroupedPlan(entries, B)
    for rep in range(2):
        for e in entries:
            e[5].fill_(float("nan"))
        plan.run()
        _sync()
        for (fmt, N, K), e, (yr, absT, _) in zip(specs, entries, refs):
            assert_close_terms(host(e[5]), yr, absT, what="grouped %s B=%d rep %d" % (NAMES[fmt], B, rep))


# ---------------------------------------------------------------------------------------------
# trellis decode, unpack, GEMM
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("oblock", [256, 32])
@pytest.mark.parametrize("N,K", [(1, 256), (33, 1024), (17, 5120), (5, 1280)])
def test_trellis_decode_bit_exact(oblock, N, K):
    raw = raw_weight(TRELLIS, N, K, 200)
    pw = gpu_weight(TRELLIS, raw, N, K)
    wq = torch.empty((N, K), dtype=torch.int8, device="cuda")
    dw = torch.empty((N, K // oblock), dtype=torch.float32, device="cuda")
    ebq.qtrellis_decode_i8(pw, oblock, wq, dw)
    _sync()
    rp, rs, rseeds = oracle_weight(TRELLIS, raw)
    rwq, rdw = oracle.trellis_decode_i8(rp, rseeds, rs, K, oblock)
    assert (host(wq) == rwq).all()
    assert (host(dw).view(np.uint32) == rdw.view(np.uint32)).all()


@pytest.mark.parametrize("oblock", [256, 32])
def test_trellis_decode_zero_and_tiny_scales(oblock):
    """Rows whose scales are zero (zero blocks: d = 0, q = 0) or the smallest
    fp16 subnormal 2^-24, and seeds 0 and 0xFFFF."""
    N, K = 6, 1024
    raw = raw_weight(TRELLIS, N, K, 202)
    raw["scales"][0] = 0
    raw["scales"][1] = 1                                   # fp16 2^-24
    raw["scales"][2, ::2] = 0
    raw["seeds"][3] = 0
    raw["seeds"][4] = 0xFFFF
    pw = gpu_weight(TRELLIS, raw, N, K)
    wq = torch.full((N, K), 77, dtype=torch.int8, device="cuda")
    dw = torch.full((N, K // oblock), -1.0, dtype=torch.float32, device="cuda")
    ebq.qtrellis_decode_i8(pw, oblock, wq, dw)
    _sync()
    rp, rs, rseeds = oracle_weight(TRELLIS, raw)
    rwq, rdw = oracle.trellis_decode_i8(rp, rseeds, rs, K, oblock)
    assert not rwq[0].any() and (rdw[0] == 0).all()
    assert (host(wq) == rwq).all()
    assert (host(dw).view(np.uint32) == rdw.view(np.uint32)).all()


def test_trellis_decode_unaligned_output():
    """int8 output at a 4-byte (not 16-byte) aligned address: the same bytes."""
    N, K = 9, 1280
    raw = raw_weight(TRELLIS, N, K, 201)
    pw = gpu_weight(TRELLIS, raw, N, K)
    buf = torch.zeros(N * K + 16, dtype=torch.int8, device="cuda")
    wq = buf[4:4 + N * K].view(N, K)
    assert wq.data_ptr() % 16 == 4
    dw = torch.empty((N, K // 256), dtype=torch.float32, device="cuda")
    ebq.qtrellis_decode_i8(pw, 256, wq, dw)
    _sync()
    rp, rs, rseeds = oracle_weight(TRELLIS, raw)
    rwq, rdw = oracle.trellis_decode_i8(rp, rseeds, rs, K, 256)
    assert (host(wq) == rwq).all()
    assert (host(dw).view(np.uint32) == rdw.view(np.uint32)).all()
    assert (host(buf[:4]) == 0).all() and (host(buf[4 + N * K:]) == 0).all()


@pytest.mark.parametrize("fmt", [TERN, INT2, SIGN1, INT4])
def test_unpack_i8(fmt):
    N, K = 40, 1024
    raw = raw_weight(fmt, N, K, 210 + fmt)
    pw = gpu_weight(fmt, raw, N, K)
    wq = torch.empty((N, K), dtype=torch.int8, device="cuda")
    dw = torch.empty((N, K // 32), dtype=torch.float32, device="cuda")
    ebq.qweight_unpack_i8(pw, wq, dw)
    _sync()
    rp, rs, _ = oracle_weight(fmt, raw)
    c = oracle.unpack(fmt, rp, K).astype(np.int32)
    lev = {TERN: c, INT2: 2 * c - 3, SIGN1: 2 * c - 1, INT4: 2 * c - 15}[fmt]
    assert (host(wq) == lev).all()
    blk = oracle.scale_block(fmt)
    f = np.repeat(rs.view(np.float16).astype(np.float32), blk // 32, axis=1)
    if fmt in (INT2, INT4):
        f = f * np.float32(0.5)
    assert (host(dw) == f).all()


@pytest.mark.parametrize("kblock", [256, 32])
@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (17, 130, 512), (200, 64, 1024), (128, 257, 2048),
                                   (300, 200, 1024), (513, 1300, 512), (256, 128, 1280),
                                   (600, 300, 3072), (64, 1000, 2048), (48, 520, 1024)])
def test_gemm_parity(kblock, M, N, K):
    xq = synth.integers([220, M, K], (M, K), -127, 127).astype(np.int8)
    wq = synth.integers([221, N, K], (N, K), -127, 127).astype(np.int8)
    dx = synth.uniform([222], (M, K // kblock), 1e-3, 0.1)
    dw = synth.uniform([223], (N, K // kblock), 1e-3, 0.1)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ebq.qgemm_i8(dev(xq), dev(dx), dev(wq), dev(dw), kblock, y)
    _sync()
    yr, absT = oracle.gemm_i8(xq, dx, wq, dw, kblock)
    assert_close_terms(host(y), yr, absT, what="gemm %dx%dx%d/%d" % (M, N, K, kblock))


def test_gemm_cut_tiles_deterministic():
    """2048 x 5120 x 17408 runs as equal runs of 1.25 tiles, so most tiles are cut
    between two runs; each cut tile gets exactly two fp32 adds onto zero:
    bit-identical reruns."""
    M, N, K = 2048, 5120, 17408
    g = torch.Generator(device="cuda")
    g.manual_seed(synth.seed64(225))
    xq = torch.randint(-127, 128, (M, K), generator=g, device="cuda", dtype=torch.int8)
    wq = torch.randint(-127, 128, (N, K), generator=g, device="cuda", dtype=torch.int8)
    dx = torch.rand((M, K // 256), generator=g, device="cuda") * 0.1 + 1e-3
    dw = torch.rand((N, K // 256), generator=g, device="cuda") * 0.1 + 1e-3
    outs = []
    for _ in range(3):
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        ebq.qgemm_i8(xq, dx, wq, dw, 256, y)
        _sync()
        outs.append(host(y).view(np.uint32).copy())
    assert (outs[0] == outs[1]).all() and (outs[0] == outs[2]).all()


@pytest.mark.parametrize("N,K", [(17408, 5120), (5120, 17408)])
def test_gemm_full_size_sampled(N, K):
    """The prefill GEMMs at their benchmark shapes (2048 x 17408 x 5120 and
    2048 x 5120 x 17408, 256-blocks), checked on sampled rows and columns against
    the oracle."""
    M = 2048
    g = torch.Generator(device="cuda")
    g.manual_seed(synth.seed64(240 + K))
    xq = torch.randint(-127, 128, (M, K), generator=g, device="cuda", dtype=torch.int8)
    wq = torch.randint(-127, 128, (N, K), generator=g, device="cuda", dtype=torch.int8)
    dx = torch.rand((M, K // 256), generator=g, device="cuda") * 0.1 + 1e-3
    dw = torch.rand((N, K // 256), generator=g, device="cuda") * 0.1 + 1e-3
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ebq.qgemm_i8(xq, dx, wq, dw, 256, y)
    _sync()
    rng = np.random.default_rng(241)
    rows = np.sort(np.concatenate([[0, M - 1], rng.choice(M, 30, replace=False)]))
    cols = np.sort(np.concatenate([[0, N - 1], rng.choice(N, 94, replace=False)]))
    yr, absT = oracle.gemm_i8(host(xq)[rows], host(dx)[rows], host(wq)[cols], host(dw)[cols], 256)
    assert_close_terms(host(y)[np.ix_(rows, cols)], yr, absT, what="gemm full size, sampled")
    assert np.isfinite(host(y)).all()


@pytest.mark.parametrize("M,N", [(2000, 5118), (2048, 4100)])
def test_gemm_cut_tiles_ragged(M, N):
    """Equal runs of K-groups with ragged edges: 2000 x 5118 (N not a multiple of 4:
    the cut tiles are zeroed 4 bytes at a time) and 2048 x 4100 (16-byte zeroing, a
    partial last column tile), K = 2048; every entry written, sampled rows and columns
    (with both edges) against the oracle."""
    K = 2048
    g = torch.Generator(device="cuda")
    g.manual_seed(synth.seed64(226, N))
    xq = torch.randint(-127, 128, (M, K), generator=g, device="cuda", dtype=torch.int8)
    wq = torch.randint(-127, 128, (N, K), generator=g, device="cuda", dtype=torch.int8)
    dx = torch.rand((M, K // 256), generator=g, device="cuda") * 0.1 + 1e-3
    dw = torch.rand((N, K // 256), generator=g, device="cuda") * 0.1 + 1e-3
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ebq.qgemm_i8(xq, dx, wq, dw, 256, y)
    _sync()
    yh = host(y)
    assert np.isfinite(yh).all()
    rng = np.random.default_rng(227)
    rows = np.sort(np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), 30, replace=False)]))
    cols = np.sort(np.concatenate([[0, N - 1], rng.choice(np.arange(1, N - 1), 62, replace=False)]))
    yr, absT = oracle.gemm_i8(host(xq)[rows], host(dx)[rows], host(wq)[cols], host(dw)[cols], 256)
    assert_close_terms(yh[np.ix_(rows, cols)], yr, absT, what="gemm cut tiles, ragged")


def test_prefill_pipeline_small():
    """Rotation + Q8, trellis decode, GEMM chained as in prefill."""
    M, K, N = 96, 1024, 160
    x = synth.with_outliers(synth.gauss([230], (M, K)), [231])
    sb = synth.sign_bits([232], K)
    raw = raw_weight(TRELLIS, N, K, 233)
    pw = gpu_weight(TRELLIS, raw, N, K)
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    dx = torch.empty((M, K // 256), dtype=torch.float32, device="cuda")
    sx = torch.empty((M, K // 256), dtype=torch.int32, device="cuda")
    ebq.qact_hadamard_quant_i8(dev(x), dev(sb), 256, xq, dx, sx)
    wq = torch.empty((N, K), dtype=torch.int8, device="cuda")
    dw = torch.empty((N, K // 256), dtype=torch.float32, device="cuda")
    ebq.qtrellis_decode_i8(pw, 256, wq, dw)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ebq.qgemm_i8(xq, dx, wq, dw, 256, y)
    _sync()
    rxq, rdx, _ = oracle.hadamard_quant(x, sb, 256)
    rp, rs, rseeds = oracle_weight(TRELLIS, raw)
    rwq, rdw = oracle.trellis_decode_i8(rp, rseeds, rs, K, 256)
    yr, absT = oracle.gemm_i8(rxq, rdx, rwq, rdw, 256)
    assert_close_terms(host(y), yr, absT, what="prefill")
