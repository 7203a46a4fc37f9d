"""GPU parity of the prefill path with one scale per row of each operand: the
rotation + Q8 per token row (qblock = K), the trellis decode with Q8 per weight
row (oblock = cols) and the int8 GEMM with kblock = K, against the oracle.
Integer outputs and scales bit-exact; the GEMM's fp32 output within
1e-4 * sum|T| (one K-block, so sum|T| = |dx dw I|)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import TRELLIS, assert_close_terms, dev, gpu_weight, host, oracle_weight, raw_weight

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import extreme_bit_quantized_amd as ebq  # noqa: E402

ebq.load()


def _sync():
    torch.cuda.synchronize()


def _rand_gemm(M, N, K, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(synth.seed64(seed, M, N, K))
    xq = torch.randint(-127, 128, (M, K), generator=g, device="cuda", dtype=torch.int8)
    wq = torch.randint(-127, 128, (N, K), generator=g, device="cuda", dtype=torch.int8)
    dx = torch.rand((M, 1), generator=g, device="cuda") * 0.1 + 1e-3
    dw = torch.rand((N, 1), generator=g, device="cuda") * 0.1 + 1e-3
    return xq, dx, wq, dw


def _check_sampled(y, xq, dx, wq, dw, K, nrows, ncols, seed, what):
    M, N = y.shape
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, nrows), replace=False)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, min(N, ncols), replace=False)]))
    yh = host(y)
    assert np.isfinite(yh).all(), what + ": an output was not written"
    yr, absT = oracle.gemm_i8(host(xq)[rows], host(dx)[rows], host(wq)[cols], host(dw)[cols], K)
    assert_close_terms(yh[np.ix_(rows, cols)], yr, absT, what=what)


# Shapes by path (256 compute units): small shapes take the 128 x 64 wave tile,
# 2048 x 5120 the 128 x 80 one, 2048 x 17408 the 128 x 96 one, 2048 x 8192 the
# 128 x 128 one; K a multiple of 128 runs 128-byte stages (1, 2, 3, 5 and more
# stages: each takes its own path through the last two stages), an odd multiple
# of 64 the 64-byte ones (odd stage count included).  A first output register
# of each wave tile read before its last MFMA had written it (in the kernel's
# final K-step) once broke 1, 3 and 5 stages here while 2 passed.
@pytest.mark.parametrize("M,N,K", [(64, 96, 64), (300, 520, 192), (513, 700, 640), (700, 333, 1280),
                                   (257, 2000, 3072), (1, 17, 128), (255, 129, 1088), (256, 128, 128),
                                   (256, 128, 256), (256, 128, 384), (512, 512, 1280)])
def test_gemm_rowscale_whole(M, N, K):
    xq, dx, wq, dw = _rand_gemm(M, N, K, 300)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ebq.qgemm_i8(xq, dx, wq, dw, K, y)
    _sync()
    yr, absT = oracle.gemm_i8(host(xq), host(dx), host(wq), host(dw), K)
    assert_close_terms(host(y), yr, absT, what="gemm per-row %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [(2048, 5120, 1088), (2048, 8192, 640), (2048, 8192, 576),
                                   (2048, 17408, 5120), (2048, 5120, 17408)])
def test_gemm_rowscale_large_sampled(M, N, K):
    """The wave-tile widths 80, 96 and 128 and both stage sizes at full width, and the
    two prefill GEMMs at their benchmark shapes: every output written, sampled
    rows and columns (both edges) against the oracle."""
    xq, dx, wq, dw = _rand_gemm(M, N, K, 301)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ebq.qgemm_i8(xq, dx, wq, dw, K, y)
    _sync()
    _check_sampled(y, xq, dx, wq, dw, K, 24, 70, 302, "gemm per-row %dx%dx%d" % (M, N, K))


def _tile_rows(M, seed, per_tile=3):
    """per_tile rows from every 256-row tile (its first and last valid row among them)."""
    rng = np.random.default_rng(seed)
    rows = []
    for m0 in range(0, M, 256):
        m1 = min(M, m0 + 256)
        rows += [m0, m1 - 1] + list(rng.integers(m0, m1, per_tile - 2))
    return np.unique(np.array(rows))


def _check_rows_all_cols(y, xq, dx, wq, dw, K, rows, what):
    yh = host(y)
    assert np.isfinite(yh).all(), what + ": an output was not written"
    yr, absT = oracle.gemm_i8(host(xq)[rows], host(dx)[rows], host(wq), host(dw), K)
    assert_close_terms(yh[rows], yr, absT, what=what)


# More tiles than compute units in rounds that do not come out whole (wave tile
# 80 or 96 on 256 units), ragged M and N, K of 1, 2, 3 and 5 stages: every tile
# checked (three rows of each 256-row tile, every column).
@pytest.mark.parametrize("M,N,K", [(1000, 17408, 128), (1000, 17408, 256), (777, 17408, 384),
                                   (1500, 15000, 640), (2048, 12000, 640), (2048, 17408, 384),
                                   (2048, 13000, 256)])
def test_gemm_rowscale_many_tiles(M, N, K):
    xq, dx, wq, dw = _rand_gemm(M, N, K, 303)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ebq.qgemm_i8(xq, dx, wq, dw, K, y)
    _sync()
    _check_rows_all_cols(y, xq, dx, wq, dw, K, _tile_rows(M, 304), "gemm %dx%dx%d" % (M, N, K))


def test_gemm_rowscale_prefill_shape_every_tile_and_repeatable():
    """The 2048 x 17408 x 5120 prefill GEMM (728 tiles, 40 stages each): every
    tile checked, and a second run bit-identical."""
    M, N, K = 2048, 17408, 5120
    xq, dx, wq, dw = _rand_gemm(M, N, K, 305)
    outs = []
    for _ in range(2):
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        ebq.qgemm_i8(xq, dx, wq, dw, K, y)
        _sync()
        outs.append(y)
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
    _check_rows_all_cols(outs[0], xq, dx, wq, dw, K, _tile_rows(M, 306, 2), "gemm prefill up")


def test_gemm_rowscale_concurrent_streams():
    """Two GEMMs in flight at once on two streams, three times over: both right."""
    shapes = [(2048, 17408, 640), (1500, 15000, 384)]
    ins = [_rand_gemm(M, N, K, 307 + i) for i, (M, N, K) in enumerate(shapes)]
    ys = [torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda") for (M, N, K) in shapes]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    _sync()
    for rep in range(3):
        for (M, N, K), (xq, dx, wq, dw), y, st in zip(shapes, ins, ys, streams):
            with torch.cuda.stream(st):
                ebq.qgemm_i8(xq, dx, wq, dw, K, y, stream=st.cuda_stream)
    _sync()
    for i, ((M, N, K), (xq, dx, wq, dw), y) in enumerate(zip(shapes, ins, ys)):
        _check_rows_all_cols(y, xq, dx, wq, dw, K, _tile_rows(M, 308 + i, 2), "gemm concurrent %d" % i)


def test_gemm_rowscale_repeatable_and_extremes():
    """Operands at the int8 extremes (every product 127 * 127 or -127 * 127:
    |I| = 16129 K, the largest sum) and zero scales: exact results, and two runs
    bit-identical."""
    M, N, K = 300, 200, 17408
    xq = torch.full((M, K), 127, dtype=torch.int8, device="cuda")
    xq[1::2] = -127
    wq = torch.full((N, K), 127, dtype=torch.int8, device="cuda")
    dx = torch.full((M, 1), 0.5, device="cuda")
    dw = torch.full((N, 1), 0.25, device="cuda")
    dw[3] = 0.0
    outs = []
    for _ in range(2):
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        ebq.qgemm_i8(xq, dx, wq, dw, K, y)
        _sync()
        outs.append(host(y).copy())
    assert (outs[0].view(np.uint32) == outs[1].view(np.uint32)).all()
    exp = np.float32(0.125) * np.float32(16129 * K)
    assert (outs[0][0::2, :3] == exp).all() and (outs[0][1::2, :3] == -exp).all()
    assert (outs[0][:, 3] == 0).all()


@pytest.mark.parametrize("B,K", [(1, 256), (3, 512), (5, 5120), (17, 17408), (2, 4096), (3, 32768)])
def test_hadamard_quant_row_bit_exact(B, K):
    x = synth.with_outliers(synth.gauss([310, B, K], (B, K)), [311, B, K])
    if B > 2:
        x[1] = 0.0                                          # a zero row: d = 0, q = 0
        x[2] *= np.float32(2.0 ** -128)                     # subnormal row: 1/d overflows
    sb = synth.sign_bits([312, K], K)
    q = torch.full((B, K), 99, dtype=torch.int8, device="cuda")
    d = torch.empty((B, 1), dtype=torch.float32, device="cuda")
    s = torch.empty((B, 1), dtype=torch.int32, device="cuda")
    ebq.qact_hadamard_quant_i8(dev(x), dev(sb), K, q, d, s)
    _sync()
    rq, rd, rs = oracle.hadamard_quant(x, sb, K)
    assert (host(q) == rq).all()
    assert (host(d).view(np.uint32) == rd.view(np.uint32)).all()
    assert (host(s) == rs).all()


@pytest.mark.parametrize("N,K", [(1, 256), (5, 1280), (33, 5120), (7, 17408), (3, 32768)])
def test_trellis_decode_row_bit_exact(N, K):
    raw = raw_weight(TRELLIS, N, K, 320 + N)
    if N > 3:
        raw["scales"][1] = 0                                # zero row
        raw["scales"][2, ::3] = 0
        raw["seeds"][3] = 0xFFFF
    pw = gpu_weight(TRELLIS, raw, N, K)
    wq = torch.full((N, K), 77, dtype=torch.int8, device="cuda")
    dw = torch.empty((N, 1), dtype=torch.float32, device="cuda")
    ebq.qtrellis_decode_i8(pw, K, wq, dw)
    _sync()
    rp, rs, rseeds = oracle_weight(TRELLIS, raw)
    rwq, rdw = oracle.trellis_decode_i8(rp, rseeds, rs, K, K)
    assert (host(wq) == rwq).all()
    assert (host(dw).view(np.uint32) == rdw.view(np.uint32)).all()


def test_prefill_chain_rowscale():
    """Rotation + Q8 per token, trellis decode + Q8 per weight row, GEMM with one
    scale pair per output, chained as in prefill, against the oracle redoing
    every step from the same draws."""
    M, K, N = 300, 5120, 272
    x = synth.with_outliers(synth.gauss([330], (M, K)), [331])
    sb = synth.sign_bits([332], K)
    raw = raw_weight(TRELLIS, N, K, 333)
    pw = gpu_weight(TRELLIS, raw, N, K)
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    dx = torch.empty((M, 1), dtype=torch.float32, device="cuda")
    sx = torch.empty((M, 1), dtype=torch.int32, device="cuda")
    ebq.qact_hadamard_quant_i8(dev(x), dev(sb), K, xq, dx, sx)
    wq = torch.empty((N, K), dtype=torch.int8, device="cuda")
    dw = torch.empty((N, 1), dtype=torch.float32, device="cuda")
    ebq.qtrellis_decode_i8(pw, K, wq, dw)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ebq.qgemm_i8(xq, dx, wq, dw, K, y)
    _sync()
    rxq, rdx, _ = oracle.hadamard_quant(x, sb, K)
    rp, rs, rseeds = oracle_weight(TRELLIS, raw)
    rwq, rdw = oracle.trellis_decode_i8(rp, rseeds, rs, K, K)
    assert (host(xq) == rxq).all() and (host(wq) == rwq).all()
    yr, absT = oracle.gemm_i8(rxq, rdx, rwq, rdw, K)
    assert_close_terms(host(y), yr, absT, what="prefill per-row")
