"""GPU parity of the trellis encoder (Viterbi over the 2^16-state bit-shift
trellis) against the CPU oracle: codes, seeds, scales and the minimum cost,
bit for bit, through the C ABI.  Sizes keep the oracle to seconds: its
textbook recursion visits 2^16 states x 4 predecessors per weight."""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import TRELLIS, dev, gpu_scales_rowmajor, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import extreme_bit_quantized_amd as ebq  # noqa: E402

ebq.load()


def gpu_encode(w, rows_per_pass=None, scales_in=None):
    N, K = w.shape
    per = N if rows_per_pass is None else rows_per_pass
    out = ebq.PackedWeight.empty(TRELLIS, N, K)
    out.codes.fill_(0xA5)                        # padding must come back zeroed
    ws = torch.empty(ebq.qtrellis_encode_workspace_bytes(N, K, per), dtype=torch.uint8, device="cuda")
    cost = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    si = None if scales_in is None else dev(scales_in)
    ebq.qtrellis_encode(dev(w), out, ws, per, scales_in=si, cost=cost)
    torch.cuda.synchronize()
    return out, host(out.codes), host(out.seeds).view(np.uint16), gpu_scales_rowmajor(out), host(cost)


def check(w, rows_per_pass=None, scales_in=None, what=""):
    out, codes, seeds, scales, cost = gpu_encode(w, rows_per_pass, scales_in)
    rp, rs, rsc, rc = oracle.trellis_encode(w, scales_in)
    assert (scales == rsc).all(), "scales " + what
    assert (seeds == rs).all(), "seeds " + what
    assert (codes == rp).all(), "codes " + what
    assert (cost.view(np.uint32) == rc.view(np.uint32)).all(), "cost %s: %s vs %s" % (what, cost, rc)
    return out


@pytest.mark.parametrize("N,K", [(3, 64), (2, 320), (4, 1024)])
def test_encode_bit_exact(N, K):
    w = synth.gauss([900, N, K], (N, K), 0.02)
    check(w, what="%dx%d" % (N, K))


def test_encode_full_row_width():
    """One row of the real 5120 input width (the oracle takes a few seconds)."""
    w = synth.gauss([901], (1, 5120), 0.02)
    check(w, what="1x5120")


def test_encode_in_passes():
    """Rows in passes of 2 (the workspace holds one pass of choices), odd count."""
    w = synth.gauss([902], (5, 256), 1.0)
    check(w, rows_per_pass=2, what="passes of 2")


def test_encode_given_scales_recovers_trellis_rows():
    """Rows the trellis produces exactly, encoded with their own scales, come
    back with zero cost and decode to themselves."""
    N, K = 3, 192
    codes = synth.symbols([903, 1], (N, K), 4)
    seeds = synth.u16([903, 2], N)
    sc = synth.uniform_f16([903, 3], (N, K // 64), 0.01, 0.03)
    w = oracle.trellis_decode_f32(oracle.pack(TRELLIS, codes), seeds, sc, K)
    check(w, scales_in=sc, what="given scales")
    out, codes, sd, scales, cost = gpu_encode(w, scales_in=sc)
    assert (cost == 0).all()
    back = oracle.trellis_decode_f32(codes, sd, scales, K)
    assert (back == w).all()


def test_encode_edge_rows():
    """Zero rows (every path ties), a zero block inside a row, constant rows
    (many ties), tiny and large magnitudes, a single 64-weight row."""
    K = 256
    w = synth.gauss([904], (6, K), 1.0)
    w[0] = 0.0
    w[1, 64:128] = 0.0
    w[2] = 0.75
    w[3] *= 1e-30
    w[4] *= 1e3
    w[5, ::2] = -w[5, 1::2]
    check(w, what="edge rows")
    check(synth.gauss([905], (1, 64), 0.02), what="one block")


def test_encode_scales_rule_many_blocks():
    """The RMS scale rule (fused sum of squares, correctly rounded square root,
    fp16 rounding) on 8192 blocks of widely spread magnitudes; the Viterbi
    result of a few of those rows against the oracle."""
    N, K = 4096, 128
    w = synth.gauss([906], (N, K), 1.0) * synth.uniform([907], (N, 1), 1e-6, 1e4)
    out, codes, seeds, scales, cost = gpu_encode(w, rows_per_pass=1024)
    want = np.array([[oracle.trellis_rms_scale(w[n, 64 * b:64 * b + 64]) for b in range(2)] for n in range(N)],
                    np.uint16)
    assert (scales == want).all()
    rows = [0, 1, 2047, 4095]
    rp, rs, rsc, rc = oracle.trellis_encode(w[rows])
    assert (codes[rows] == rp).all() and (seeds[rows] == rs).all()
    assert (cost[rows].view(np.uint32) == rc.view(np.uint32)).all()


def test_encode_deterministic():
    w = synth.gauss([908], (3, 512), 0.02)
    a = gpu_encode(w)
    b = gpu_encode(w, rows_per_pass=1)
    for x, y in zip(a[1:], b[1:]):
        assert (np.asarray(x).view(np.uint8) == np.asarray(y).view(np.uint8)).all()
