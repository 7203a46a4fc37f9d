"""GPU parity of the Q8/Q4 KV cache quantizer (bit-exact) and of grouped decode
attention over it (within the oracle's fp32 error allowance), through the C ABI."""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import extreme_bit_quantized_amd as ebq  # noqa: E402

ebq.load()
D = 256
FMTS = [ebq.QKV_Q8, ebq.QKV_Q4]


def gpu_quant(fmt, x):
    xs = dev(np.ascontiguousarray(x, np.float32))
    codes = torch.empty(x.shape[:-1] + (ebq.qkv_row_bytes(fmt),), dtype=torch.uint8, device="cuda")
    scales = torch.empty(x.shape[:-1] + (D // 32,), dtype=torch.int16, device="cuda")
    ebq.qkv_quant(fmt, xs, codes, scales)
    return codes, scales


@pytest.mark.parametrize("fmt", FMTS)
def test_kv_quant_bit_exact(fmt):
    x = synth.gauss([950, fmt], (300, D)) * synth.uniform([951, fmt], (300, 1), 1e-4, 1e3)
    x[0, :32] = 0.0
    x[1, 32:64] = 1e-38                       # reciprocal of the scale overflows: codes 0
    x[2, 64:96] = np.float32(3.5)             # every value on the top level
    x[3] = np.tile(np.float32([0.5, -1.5, 2.5, 7.0]), D // 4)   # ties
    codes, scales = gpu_quant(fmt, x)
    torch.cuda.synchronize()
    rc, rs = oracle.kv_quant(fmt, x)
    assert (host(codes) == rc).all()
    assert (host(scales).view(np.uint16) == rs).all()


def _cache(fmt, seed, n_kv, t_cap, kscale=1.0):
    K = synth.gauss([seed, 1], (n_kv, t_cap, D)) * np.float32(kscale)
    V = synth.gauss([seed, 2], (n_kv, t_cap, D))
    kc, ks = gpu_quant(fmt, K)
    vc, vs = gpu_quant(fmt, V)
    return K, V, kc, ks, vc, vs


def run_attn(fmt, q, kc, ks, vc, vs, T, hpb=None):
    n_kv = kc.shape[0]
    group = q.shape[0] // n_kv
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(ebq.qattn_decode_workspace_bytes(n_kv, group, T), dtype=torch.uint8, device="cuda")
    ebq.qattn_decode(fmt, dev(q), kc, ks, vc, vs, T, out, ws, heads_per_block=hpb)
    torch.cuda.synchronize()
    return host(out)


def check(fmt, q, kc, ks, vc, vs, T, hpb=None, what=""):
    got = run_attn(fmt, q, kc, ks, vc, vs, T, hpb)
    want, bound = oracle.attn_decode(fmt, q, host(kc), host(ks).view(np.uint16), host(vc),
                                     host(vs).view(np.uint16), T)
    err = np.abs(got.astype(np.float64) - want)
    assert np.isfinite(got).all(), what
    assert (err <= bound).all(), "%s: worst err/bound %.3g" % (what, float((err / bound).max()))
    return got


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n_kv,group,T,t_cap", [(1, 6, 1, 1), (2, 6, 77, 96), (4, 6, 1000, 1024),
                                                (1, 1, 300, 300), (2, 8, 513, 600), (3, 3, 256, 256),
                                                (4, 6, 4099, 5000)])
def test_attn_parity(fmt, n_kv, group, T, t_cap):
    _, _, kc, ks, vc, vs = _cache(fmt, 960 + T, n_kv, t_cap)
    q = synth.gauss([961, T], (n_kv * group, D))
    a = check(fmt, q, kc, ks, vc, vs, T, what="packed T=%d" % T)
    b = check(fmt, q, kc, ks, vc, vs, T, hpb=1, what="one row per block T=%d" % T)
    # the two launches do the same arithmetic per row
    assert (a == b).all()


@pytest.mark.parametrize("fmt", FMTS)
def test_attn_dominant_tokens_at_chunk_edges(fmt):
    """Long ragged context; each query row of a group has its own dominant
    token, placed at chunk edges and at the last token: the output is close to
    that token's value row, within the allowance."""
    n_kv, group, T = 2, 6, 70001
    K = synth.gauss([970, 1], (n_kv, T, D)) * np.float32(0.05)
    q = synth.gauss([970, 3], (n_kv * group, D))
    spots = [0, 255, 256, 65535, 65536, T - 1]
    for h in range(n_kv):
        for g in range(group):
            K[h, spots[g]] = q[h * group + g] * np.float32(2.0)
    V = synth.gauss([970, 2], (n_kv, T, D))
    kc, ks = gpu_quant(fmt, K)
    vc, vs = gpu_quant(fmt, V)
    got = check(fmt, q, kc, ks, vc, vs, T, what="dominant")
    Vd = oracle.kv_dequant(fmt, host(vc), host(vs).view(np.uint16), D)
    for h in range(n_kv):
        for g in range(group):
            assert np.abs(got[h * group + g] - Vd[h, spots[g]]).max() < 0.05


def test_attn_full_context_64k():
    """The 27B-shaped decode step at a 64K context: 4 KV heads x 6 query heads."""
    fmt, n_kv, group, T = ebq.QKV_Q4, 4, 6, 65536
    _, _, kc, ks, vc, vs = _cache(fmt, 980, n_kv, T, kscale=2.0)
    q = synth.gauss([981], (n_kv * group, D))
    check(fmt, q, kc, ks, vc, vs, T, what="64K")


def test_attn_deterministic_and_zero_query():
    fmt, n_kv, group, T = ebq.QKV_Q8, 2, 6, 3000
    _, V, kc, ks, vc, vs = _cache(fmt, 990, n_kv, T)
    q = synth.gauss([991], (n_kv * group, D))
    a = run_attn(fmt, q, kc, ks, vc, vs, T)
    b = run_attn(fmt, q, kc, ks, vc, vs, T)
    assert (a == b).all()
    # a zero query weighs every token equally: the mean of the cached values
    z = check(fmt, np.zeros_like(q), kc, ks, vc, vs, T, what="zero query")
    Vd = oracle.kv_dequant(fmt, host(vc), host(vs).view(np.uint16), D)
    for h in range(n_kv):
        assert np.abs(z[h * group] - Vd[h].mean(axis=0)).max() < 1e-5


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("pos", [0, 70])
def test_attn_small_terms_beside_a_dominant_token(fmt, pos):
    """One chunk, one dominant token whose value row has zero codes: those
    outputs are sums of terms some 1e-14 times smaller than the dominant one,
    and must keep their relative accuracy (no offset added to the codes and
    taken off again, which would swamp them)."""
    T, G = 100, 6
    K = synth.gauss([995, pos, 1], (1, T, D)) * np.float32(0.05)
    q = synth.gauss([995, pos, 3], (G, D))
    K[0, pos] = q[0] * np.float32(2.0)
    V = synth.gauss([995, pos, 2], (1, T, D))
    V[0, pos, 8:16] = 0.0
    kc, ks = gpu_quant(fmt, K)
    vc, vs = gpu_quant(fmt, V)
    got = check(fmt, q, kc, ks, vc, vs, T, what="small terms")
    want, _ = oracle.attn_decode(fmt, q, host(kc), host(ks).view(np.uint16), host(vc), host(vs).view(np.uint16), T)
    assert (np.abs(got[0, 8:16] - want[0, 8:16]) <= 1e-4 * np.abs(want[0, 8:16])).all()
