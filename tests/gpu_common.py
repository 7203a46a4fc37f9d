"""Helpers shared by the GPU tests: move arrays, build the same matrix on both
sides from one set of raw draws, and the parity assertion for fp32 results."""
import numpy as np

import oracle
import synth

TERN, INT2, SIGN1, INT4, TRELLIS = 1, 2, 3, 4, 5
NAMES = {TERN: "tern_b3", INT2: "int2", SIGN1: "sign1", INT4: "int4", TRELLIS: "trellis2"}


def dev(a):
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).cuda()


def host(t, dtype=None):
    a = t.detach().cpu().numpy()
    return a.view(dtype) if dtype is not None else a


def gpu_scales_rowmajor(pw):
    """The packed matrix's scales read back as row-major fp16 bits [rows][cols/block]."""
    import torch

    import extreme_bit_quantized_amd as ebq

    out = torch.empty((pw.rows, pw.cols // ebq.qfmt_scale_block(pw.fmt)), dtype=torch.int16, device="cuda")
    ebq.qweight_get_scales(pw, out)
    return host(out).view(np.uint16)


def raw_weight(fmt, N, K, seed):
    """Raw draws for one matrix: floats for the quantized formats, integer
    codes + fp16 scales (+ seeds) for ternary-from-trits and trellis."""
    if fmt == TRELLIS:
        return {"codes": synth.symbols([seed, 1], (N, K), 4),
                "scales": synth.uniform_f16([seed, 2], (N, K // 64), 0.01, 0.03),
                "seeds": synth.u16([seed, 3], N)}
    return {"w": synth.gauss([seed, 0], (N, K), 0.02)}


def oracle_weight(fmt, raw):
    """Oracle's packed bytes, fp16 scales, seeds."""
    if "w" in raw:
        c, s = oracle.quantize(fmt, raw["w"])
        return oracle.pack(fmt, c), s, None
    return oracle.pack(fmt, raw["codes"]), raw["scales"], raw.get("seeds")


def gpu_weight(fmt, raw, N, K):
    """Library's packed matrix built on the GPU from the same raw draws."""
    import extreme_bit_quantized_amd as ebq

    pw = ebq.PackedWeight.empty(fmt, N, K)
    if "w" in raw:
        ebq.qweight_quantize(fmt, dev(raw["w"]), pw)
    else:
        ebq.qweight_pack(fmt, dev(raw["codes"]), pw)
        ebq.qweight_set_scales(pw, dev(raw["scales"]))
        if raw.get("seeds") is not None:
            pw.seeds.copy_(dev(raw["seeds"]))
    return pw


def gpu_act(x, qblock=32):
    import torch

    import extreme_bit_quantized_amd as ebq

    xt = dev(x) if isinstance(x, np.ndarray) else x
    B, K = xt.shape
    q = torch.empty((B, K), dtype=torch.int8, device="cuda")
    d = torch.empty((B, K // qblock), dtype=torch.float32, device="cuda")
    s = torch.empty((B, K // qblock), dtype=torch.int32, device="cuda")
    ebq.qact_quant_i8(xt, qblock, q, d, s)
    return q, d, s


def gpu_act_planes(x):
    """Q8 per 32 plus the 4-bit planes of q: (q, planes, d, qsum) on the device."""
    import torch

    import extreme_bit_quantized_amd as ebq

    q, d, s = gpu_act(x)
    B, K = q.shape
    planes = torch.empty((B, K // 32, 8), dtype=torch.int32, device="cuda")
    ebq.qact_planes(q, planes)
    return q, planes, d, s


def assert_close_terms(y_gpu, y_ref, absT, rel=1e-4, what=""):
    """|y_gpu - y_ref| <= rel * sum|T|, and y_gpu == 0 exactly where sum|T| == 0."""
    y_gpu = np.asarray(y_gpu, np.float64)
    err = np.abs(y_gpu - y_ref)
    bad = err > rel * absT
    assert not bad.any(), "%s: %d/%d outside tolerance, worst ratio %.3g" % (
        what, bad.sum(), bad.size, (err / np.maximum(absT, 1e-300)).max())
    z = absT == 0
    assert (y_gpu[z] == 0).all(), what + ": nonzero output where every term is zero"
