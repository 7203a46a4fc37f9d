#!/usr/bin/env python3
"""Benchmark of the extreme low-bit GEMV/GEMM path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]

Headline (the JSON line's `value`): weight-stream GB/s of batch-1 decode over the
64-layer 27B-shaped 1-bit sign stack (7 matrices per layer, 448 matrices,
21,810,380,800 weights, 3,067,084,800 bytes of codes and fp16 scales).  One step
= int8 quantization of every activation of the stack (one launch per input
width, all 64 layers at once) + one persistent grouped GEMV launch that streams
all 448 matrices.  Inputs are resident in HBM before timing starts.

The same line carries:
  roofline      the grouped GEMV kernel's algorithmic bytes per launch over its
                HIP-event duration, against 8 TB/s
  cpu_baseline  the CPU oracle timed on one layer of the same stack
  extra         the other workloads: mixed 4-bit/ternary stack at batch 1 and 8,
                one 2-bit layer (8 copies cycled), the 1024x1024 ternary GEMV,
                prefill (rotation, trellis decode, int8 MFMA GEMM), and the same
                stack as a dependent chain of 448 launches in a HIP graph
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA
TERN, INT2, SIGN1, INT4, TRELLIS = 1, 2, 3, 4, 5
WIDTHS = (5120, 6144, 17408)
METRIC = "weight-stream HBM GB/s (% of peak) + equiv. tok/s, 27B-shaped batch-1 GEMV stack"


# ---------------------------------------------------------------------------------------
# workload construction (synthetic, seeded, generated on the GPU)
# ---------------------------------------------------------------------------------------

def layer_fmt(kind: str, name: str) -> int:
    if kind == "sign1":
        return SIGN1
    if kind == "int2":
        return INT2
    if kind == "mixed":
        return INT4 if name in synth.ATTN else TERN
    raise ValueError(kind)


def seed_of(kind: str) -> int:
    return {"int2": 2, "sign1": 3, "mixed": 4}[kind]


def build_matrix(ebq, kind, layer, mi, name, N, K):
    """Quantize N(0, sigma) draws for one matrix on the GPU with the library's
    quantizer.  1-bit draws are N(0,1) (sign + mean|w|), the others N(0,0.02)."""
    import torch

    fmt = layer_fmt(kind, name)
    sigma = 1.0 if kind == "sign1" else 0.02
    w = synth.gauss_torch([seed_of(kind), layer, mi], (N, K), sigma)
    pw = ebq.PackedWeight.empty(fmt, N, K)
    ebq.qweight_quantize(fmt, w, pw)
    del w
    return pw


class Stack:
    """Packed weights of `layers` layers plus activations for batch B."""

    def __init__(self, ebq, kind: str, layers: int, B: int, shapes=synth.LAYER_SHAPES, copies_of=None):
        import torch

        self.kind, self.layers, self.B, self.shapes = kind, layers, B, shapes
        self.weights = []
        for l in range(layers):
            src = l if copies_of is None else copies_of(l)
            self.weights.append([build_matrix(ebq, kind, src, mi, name, N, K)
                                 for mi, (name, N, K) in enumerate(shapes)])
        # activations: one fp32 row per (layer, token) for each input width
        self.x = {K: synth.gauss_torch([seed_of(kind), 1000, K, B], (layers * B, K)) for K in WIDTHS}
        self.q = {K: torch.empty((layers * B, K), dtype=torch.int8, device="cuda") for K in WIDTHS}
        self.d = {K: torch.empty((layers * B, K // 32), dtype=torch.float32, device="cuda") for K in WIDTHS}
        self.s = {K: torch.empty((layers * B, K // 32), dtype=torch.int32, device="cuda") for K in WIDTHS}
        # 4-bit planes of q, read by the 1- and 2-bit GEMV instead of q
        self.planes = kind in ("sign1", "int2")
        self.pl = {K: torch.empty((layers * B, K // 32, 8), dtype=torch.int32, device="cuda") for K in WIDTHS} \
            if self.planes else None
        self.y = [[torch.empty((B, N), dtype=torch.float32, device="cuda") for (_, N, _) in shapes]
                  for _ in range(layers)]
        torch.cuda.synchronize()

    def act(self, l, K):
        """(q, planes or None, d, qsum) of layer l's tokens at input width K."""
        B = self.B
        sl = slice(l * B, (l + 1) * B)
        return (self.q[K][sl], self.pl[K][sl] if self.planes else None, self.d[K][sl], self.s[K][sl])

    def entries(self):
        out = []
        for l in range(self.layers):
            for mi, (name, N, K) in enumerate(self.shapes):
                q, pl, d, s = self.act(l, K)
                out.append((self.weights[l][mi], q, pl, d, s, self.y[l][mi]))
        return out

    def quantize_acts(self, ebq):
        """Q8 per 32 of every input width in one launch: 4-bit planes for the 1- and
        2-bit formats (which read nothing else of q), int8 q for the others."""
        ebq.qact_quant_batch([(self.x[K], None if self.planes else self.q[K], self.pl[K] if self.planes else None,
                               self.d[K], self.s[K]) for K in WIDTHS])

    def weight_bytes(self):
        return sum(w.nbytes for row in self.weights for w in row)

    def gemv_bytes(self):
        """Algorithmic bytes of one grouped launch: weights + activation reads
        (q or its planes, same size, + d, qsum per matrix) + fp32 outputs."""
        b = self.weight_bytes()
        for l in range(self.layers):
            for (name, N, K) in self.shapes:
                b += self.B * (K + (K // 32) * 8) + self.B * N * 4
        return b

    def step_bytes(self):
        """Algorithmic bytes of one step: the grouped launch + activation quantization
        (fp32 in; int8 q or its 4-bit planes, same size, + scales + sums out)."""
        b = self.gemv_bytes()
        for K in WIDTHS:
            b += self.layers * self.B * (K * 4 + K + (K // 32) * 8)
        return b

    def n_weights(self):
        return self.layers * sum(N * K for (_, N, K) in self.shapes)


# ---------------------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------------------

def time_region(fn, steps, warmup):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps * 1e-3, wall


def time_kernel(fn, reps, warmup):
    """Average duration of fn's launches from events recorded around each one
    on torch's current stream (the stream the library launches on)."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) * 1e-3 for a, b in evs)
    return sum(ts) / len(ts), ts[len(ts) // 2]


# ---------------------------------------------------------------------------------------
# parity spot checks against the oracle (rows sampled from the large workloads)
# ---------------------------------------------------------------------------------------

def sampled_parity(ebq, stack, layer_ids, rows_per_matrix=16, seed=0):
    import oracle

    rng = np.random.default_rng(seed)
    worst = 0.0
    for l in layer_ids:
        for mi, (name, N, K) in enumerate(stack.shapes):
            fmt = layer_fmt(stack.kind, name)
            rows = np.sort(rng.choice(N, size=min(rows_per_matrix, N), replace=False))
            sigma = 1.0 if stack.kind == "sign1" else 0.02
            w = synth.gauss_torch([seed_of(stack.kind), l, mi], (N, K), sigma)[rows].cpu().numpy()
            codes, sc = oracle.quantize(fmt, w)
            packed = oracle.pack(fmt, codes)
            x = stack.x[K][l * stack.B:(l + 1) * stack.B].cpu().numpy()
            rq, rd, _ = oracle.act_quant(x, 32)
            yr, absT, _ = oracle.gemv(fmt, packed, sc, None, K, rq, rd)
            yg = stack.y[l][mi].cpu().numpy()[:, rows].astype(np.float64)
            err = np.abs(yg - yr)
            ratio = float((err / np.maximum(absT, 1e-300)).max())
            worst = max(worst, ratio)
            if not (err <= 1e-4 * absT).all():
                return False, worst
    return True, worst


# ---------------------------------------------------------------------------------------
# CPU baseline: the oracle on one layer of the headline stack
# ---------------------------------------------------------------------------------------

def cpu_baseline(ebq, stack):
    import torch

    import oracle

    threads = os.cpu_count() or 1
    os.environ.setdefault("OMP_NUM_THREADS", str(threads))
    threads = int(os.environ["OMP_NUM_THREADS"])
    layer = 0
    prep = []
    for mi, (name, N, K) in enumerate(stack.shapes):
        fmt = layer_fmt(stack.kind, name)
        w = synth.gauss_torch([seed_of(stack.kind), layer, mi], (N, K), 1.0 if stack.kind == "sign1" else 0.02)
        w = w.cpu().numpy()
        codes, sc = oracle.quantize(fmt, w)
        del w
        packed = oracle.pack(fmt, codes)
        del codes
        x = stack.x[K][layer * stack.B:(layer + 1) * stack.B].cpu().numpy()
        rq, rd, _ = oracle.act_quant(x, 32)
        prep.append((fmt, packed, sc, K, rq, rd))
    nbytes = sum(p.nbytes + s.nbytes for _, p, s, _, _, _ in prep)
    # the layer's GEMVs, repeated until about 10 s of CPU work have been timed
    reps = 0
    t0 = time.perf_counter()
    while True:
        outs = [oracle.gemv(fmt, p, s, None, K, rq, rd) for fmt, p, s, K, rq, rd in prep]
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0:
            break
    # full-layer parity of the GPU result against the oracle
    ok = True
    for (yr, absT, _), y in zip(outs, stack.y[layer]):
        yg = y.cpu().numpy().astype(np.float64)
        ok &= bool((np.abs(yg - yr) <= 1e-4 * absT).all())
    return {
        "value": round(nbytes * reps / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "layer 0 of the 1-bit stack (7 matrices, %d weights, %d bytes) at batch 1, its 7 GEMVs run %d "
                  "times (OpenMP over rows): %.2f s" % (sum(p.shape[0] * K for _, p, _, K, _, _ in prep), nbytes,
                                                       reps, dt),
        "equiv_tok_s": round(reps / (dt * stack.layers), 6),
        "layer_parity": "ok" if ok else "FAIL",
    }


# ---------------------------------------------------------------------------------------
# secondary workloads
# ---------------------------------------------------------------------------------------

def bench_stack_grouped(ebq, stack, steps, warmup):
    plan = ebq.GroupedPlan(stack.entries(), stack.B)

    def step():
        stack.quantize_acts(ebq)
        plan.run()

    t, _ = time_region(step, steps, warmup)
    tk, tk_med = time_kernel(plan.run, max(steps, 5), 2)
    return plan, t, tk, tk_med


def bench_dependent_chain(ebq, stack, reps):
    """448 single-matrix launches captured in a HIP graph (layers one after another)."""
    import torch

    ents = stack.entries()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        for e in ents:                                  # warm the launch path first
            ebq.qgemv(e[0], e[1], e[2], e[3], e[4], stack.B, e[5])
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for e in ents:
                ebq.qgemv(e[0], e[1], e[2], e[3], e[4], stack.B, e[5])
    torch.cuda.synchronize()
    t, _ = time_region(g.replay, reps, 2)
    return t


def bench_prefill(ebq, reps):
    import torch

    M = 2048
    out = {}
    sb = {K: torch.from_numpy(synth.sign_bits([5, 99, K], K).view(np.int32)).cuda() for K in (5120, 17408)}
    for (Kin, Nout, tag) in ((5120, 17408, "up_5120x17408"), (17408, 5120, "down_17408x5120")):
        x = synth.gauss_torch([5, 0, Kin], (M, Kin))
        # rare outliers: 0.1% of entries x20
        g = torch.Generator(device="cuda")
        g.manual_seed(synth.seed64(5, 1, Kin))
        mask = torch.rand((M, Kin), generator=g, device="cuda") < 0.001
        x[mask] *= 20.0
        xq = torch.empty((M, Kin), dtype=torch.int8, device="cuda")
        dx = torch.empty((M, Kin // 256), dtype=torch.float32, device="cuda")
        sx = torch.empty((M, Kin // 256), dtype=torch.int32, device="cuda")
        rng = synth.rng(5, 2, Kin)
        codes = torch.from_numpy(rng.integers(0, 4, size=(Nout, Kin), dtype=np.int8)).cuda()
        pw = ebq.PackedWeight.empty(TRELLIS, Nout, Kin)
        ebq.qweight_pack(TRELLIS, codes, pw)
        del codes
        ebq.qweight_set_scales(pw, torch.from_numpy(
            synth.uniform_f16([5, 3, Kin], (Nout, Kin // 64), 0.01, 0.03).view(np.int16)).cuda())
        pw.seeds.copy_(torch.from_numpy(synth.u16([5, 4, Kin], Nout).view(np.int16)).cuda())
        wq = torch.empty((Nout, Kin), dtype=torch.int8, device="cuda")
        dw = torch.empty((Nout, Kin // 256), dtype=torch.float32, device="cuda")
        y = torch.empty((M, Nout), dtype=torch.float32, device="cuda")
        t_rot, _ = time_kernel(lambda: ebq.qact_hadamard_quant_i8(x, sb[Kin], 256, xq, dx, sx), reps, 2)
        t_dec, _ = time_kernel(lambda: ebq.qtrellis_decode_i8(pw, 256, wq, dw), reps, 2)
        t_gemm, _ = time_kernel(lambda: ebq.qgemm_i8(xq, dx, wq, dw, 256, y), reps, 2)
        ops = 2.0 * M * Nout * Kin
        out[tag] = {
            "gemm_us": round(t_gemm * 1e6, 2),
            "gemm_tops": round(ops / t_gemm / 1e12, 1),
            "mfma_frac": round(ops / t_gemm / 1e12 / INT8_PEAK_TOPS, 4),
            "rotate_quant_us": round(t_rot * 1e6, 2),
            "rotate_quant_gbs": round((M * Kin * 4 + M * Kin + M * (Kin // 256) * 8) / t_rot / 1e9, 1),
            "trellis_decode_us": round(t_dec * 1e6, 2),
            "trellis_decode_gbs": round((pw.nbytes + Nout * Kin + Nout * (Kin // 256) * 4) / t_dec / 1e9, 1),
            "prefill_tok_s_this_matrix": round(M / (t_rot + t_dec + t_gemm), 1),
        }
        del x, xq, wq, y
    return out


def bench_mixed_b64_gemv(ebq, reps):
    """Mixed stack at 64 tokens through the packed weights: one Q8 launch for all
    64 tokens of every layer, then the grouped GEMV for 8 tokens at a time, 8
    plans over consecutive token slices (weights read 8 times per step)."""
    import torch

    B, sub = 64, 8
    ms = Stack(ebq, "mixed", synth.N_LAYERS, B)
    plans = []
    for j in range(B // sub):
        sl = slice(j * sub, (j + 1) * sub)
        ents = [(w, q[sl] if q is not None else None, pl[sl] if pl is not None else None, d[sl], s_[sl], y[sl])
                for (w, q, pl, d, s_, y) in ms.entries()]
        plans.append(ebq.GroupedPlan(ents, sub))

    def step():
        ms.quantize_acts(ebq)
        for p in plans:
            p.run()

    t, _ = time_region(step, reps, 2)
    ok, worst = sampled_parity(ebq, ms, [0, 63], rows_per_matrix=8)
    out = {
        "step_us": round(t * 1e6, 1),
        "plans": "%d grouped launches of %d tokens" % (B // sub, sub),
        "weight_bytes_read": (B // sub) * ms.weight_bytes(),
        "gbs": round((B // sub) * ms.weight_bytes() / t / 1e9, 1),
        "equiv_tok_s": round(B / t, 1),
        "parity": "ok" if ok else "FAIL",
        "worst_err_over_sum_abs_terms": worst,
    }
    del plans, ms
    torch.cuda.empty_cache()
    return out


def bench_mixed_b64_int8_gemm(ebq, reps, layers=2, seed=0):
    """Mixed stack at 64 tokens: weights unpacked once to int8 levels with fp32
    per-32 factors (qweight_unpack_i8: W = dw * wq exactly), activations Q8 per
    32, and a layer's seven products as int8 matrix-core GEMMs rescaled per 32.
    `layers` distinct layers (more bytes than the last-level cache) are timed
    back to back; the 64-layer figure is that time x 64 / layers (stated)."""
    import torch

    import oracle

    B = 64
    mats = []
    for l in range(layers):
        for mi, (name, N, K) in enumerate(synth.LAYER_SHAPES):
            pw = build_matrix(ebq, "mixed", l, mi, name, N, K)
            wq = torch.empty((N, K), dtype=torch.int8, device="cuda")
            dw = torch.empty((N, K // 32), dtype=torch.float32, device="cuda")
            ebq.qweight_unpack_i8(pw, wq, dw)
            del pw
            mats.append((l, mi, name, N, K, wq, dw, torch.empty((B, N), dtype=torch.float32, device="cuda")))
    x = {K: synth.gauss_torch([seed_of("mixed"), 2000, K, B], (B, K)) for K in WIDTHS}
    xq = {K: torch.empty((B, K), dtype=torch.int8, device="cuda") for K in WIDTHS}
    dx = {K: torch.empty((B, K // 32), dtype=torch.float32, device="cuda") for K in WIDTHS}
    sx = {K: torch.empty((B, K // 32), dtype=torch.int32, device="cuda") for K in WIDTHS}

    def step():
        for K in WIDTHS:
            ebq.qact_quant_i8(x[K], 32, xq[K], dx[K], sx[K])
        for (_, _, _, N, K, wq, dw, y) in mats:
            ebq.qgemm_i8(xq[K], dx[K], wq, dw, 32, y)

    t, _ = time_region(step, reps, 2)
    ops = sum(2.0 * B * N * K for (_, _, _, N, K, _, _, _) in mats)
    int8_bytes = sum(wq.numel() + dw.numel() * 4 for (_, _, _, _, _, wq, dw, _) in mats)
    # parity: sampled rows of every product of layer 0 against the oracle's GEMV
    # from the same float draws (the unpacked product is the same sum)
    rng = np.random.default_rng(seed)
    ok, worst = True, 0.0
    for (l, mi, name, N, K, _, _, y) in mats:
        if l != 0:
            continue
        fmt = layer_fmt("mixed", name)
        rows = np.sort(rng.choice(N, size=8, replace=False))
        w = synth.gauss_torch([seed_of("mixed"), l, mi], (N, K), 0.02)[rows].cpu().numpy()
        codes, sc = oracle.quantize(fmt, w)
        rq, rd, _ = oracle.act_quant(x[K].cpu().numpy(), 32)
        yr, absT, _ = oracle.gemv(fmt, oracle.pack(fmt, codes), sc, None, K, rq, rd)
        err = np.abs(y.cpu().numpy()[:, rows].astype(np.float64) - yr)
        worst = max(worst, float((err / np.maximum(absT, 1e-300)).max()))
        ok = ok and bool((err <= 1e-4 * absT).all())
    per_layer = t / layers
    del mats, x, xq, dx, sx
    return {
        "layers_timed": layers,
        "per_layer_us": round(per_layer * 1e6, 1),
        "step_us_64_layers": round(per_layer * 64 * 1e6, 1),
        "extrapolation": "64 x the per-layer time of %d distinct layers timed back to back" % layers,
        "tops": round(ops / t / 1e12, 1),
        "int8_weight_gbs": round(int8_bytes / t / 1e9, 1),
        "equiv_tok_s": round(B / (per_layer * 64), 1),
        "parity": "ok" if ok else "FAIL",
        "worst_err_over_sum_abs_terms": worst,
    }


def bench_mfma_ceiling(ebq):
    """The dense int8 matrix-core rate this part sustains: MFMA 32x32x32 i8 only,
    two waves per SIMD on every CU, and the shader clock it ran at (the waves'
    cycle counter over the launch's elapsed time)."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 2 * cus, 50000
    clocks = torch.zeros(4 * blocks, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    t, _ = time_kernel(lambda: ebq.qcalib_mfma_i8(blocks, iters, clocks, sink), 5, 1)
    c = clocks.view(blocks, 4).cpu().numpy().astype(np.float64)
    cycles = float(np.mean(c[:, 1] - c[:, 0]))
    ref = float(np.mean(c[:, 3] - c[:, 2]))
    tops = blocks * 4 * iters * 16 * 65536 / t / 1e12
    return {
        "tops": round(tops, 1),
        "frac_of_published": round(tops / INT8_PEAK_TOPS, 4),
        "kernel_us": round(t * 1e6, 1),
        "shader_clock_mhz": round(cycles / t / 1e6, 1),
        "reference_counter_mhz": round(ref / t / 1e6, 2),
        "cycles_per_mfma_per_simd": round(cycles / (2 * iters * 16), 2),
    }


def bench_small_ternary(ebq, reps):
    """1024x1024 ternary GEMV (L2-resident: reported as latency)."""
    import torch

    N = K = 1024
    trits = torch.from_numpy(synth.trits([1], (N, K))).cuda()
    pw = ebq.PackedWeight.empty(TERN, N, K)
    ebq.qweight_pack(TERN, trits, pw)
    ebq.qweight_set_scales(pw, torch.from_numpy(synth.uniform_f16([1, 1], (N, K // 256), 0.01, 0.1).view(np.int16)).cuda())
    x = torch.from_numpy(synth.gauss([1, 2], (1, K))).cuda()
    q = torch.empty((1, K), dtype=torch.int8, device="cuda")
    d = torch.empty((1, K // 32), dtype=torch.float32, device="cuda")
    s = torch.empty((1, K // 32), dtype=torch.int32, device="cuda")
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")

    def step():
        ebq.qact_quant_i8(x, 32, q, d, s)
        ebq.qgemv(pw, q, None, d, s, 1, y)

    t, _ = time_region(step, reps, 10)
    tk, _ = time_kernel(lambda: ebq.qgemv(pw, q, None, d, s, 1, y), reps, 10)
    return {"step_us": round(t * 1e6, 2), "gemv_us": round(tk * 1e6, 2)}


def copy_calibration():
    """One device-to-device copy of exactly 1 GiB: a kernel of known traffic
    (2^30 bytes read, 2^30 written) against which the HBM byte counters of a
    profiling run are scaled."""
    import torch

    a = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def bench_copy_ceiling(reps):
    """Device-to-device copy of 2 GiB: the achievable read+write HBM rate."""
    import torch

    n = 1 << 31
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    t, _ = time_kernel(lambda: b.copy_(a), reps, 2)
    del a, b
    return round(2 * n / t / 1e9, 1)


# ---------------------------------------------------------------------------------------

# ---------------------------------------------------------------------------------------
# measured HBM traffic of the headline kernel (rocprofv3 byte counters)
# ---------------------------------------------------------------------------------------

# Sources whose change invalidates recorded counters.
GEMV_SOURCES = ("extreme_bit_quantized_amd/csrc/gemv_impl.hpp", "extreme_bit_quantized_amd/csrc/gemv_inst.hip",
                "extreme_bit_quantized_amd/csrc/internal.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_grouped_sign1_64layer_stack_b1.traffic.json")
HEADLINE_KERNEL = "k_gemv_grouped<1, 3>"  # batch 1, 1-bit (format code 3)


def gemv_source_hash():
    h = hashlib.sha256()
    for p in GEMV_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per headline launch from the recorded counters, or None when
    none are recorded or the kernel sources changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != gemv_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def _counter_rows(run_dir, counter):
    out = []
    for root, _, files in os.walk(run_dir):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                with open(os.path.join(root, fn)) as f:
                    out += [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
    return out


def record_traffic(fetch_dir, write_dir):
    """Write TRAFFIC_FILE from two rocprofv3 --pmc runs of `bench.py --quick`
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).  Each counter is scaled by
    what it reads for the run's 1 GiB device copy (2^30 bytes read and written)."""
    rec = {"kernel": HEADLINE_KERNEL, "source_sha256": gemv_source_hash()}
    total = 0.0
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d, name)
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        kern = [float(r["Counter_Value"]) for r in rows if HEADLINE_KERNEL in r["Kernel_Name"]]
        if not copies or not kern:
            raise SystemExit("no %s rows for the copy or the headline kernel under %s" % (name, d))
        factor = (1 << 30) / 1024.0 / max(copies)       # the largest copy is the 1 GiB one
        kib = sum(kern) / len(kern)
        rec[name] = {"kib_per_dispatch": kib, "dispatches": len(kern), "copy_kib": max(copies),
                     "scale_factor": round(factor, 4), "bytes_per_launch": kib * 1024.0 * factor}
        total += kib * 1024.0 * factor
    rec["traffic_bytes_per_launch"] = round(total)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--quick", action="store_true", help="headline only (no secondary workloads, no CPU baseline)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the prefill pieces (--steps launches each) and the 1 GiB copy, for counter runs")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="record the headline kernel's HBM bytes from two rocprofv3 --pmc output folders and exit")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    import extreme_bit_quantized_amd as ebq

    ebq.load()
    log = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)
    torch.cuda.init()
    log("device", torch.cuda.get_device_name(0))
    if args.prefill_only:
        pre = bench_prefill(ebq, max(2, args.steps))
        copy_calibration()
        print(json.dumps({"prefill_2048_tokens": pre}), flush=True)
        return

    # ---- headline: 1-bit 64-layer stack, batch 1 ----
    log("building the 1-bit 64-layer stack")
    stack = Stack(ebq, "sign1", synth.N_LAYERS, 1)
    plan, t_step, t_kern, t_kern_med = bench_stack_grouped(ebq, stack, args.steps, args.warmup)
    log("step %.1f us, grouped kernel %.1f us" % (t_step * 1e6, t_kern * 1e6))
    ok, worst = sampled_parity(ebq, stack, [0, 31, 63])
    step_bytes = stack.step_bytes()
    gemv_bytes = stack.gemv_bytes()
    value = step_bytes / t_step / 1e9
    achieved = gemv_bytes / t_kern / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {
            "workload": "1-bit sign GEMV, 64-layer 27B-shaped stack (q 6144x5120, k/v 1024x5120, o 5120x6144, "
                        "gate/up 17408x5120, down 5120x17408; 448 matrices, %d weights), batch 1" % stack.n_weights(),
            "batch": 1,
            "weight_bytes_per_token": stack.weight_bytes(),
            "step_bytes": step_bytes,
        },
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "equiv_tok_s": round(1.0 / t_step, 1),
        "parity": {"sampled_rows": "ok" if ok else "FAIL", "worst_err_over_sum_abs_terms": worst},
        "roofline": {
            "kernel": "qk::k_gemv_grouped<1, QFMT_SIGN1>",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "bytes_per_launch": gemv_bytes,
            "avg_launch_us": round(t_kern * 1e6, 2),
            "median_launch_us": round(t_kern_med * 1e6, 2),
        },
    }
    extra = {}
    if not args.quick:
        try:
            reps = min(30, max(5, args.steps // 2))
            extra["dependent_chain_hipgraph"] = {}
            t_chain = bench_dependent_chain(ebq, stack, reps)
            extra["dependent_chain_hipgraph"] = {
                "gemv_us": round(t_chain * 1e6, 1),
                "gbs": round(gemv_bytes / t_chain / 1e9, 1),
            }
            log("chain done")
        except Exception as e:  # report, do not hide
            extra["dependent_chain_hipgraph"] = {"error": repr(e)}
    if not args.no_cpu and not args.quick:
        log("cpu baseline")
        res["cpu_baseline"] = cpu_baseline(ebq, stack)
    del plan
    del stack
    torch.cuda.empty_cache()

    if not args.quick:
        reps = min(30, max(5, args.steps // 2))
        for B in (1, 8):
            log("mixed stack B=%d" % B)
            ms = Stack(ebq, "mixed", synth.N_LAYERS, B)
            plan, t, tk, _ = bench_stack_grouped(ebq, ms, reps, 2)
            okm, wm = sampled_parity(ebq, ms, [0, 63], rows_per_matrix=8)
            extra["mixed_int4_attn_ternary_ffn_B%d" % B] = {
                "step_us": round(t * 1e6, 1),
                "gemv_us": round(tk * 1e6, 1),
                "gbs": round(ms.step_bytes() / t / 1e9, 1),
                "gemv_gbs": round(ms.gemv_bytes() / tk / 1e9, 1),
                "equiv_tok_s": round(B / t, 1),
                "weight_bytes": ms.weight_bytes(),
                "parity": "ok" if okm else "FAIL",
            }
            del plan, ms
            torch.cuda.empty_cache()
        log("mixed stack B=64")
        extra["mixed_int4_attn_ternary_ffn_B64"] = bench_mixed_b64_gemv(ebq, min(reps, 10))
        extra["mixed_int4_attn_ternary_ffn_B64_int8_gemm"] = bench_mixed_b64_int8_gemm(ebq, min(reps, 10))
        torch.cuda.empty_cache()
        log("2-bit layer x8 copies")
        l2 = Stack(ebq, "int2", 8, 1, shapes=synth.LAYER_SHAPES_FUSED, copies_of=lambda l: l)
        plan, t, tk, _ = bench_stack_grouped(ebq, l2, reps, 2)
        ok2, _ = sampled_parity(ebq, l2, [0], rows_per_matrix=8)
        extra["int2_one_layer_8_copies"] = {
            "step_us_8_layers": round(t * 1e6, 1),
            "gbs": round(l2.step_bytes() / t / 1e9, 1),
            "per_layer_us": round(t / 8 * 1e6, 2),
            "layer_bytes": l2.weight_bytes() // 8,
            "parity": "ok" if ok2 else "FAIL",
        }
        del plan, l2
        torch.cuda.empty_cache()
        log("ternary 1024x1024")
        extra["ternary_1024x1024_latency"] = bench_small_ternary(ebq, 50)
        log("prefill")
        ceiling = bench_mfma_ceiling(ebq)
        extra["mfma_i8_ceiling"] = ceiling
        pre = bench_prefill(ebq, reps)
        for v in pre.values():
            v["mfma_frac_of_measured"] = round(v["gemm_tops"] / ceiling["tops"], 4)
        extra["prefill_2048_tokens"] = pre
        extra["hbm_copy_ceiling_gbs"] = bench_copy_ceiling(5)
        res["extra"] = extra
    elif extra:
        res["extra"] = extra
    if args.quick:
        copy_calibration()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
