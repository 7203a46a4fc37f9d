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
                HIP-event duration, against 8 TB/s and against the measured
                streaming-read ceiling (a 4 GiB read, qcalib_hbm_read)
  settle_*      after --warmup, headline steps run back to back for --settle
                seconds before timing (the first launches after the stack is
                built run slower while clocks settle); sclk_mhz is the shader
                clock just before and just after the timed region
  cpu_baseline  the CPU oracle timed on one layer of the same stack (OpenMP and
                one thread), plus bounded samples of the other workloads
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
    if kind == "trellis":
        return TRELLIS
    if kind == "int2":
        return INT2
    if kind == "mixed":
        return INT4 if name in synth.ATTN else TERN
    raise ValueError(kind)


def seed_of(kind: str) -> int:
    return {"int2": 2, "sign1": 3, "mixed": 4, "trellis": 5}[kind]


def trellis_draws(layer, mi, N, K):
    """Synthetic trellis-coded matrix, drawn on the device: uniform 2-bit symbols
    (as bytes), uniform 16-bit seeds, fp16 scales U[0.01, 0.03] per 64 (row-major)."""
    return (synth.bytes_torch([5, layer, mi, 1], (N, K // 4)), synth.u16_torch([5, layer, mi, 2], (N,)),
            synth.uniform_f16_torch([5, layer, mi, 3], (N, K // 64), 0.01, 0.03))


def build_matrix(ebq, kind, layer, mi, name, N, K):
    """Quantize N(0, sigma) draws for one matrix on the GPU with the library's
    quantizer.  1-bit draws are N(0,1) (sign + mean|w|), the others N(0,0.02).
    Trellis matrices are random codes, seeds and scales (trellis_draws)."""
    import torch

    fmt = layer_fmt(kind, name)
    if fmt == TRELLIS:
        codes, seeds, sc = trellis_draws(layer, mi, N, K)
        pw = ebq.PackedWeight.empty(fmt, N, K)
        pw.codes.copy_(codes)
        pw.seeds.copy_(seeds)
        ebq.qweight_set_scales(pw, sc)
        del codes, seeds, sc
        return pw
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


def settle(fn, seconds):
    """Run fn back to back for at least `seconds` of wall time (after the
    --warmup steps): the first launches after the stack is built run slower
    while the part's clocks and power settle, so the timed region starts from
    a steady state.  Returns (calls, seconds)."""
    import torch

    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(20):
            fn()
        n += 20
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        if dt >= seconds:
            return n, dt


REFCLK_MHZ = 100.0  # rate of the constant-rate counter s_memrealtime on this part


def sclk_probe(ebq):
    """Shader clock right now: one small matrix-core calibration launch (one
    workgroup, ~1 M cycles), its wave cycle counter over the constant-rate
    counter (s_memtime / s_memrealtime) x 100 MHz."""
    import torch

    clocks = torch.zeros(4, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ebq.qcalib_mfma_i8(1, 2000, clocks, sink)
    c = clocks.cpu().numpy().astype(np.float64)
    return round(float((c[1] - c[0]) / max(c[3] - c[2], 1.0) * REFCLK_MHZ), 1)


# ---------------------------------------------------------------------------------------
# parity spot checks against the oracle (rows sampled from the large workloads)
# ---------------------------------------------------------------------------------------

def sampled_parity(ebq, stack, layer_ids, rows_per_matrix=16, seed=0):
    import torch

    import oracle

    rng = np.random.default_rng(seed)
    worst = 0.0
    for l in layer_ids:
        for mi, (name, N, K) in enumerate(stack.shapes):
            fmt = layer_fmt(stack.kind, name)
            rows = np.sort(rng.choice(N, size=min(rows_per_matrix, N), replace=False))
            seeds = None
            if fmt == TRELLIS:
                # the sampled rows of the same device draws
                ct, st, sct = trellis_draws(l, mi, N, K)
                idx = torch.from_numpy(rows).cuda()
                packed = ct[idx].cpu().numpy()
                seeds = st[idx].cpu().numpy().view(np.uint16)
                sc = sct[idx].cpu().numpy().view(np.uint16)
                del ct, st, sct
            else:
                sigma = 1.0 if stack.kind == "sign1" else 0.02
                w = synth.gauss_torch([seed_of(stack.kind), l, mi], (N, K), sigma)[rows].cpu().numpy()
                codes, sc = oracle.quantize(fmt, w)
                packed = oracle.pack(fmt, codes)
            x = stack.x[K][l * stack.B:(l + 1) * stack.B].cpu().numpy()
            rq, rd, _ = oracle.act_quant(x, 32)
            yr, absT, _ = oracle.gemv(fmt, packed, sc, seeds, K, rq, rd)
            yg = stack.y[l][mi].cpu().numpy()[:, rows].astype(np.float64)
            err = np.abs(yg - yr)
            ratio = float((err / np.maximum(absT, 1e-300)).max())
            worst = max(worst, ratio)
            if not (err <= 1e-4 * absT).all():
                return False, worst
    return True, worst


# ---------------------------------------------------------------------------------------
# CPU baseline: the oracle on bounded samples of every workload
# ---------------------------------------------------------------------------------------

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def _timed(fn, min_s, max_reps=10 ** 6):
    """Run fn until at least min_s seconds have passed; (reps, seconds, last result)."""
    reps, t0, out = 0, time.perf_counter(), None
    while True:
        out = fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_s or reps >= max_reps:
            return reps, dt, out


def _oracle_layer(kind, layer, B, shapes=synth.LAYER_SHAPES, x_seed=2000):
    """Oracle inputs of one layer of a stack: packed weights and Q8 activations."""
    import oracle

    prep = []
    for mi, (name, N, K) in enumerate(shapes):
        fmt = layer_fmt(kind, name)
        w = synth.gauss_torch([seed_of(kind), layer, mi], (N, K), 1.0 if kind == "sign1" else 0.02).cpu().numpy()
        codes, sc = oracle.quantize(fmt, w)
        del w
        packed = oracle.pack(fmt, codes)
        del codes
        rq, rd, _ = oracle.act_quant(synth.gauss([seed_of(kind), x_seed, K, B], (B, K)), 32)
        prep.append((fmt, packed, sc, K, rq, rd))
    return prep


def _run_layer(prep):
    import oracle

    return [oracle.gemv(fmt, p, s, None, K, rq, rd) for fmt, p, s, K, rq, rd in prep]


def cpu_other_configs():
    """The oracle on the other workloads, each a bounded sample (OpenMP threads)."""
    import oracle

    out = {}
    # ternary 1024 x 1024, batch 1: the whole GEMV
    N = K = 1024
    packed = oracle.pack(TERN, synth.trits([1], (N, K)))
    sc = synth.uniform_f16([1, 1], (N, K // 256), 0.01, 0.1)
    rq, rd, _ = oracle.act_quant(synth.gauss([1, 2], (1, K)), 32)
    reps, dt, _ = _timed(lambda: oracle.gemv(TERN, packed, sc, None, K, rq, rd), 0.5)
    out["ternary_1024x1024"] = {"gemv_us": round(dt / reps * 1e6, 1), "sample": "whole GEMV, %d runs" % reps}
    # one 2-bit layer (q/k/v fused), batch 1
    prep = _oracle_layer("int2", 0, 1, synth.LAYER_SHAPES_FUSED)
    nbytes = sum(p.nbytes + s.nbytes for _, p, s, _, _, _ in prep)
    reps, dt, _ = _timed(lambda: _run_layer(prep), 1.0)
    out["int2_one_layer"] = {"gbs": round(nbytes * reps / dt / 1e9, 4), "layer_ms": round(dt / reps * 1e3, 2),
                             "sample": "one whole layer (%d bytes), %d runs" % (nbytes, reps)}
    del prep
    # mixed stack: one layer at 1, 8 and 64 tokens, x64 for the stack
    for B in (1, 8, 64):
        prep = _oracle_layer("mixed", 0, B)
        reps, dt, _ = _timed(lambda: _run_layer(prep), 0.5 if B < 64 else 0.1, max_reps=50)
        per_layer = dt / reps
        out["mixed_B%d" % B] = {"layer_ms": round(per_layer * 1e3, 2), "step_ms_64_layers": round(per_layer * 64e3, 1),
                                "tok_s": round(B / (per_layer * 64), 4),
                                "sample": "layer 0 (7 matrices), %d runs; 64-layer step = 64 x the layer" % reps}
        del prep
    # prefill, 5120 -> 17408: rotation + Q8 and the GEMM on 16 of the 2048 tokens,
    # the trellis decode of the whole matrix
    M, Ms, Kin, Nout = 2048, 16, 5120, 17408
    xs = synth.with_outliers(synth.gauss([5, 7, Kin], (Ms, Kin)), [5, 8, Kin])
    sb = synth.sign_bits([5, 99, Kin], Kin)
    packed = oracle.pack(TRELLIS, synth.rng(5, 2, Kin).integers(0, 4, size=(Nout, Kin), dtype=np.int8))
    sc = synth.uniform_f16([5, 3, Kin], (Nout, Kin // 64), 0.01, 0.03)
    seeds = synth.u16([5, 4, Kin], Nout)
    t0 = time.perf_counter()
    xq, dx, _ = oracle.hadamard_quant(xs, sb, Kin)
    t_rot = time.perf_counter() - t0
    t0 = time.perf_counter()
    wq, dw = oracle.trellis_decode_i8(packed, seeds, sc, Kin, Kin)
    t_dec = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.gemm_i8(xq, dx, wq, dw, Kin)
    t_gemm = time.perf_counter() - t0
    scale = M / Ms
    total = (t_rot + t_gemm) * scale + t_dec
    out["prefill_5120x17408"] = {
        "gemm_gops": round(2.0 * Ms * Nout * Kin / t_gemm / 1e9, 2),
        "rotate_quant_ms_16_tokens": round(t_rot * 1e3, 2),
        "trellis_decode_ms": round(t_dec * 1e3, 1),
        "gemm_ms_16_tokens": round(t_gemm * 1e3, 1),
        "tok_s_this_matrix": round(M / total, 2),
        "sample": "one scale per row: rotation + Q8 and GEMM on %d of %d tokens (x%d stated), decode of the "
                  "whole matrix" % (Ms, M, scale),
    }
    return out


def cpu_baseline(ebq, stack):
    """The oracle on layer 0 of the headline stack (OpenMP over rows, the thread
    count it actually uses, then single-threaded), checked against the GPU's
    layer-0 outputs, plus bounded samples of the other workloads."""
    import oracle

    threads = oracle.threads()
    prep = []
    for mi, (name, N, K) in enumerate(stack.shapes):
        fmt = layer_fmt(stack.kind, name)
        w = synth.gauss_torch([seed_of(stack.kind), 0, mi], (N, K), 1.0 if stack.kind == "sign1" else 0.02)
        w = w.cpu().numpy()
        codes, sc = oracle.quantize(fmt, w)
        del w
        packed = oracle.pack(fmt, codes)
        del codes
        rq, rd, _ = oracle.act_quant(stack.x[K][0:stack.B].cpu().numpy(), 32)
        prep.append((fmt, packed, sc, K, rq, rd))
    nbytes = sum(p.nbytes + s.nbytes for _, p, s, _, _, _ in prep)
    nw = sum(p.shape[0] * K for _, p, _, K, _, _ in prep)
    reps, dt, outs = _timed(lambda: _run_layer(prep), 8.0)
    oracle.set_threads(1)
    reps1, dt1, _ = _timed(lambda: _run_layer(prep), 2.0)
    oracle.set_threads(threads)
    ok = True
    for (yr, absT, _), y in zip(outs, stack.y[0]):
        yg = y.cpu().numpy().astype(np.float64)
        ok &= bool((np.abs(yg - yr) <= 1e-4 * absT).all())
    del prep
    return {
        "value": round(nbytes * reps / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "layer 0 of the 1-bit stack (7 matrices, %d weights, %d bytes) at batch 1, its 7 GEMVs run %d "
                  "times on %d OpenMP threads: %.2f s" % (nw, nbytes, reps, threads, dt),
        "equiv_tok_s": round(reps / (dt * stack.layers), 6),
        "single_thread_gbs": round(nbytes * reps1 / dt1 / 1e9, 4),
        "single_thread_sample": "the same layer, %d runs on 1 thread: %.2f s" % (reps1, dt1),
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "layer_parity": "ok" if ok else "FAIL",
        "other_workloads": cpu_other_configs(),
    }


# ---------------------------------------------------------------------------------------
# secondary workloads
# ---------------------------------------------------------------------------------------

def bench_stack_grouped(ebq, stack, steps, warmup, settle_s=0.0):
    plan = ebq.GroupedPlan(stack.entries(), stack.B)

    def step():
        stack.quantize_acts(ebq)
        plan.run()

    for _ in range(warmup):
        step()
    pre = settle(step, settle_s) if settle_s > 0 else (0, 0.0)
    clk0 = sclk_probe(ebq)
    t, _ = time_region(step, steps, 0)
    clk1 = sclk_probe(ebq)
    tk, tk_med = time_kernel(plan.run, max(steps, 5), 2)
    return plan, t, tk, tk_med, {"settle_steps": pre[0], "settle_s": round(pre[1], 3),
                                 "sclk_mhz_before": clk0, "sclk_mhz_after": clk1}


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
    for l in range(stack.layers):                       # the replays must write these afresh
        for y in stack.y[l]:
            y.fill_(float("nan"))
    t, _ = time_region(g.replay, reps, 2)
    ok, worst = sampled_parity(ebq, stack, [0, stack.layers - 1], rows_per_matrix=8, seed=5)
    return t, ok, worst


def bench_prefill(ebq, reps):
    """The prefill chain per FFN shape at 2048 tokens, in both scale readings: one
    scale per row of each operand (per-token activations after the rotation,
    per-output-row weights: the int8 GEMM's own scaling; the headline GEMM
    figures) and one scale pair per 256-block (the rotation block)."""
    import torch

    import oracle

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
        rng = synth.rng(5, 2, Kin)
        codes_h = rng.integers(0, 4, size=(Nout, Kin), dtype=np.int8)
        scales_h = synth.uniform_f16([5, 3, Kin], (Nout, Kin // 64), 0.01, 0.03)
        seeds_h = synth.u16([5, 4, Kin], Nout)
        pw = ebq.PackedWeight.empty(TRELLIS, Nout, Kin)
        ebq.qweight_pack(TRELLIS, torch.from_numpy(codes_h).cuda(), pw)
        ebq.qweight_set_scales(pw, torch.from_numpy(scales_h.view(np.int16)).cuda())
        pw.seeds.copy_(torch.from_numpy(seeds_h.view(np.int16)).cuda())
        xq = torch.empty((M, Kin), dtype=torch.int8, device="cuda")
        wq = torch.empty((Nout, Kin), dtype=torch.int8, device="cuda")
        y = torch.empty((M, Nout), dtype=torch.float32, device="cuda")
        ops = 2.0 * M * Nout * Kin
        # parity of each chain (rotation + Q8, trellis decode, GEMM) on sampled
        # tokens and output columns: the oracle redoes every step from the same draws
        prng = np.random.default_rng(Kin)
        rows = np.sort(np.concatenate([[0, M - 1], prng.choice(np.arange(1, M - 1), 6, replace=False)]))
        cols = np.sort(np.concatenate([[0, Nout - 1], prng.choice(np.arange(1, Nout - 1), 62, replace=False)]))
        xs = x[torch.from_numpy(rows).cuda()].cpu().numpy()
        rsub = oracle.pack(TRELLIS, codes_h[cols])
        res = {}
        for blk_name, blk in (("per_row", Kin), ("per_256", 256)):
            nb = Kin // blk
            dx = torch.empty((M, nb), dtype=torch.float32, device="cuda")
            sx = torch.empty((M, nb), dtype=torch.int32, device="cuda")
            dw = torch.empty((Nout, nb), dtype=torch.float32, device="cuda")
            t_rot, _ = time_kernel(lambda: ebq.qact_hadamard_quant_i8(x, sb[Kin], blk, xq, dx, sx), reps, 2)
            t_dec, _ = time_kernel(lambda: ebq.qtrellis_decode_i8(pw, blk, wq, dw), reps, 2)
            t_gemm, _ = time_kernel(lambda: ebq.qgemm_i8(xq, dx, wq, dw, blk, y), reps, 2)
            rxq, rdx, _ = oracle.hadamard_quant(xs, sb[Kin].cpu().numpy().view(np.uint32), blk)
            rwq, rdw = oracle.trellis_decode_i8(rsub, seeds_h[cols], scales_h[cols], Kin, blk)
            yr, absT = oracle.gemm_i8(rxq, rdx, rwq, rdw, blk)
            err = np.abs(y.cpu().numpy()[np.ix_(rows, cols)].astype(np.float64) - yr)
            res[blk_name] = {
                "scales": "one per row of each operand (dx [M][1], dw [N][1])" if blk == Kin
                          else "one pair per 256-block (dx [M][K/256], dw [N][K/256])",
                "gemm_kernel": "qk::k_gemm_i8_rs128" if blk == Kin else "qk::k_gemm_i8_p256",
                "gemm_us": round(t_gemm * 1e6, 2),
                "gemm_tops": round(ops / t_gemm / 1e12, 1),
                "mfma_frac": round(ops / t_gemm / 1e12 / INT8_PEAK_TOPS, 4),
                "rotate_quant_us": round(t_rot * 1e6, 2),
                "rotate_quant_gbs": round((M * Kin * 4 + M * Kin + M * nb * 8) / t_rot / 1e9, 1),
                "trellis_decode_us": round(t_dec * 1e6, 2),
                "trellis_decode_gbs": round((pw.nbytes + Nout * Kin + Nout * nb * 4) / t_dec / 1e9, 1),
                "chain_us": round((t_rot + t_dec + t_gemm) * 1e6, 2),
                "parity": "ok" if bool((err <= 1e-4 * absT).all()) else "FAIL",
                "parity_sample": "%d tokens x %d output columns, rotation + Q8, decode and GEMM redone by the oracle"
                                 % (len(rows), len(cols)),
                "worst_err_over_sum_abs_terms": float((err / np.maximum(absT, 1e-300)).max()),
            }
            del dx, sx, dw
        out[tag] = dict(res["per_row"])
        out[tag]["per_256_block"] = res["per_256"]
        del codes_h, x, xq, wq, y
    return out


def bench_trellis_encoder(ebq, reps, N=512, K=5120, per=512, sample=(0, 511)):
    """Trellis encoder (Viterbi over the 2^16-state trellis) on N(0, 0.02) rows of
    the 5120 input width in one pass of 512 rows (two rows per compute unit; the
    backtrack's time per pass does not grow with the rows, so larger passes
    spread it thinner; the workspace holds 20 MB of choices per row).
    Parity: codes, seeds, scales and costs of the sampled rows bit-exact against
    the oracle.  Roofline: VALU issue (the recursion is plain fp32 arithmetic)."""
    import torch

    import oracle

    w_h = synth.gauss([5, 900, N, K], (N, K), 0.02)
    w = torch.from_numpy(w_h).cuda()
    out = ebq.PackedWeight.empty(TRELLIS, N, K)
    ws = torch.empty(ebq.qtrellis_encode_workspace_bytes(N, K, per), dtype=torch.uint8, device="cuda")
    cost = torch.empty(N, dtype=torch.float32, device="cuda")
    t, _ = time_region(lambda: ebq.qtrellis_encode(w, out, ws, per, cost=cost), reps, 1)
    codes, seeds = out.codes.cpu().numpy(), out.seeds.cpu().numpy().view(np.uint16)
    sc = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
    ebq.qweight_get_scales(out, sc)
    sc = sc.cpu().numpy().view(np.uint16)
    cost_h = cost.cpu().numpy()
    rows = list(sample)
    rp, rs, rsc, rc = oracle.trellis_encode(w_h[rows])
    ok = bool((codes[rows] == rp).all() and (seeds[rows] == rs).all() and (sc[rows] == rsc).all()
              and (cost_h[rows].view(np.uint32) == rc.view(np.uint32)).all())
    state_steps = float(N) * K * 65536
    nmse = float(cost_h.astype(np.float64).sum() / (w_h.astype(np.float64) ** 2).sum())
    del w, out, ws, cost
    torch.cuda.empty_cache()
    return {
        "rows": N, "cols": K, "rows_per_pass": per,
        "ms": round(t * 1e3, 3),
        "rows_per_s": round(N / t, 1),
        "weights_per_s": round(N * K / t, 1),
        "state_steps_per_s": round(state_steps / t, 1),
        "nmse": round(nmse, 5),
        "nmse_bounds": "above 0.0625 (Gaussian rate-distortion at 2 bits), below 0.1175 (4-level Lloyd-Max)",
        "parity": "ok" if ok else "FAIL",
        "parity_sample": "rows %s: codes, seeds, scales and cost bit-exact against the oracle" % (rows,),
    }


def bench_decode_attention(ebq, reps, T=65536, n_kv=4, group=6):
    """Decode attention of one token over a 64K-token KV cache in Q8 and in Q4,
    the 27B-shaped grouping (4 KV heads, 6 query heads each, head dim 256):
    the six query heads of a KV head packed into one workgroup (each cached
    byte read once per group) against one query head per workgroup (read six
    times).  Bytes: the cache (codes + fp16 scales of K and V), q, out and the
    per-chunk partial sums written and read back.  Parity against the oracle
    on one KV head's group (within its fp32 allowance)."""
    import torch

    import oracle

    D = 256
    out = {}
    for fmt, name in ((ebq.QKV_Q8, "q8"), (ebq.QKV_Q4, "q4")):
        rb = ebq.qkv_row_bytes(fmt)
        kc = torch.empty((n_kv, T, rb), dtype=torch.uint8, device="cuda")
        vc = torch.empty_like(kc)
        ks = torch.empty((n_kv, T, D // 32), dtype=torch.int16, device="cuda")
        vs = torch.empty_like(ks)
        for i, (c, s_) in enumerate(((kc, ks), (vc, vs))):
            x = synth.gauss_torch([7, 100 + i, fmt], (n_kv, T, D))
            ebq.qkv_quant(fmt, x, c, s_)
            del x
        q = synth.gauss_torch([7, 200], (n_kv * group, D))
        o = torch.empty_like(q)
        ws = torch.empty(ebq.qattn_decode_workspace_bytes(n_kv, group, T), dtype=torch.uint8, device="cuda")
        cache = 2 * n_kv * T * (rb + D // 32 * 2)
        part = ebq.qattn_decode_workspace_bytes(n_kv, group, T)
        alg = cache + 2 * q.numel() * 4 + 2 * part
        res = {}
        for hpb, tag in ((group, "packed"), (1, "one_head_per_block")):
            t, _ = time_region(lambda: ebq.qattn_decode(fmt, q, kc, ks, vc, vs, T, o, ws, heads_per_block=hpb),
                               reps, 3)
            res[tag] = {"us": round(t * 1e6, 2), "gbs": round(alg / t / 1e9, 1),
                        "frac_of_8tbs": round(alg / t / 8e12, 4)}
        h = 1
        want, bound = oracle.attn_decode(fmt, q[h * group:(h + 1) * group].cpu().numpy(), kc[h:h + 1].cpu().numpy(),
                                         ks[h:h + 1].cpu().numpy().view(np.uint16), vc[h:h + 1].cpu().numpy(),
                                         vs[h:h + 1].cpu().numpy().view(np.uint16), T)
        ebq.qattn_decode(fmt, q, kc, ks, vc, vs, T, o, ws)
        got = o[h * group:(h + 1) * group].cpu().numpy().astype(np.float64)
        ok = bool((np.abs(got - want) <= bound).all())
        res.update({"cache_bytes": cache, "algorithmic_bytes": alg,
                    "packing_speedup": round(res["one_head_per_block"]["us"] / res["packed"]["us"], 3),
                    "parity": "ok" if ok else "FAIL",
                    "parity_sample": "KV head 1's six query rows against the oracle, within its fp32 allowance"})
        out[name] = res
        del kc, vc, ks, vs, q, o, ws
        torch.cuda.empty_cache()
    return out


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
        "shader_clock_mhz": round(cycles / ref * REFCLK_MHZ, 1),
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
    import oracle

    xh = x.cpu().numpy()
    rq, rd, _ = oracle.act_quant(xh, 32)
    sc = synth.uniform_f16([1, 1], (N, K // 256), 0.01, 0.1)
    yr, absT, _ = oracle.gemv(TERN, oracle.pack(TERN, trits.cpu().numpy()), sc, None, K, rq, rd)
    ok = bool((np.abs(y.cpu().numpy().astype(np.float64) - yr) <= 1e-4 * absT).all())
    return {"step_us": round(t * 1e6, 2), "gemv_us": round(tk * 1e6, 2), "parity": "ok" if ok else "FAIL",
            "parity_sample": "all 1024 outputs against the oracle"}


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


def bench_hbm_read_ceiling(ebq, reps=5, nbytes=1 << 32):
    """Streaming read of 4 GiB (qcalib_hbm_read): the achievable HBM read rate,
    the ceiling for the weight-streaming GEMV (which reads and barely writes)."""
    import torch

    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    t, t_med = time_kernel(lambda: ebq.qcalib_hbm_read(a, sink), reps, 2)
    del a
    torch.cuda.empty_cache()
    return {"gbs": round(nbytes / t / 1e9, 1), "bytes": nbytes, "avg_us": round(t * 1e6, 1),
            "frac_of_8tbs": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}


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
    ap.add_argument("--settle", type=float, default=1.5,
                    help="seconds of headline steps run after --warmup and before timing (clocks settle)")
    ap.add_argument("--quick", action="store_true", help="headline only (no secondary workloads, no CPU baseline)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    ap.add_argument("--mixed-only", action="store_true",
                    help="only the mixed 4-bit/ternary stack at batch 1 (--steps launches), for counter runs")
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
    if args.mixed_only:
        ms = Stack(ebq, "mixed", synth.N_LAYERS, 1)
        plan, t, tk, _, cond = bench_stack_grouped(ebq, ms, max(2, args.steps), args.warmup, args.settle)
        okm, wm = sampled_parity(ebq, ms, [0, 63], rows_per_matrix=8)
        print(json.dumps({"mixed_int4_attn_ternary_ffn_B1": {
            "step_us": round(t * 1e6, 1), "gemv_us": round(tk * 1e6, 1),
            "gemv_weight_gbs": round(ms.weight_bytes() / tk / 1e9, 1), "sclk_mhz": cond.get("sclk_mhz_after"),
            "parity": "ok" if okm else "FAIL"}}), flush=True)
        return
    if args.prefill_only:
        pre = bench_prefill(ebq, max(2, args.steps))
        copy_calibration()
        print(json.dumps({"prefill_2048_tokens": pre}), flush=True)
        return

    # ---- headline: 1-bit 64-layer stack, batch 1 ----
    log("building the 1-bit 64-layer stack")
    stack = Stack(ebq, "sign1", synth.N_LAYERS, 1)
    plan, t_step, t_kern, t_kern_med, cond = bench_stack_grouped(ebq, stack, args.steps, args.warmup, args.settle)
    log("step %.1f us, grouped kernel %.1f us, %s" % (t_step * 1e6, t_kern * 1e6, cond))
    ok, worst = sampled_parity(ebq, stack, [0, 31, 63])
    ceiling = bench_hbm_read_ceiling(ebq)
    log("streaming-read ceiling %.1f GB/s" % ceiling["gbs"])
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
        "pct_of_read_ceiling": round(100 * value / ceiling["gbs"], 2),
        "hbm_read_ceiling": ceiling,
        "equiv_tok_s": round(1.0 / t_step, 1),
        "settle_steps": cond["settle_steps"],
        "settle_s": cond["settle_s"],
        "sclk_mhz": {"before_timed": cond["sclk_mhz_before"], "after_timed": cond["sclk_mhz_after"]},
        "parity": {"sampled_rows": "ok" if ok else "FAIL", "worst_err_over_sum_abs_terms": worst},
        "roofline": {
            "kernel": "qk::k_gemv_grouped<1, QFMT_SIGN1>",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "frac_of_read_ceiling": round(achieved / ceiling["gbs"], 4),
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
            t_chain, okc, wc = bench_dependent_chain(ebq, stack, reps)
            extra["dependent_chain_hipgraph"] = {
                "gemv_us": round(t_chain * 1e6, 1),
                "gbs": round(gemv_bytes / t_chain / 1e9, 1),
                "parity": "ok" if okc else "FAIL",
                "worst_err_over_sum_abs_terms": wc,
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
        t_b1 = None
        for B in (1, 8, 16, 64):
            # one grouped plan over all 448 matrices whatever B is: up to 6 tokens
            # the dot4 kernels, from 7 the matrix cores; the weights are read once
            log("mixed stack B=%d" % B)
            ms = Stack(ebq, "mixed", synth.N_LAYERS, B)
            plan, t, tk, _, cond = bench_stack_grouped(ebq, ms, reps, 2, 0.3)
            okm, wm = sampled_parity(ebq, ms, [0, 63], rows_per_matrix=8)
            t_b1 = t if B == 1 else t_b1
            extra["mixed_int4_attn_ternary_ffn_B%d" % B] = {
                "step_us": round(t * 1e6, 1),
                "gemv_us": round(tk * 1e6, 1),
                "per_token_us": round(t * 1e6 / B, 1),
                "step_cost_vs_B1": round(t / t_b1, 3),
                "kernels": ("4-bit: dot4, lane per row; ternary: sparse int8 matrix cores, telescoped digits"
                            if B == 1 else "dot4, lane per row") if B <= 6
                           else "int8 matrix cores, %d group(s) of 16 tokens" % ((B + 15) // 16),
                "gbs": round(ms.step_bytes() / t / 1e9, 1),
                "gemv_weight_gbs": round(ms.weight_bytes() / tk / 1e9, 1),
                "equiv_tok_s": round(B / t, 1),
                "weight_bytes": ms.weight_bytes(),
                "sclk_mhz": cond.get("sclk_mhz_after"),
                "parity": "ok" if okm else "FAIL",
                "parity_sample": "8 rows of every matrix of layers 0 and 63, all tokens",
                "worst_err_over_sum_abs_terms": wm,
            }
            del plan, ms
            torch.cuda.empty_cache()
        log("2-bit layer x8 copies")
        l2 = Stack(ebq, "int2", 8, 1, shapes=synth.LAYER_SHAPES_FUSED, copies_of=lambda l: l)
        plan, t, tk, _, _ = bench_stack_grouped(ebq, l2, reps, 2, 0.3)
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
        log("trellis 64-layer stack B=1")
        ts = Stack(ebq, "trellis", synth.N_LAYERS, 1)
        plan, t, tk, _, cond = bench_stack_grouped(ebq, ts, reps, 2, 0.3)
        okt, wt = sampled_parity(ebq, ts, [0, 63], rows_per_matrix=8)
        extra["trellis2_64layer_stack_B1"] = {
            "step_us": round(t * 1e6, 1),
            "gemv_us": round(tk * 1e6, 1),
            "gbs": round(ts.step_bytes() / t / 1e9, 1),
            "gemv_gbs": round(ts.gemv_bytes() / tk / 1e9, 1),
            "frac_of_8tbs": round(ts.gemv_bytes() / tk / 8e12, 4),
            "equiv_tok_s": round(1 / t, 1),
            "weight_bytes": ts.weight_bytes(),
            "sclk_mhz": cond.get("sclk_mhz_after"),
            "parity": "ok" if okt else "FAIL",
            "parity_sample": "8 rows of every matrix of layers 0 and 63",
            "worst_err_over_sum_abs_terms": wt,
        }
        del plan, ts
        torch.cuda.empty_cache()
        log("trellis encoder")
        extra["trellis_encoder_512x5120"] = bench_trellis_encoder(ebq, 3)
        log("decode attention 64K")
        extra["decode_attention_64k_gqa6"] = bench_decode_attention(ebq, 20)
        log("ternary 1024x1024")
        extra["ternary_1024x1024_latency"] = bench_small_ternary(ebq, 50)
        log("prefill")
        # prefill before the matrix-core calibration: that one runs 130 ms at the
        # part's full matrix power, and the GEMMs timed right after it ran
        # 10-15 % slower (clocks still held down)
        pre = bench_prefill(ebq, reps)
        ceiling = bench_mfma_ceiling(ebq)
        extra["mfma_i8_ceiling"] = ceiling
        for v in pre.values():
            v["mfma_frac_of_measured"] = round(v["gemm_tops"] / ceiling["tops"], 4)
        extra["prefill_2048_tokens"] = pre
        res["extra"] = extra
    elif extra:
        res["extra"] = extra
    if args.quick:
        copy_calibration()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
