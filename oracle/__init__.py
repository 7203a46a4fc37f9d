"""Plain CPU oracle for the extreme low-bit GEMV/GEMM path (numpy front end).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product library never links,
loads or calls it, and this package imports nothing from the product library.

The arithmetic lives in ``qref.c`` (plain C11 loops, fp64 unless a function
states otherwise, built with ``-O2 -ffp-contract=off``); this module only builds
it with gcc and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qref.c")
_LIB = os.path.join(_HERE, "libqref.so")
_lock = threading.Lock()
_lib = None

TERN_B3, INT2, SIGN1, INT4, TRELLIS2 = 1, 2, 3, 4, 5
FORMATS = (TERN_B3, INT2, SIGN1, INT4, TRELLIS2)


def build(force: bool = False) -> str:
    """Compile qref.c into libqref.so next to it; returns the library path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
        os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "qref.h"))
    ):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _L():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            i32, i64, u32, u16, d = ctypes.c_int, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint16, ctypes.c_double
            sig = {
                "qref_threads": (i32, []),
                "qref_set_threads": (None, [i32]),
                "qref_scale_block": (i32, [i32]),
                "qref_packed_row_bytes": (i64, [i32, i32]),
                "qref_row_stride": (i64, [i32, i32]),
                "qref_f64_to_f16": (u16, [d]),
                "qref_f16_to_f64": (d, [u16]),
                "qref_q8_block": (None, [P, i32, P, P, P]),
                "qref_act_quant": (None, [P, i32, i32, i32, P, P, P]),
                "qref_act_planes": (None, [P, i32, i32, P]),
                "qref_quant_tern": (None, [P, i32, i32, P, P]),
                "qref_quant_int2": (None, [P, i32, i32, P, P]),
                "qref_quant_sign1": (None, [P, i32, i32, P, P]),
                "qref_quant_int4": (None, [P, i32, i32, P, P]),
                "qref_pack": (i32, [i32, P, i32, i32, P]),
                "qref_unpack": (i32, [i32, P, i32, i32, P]),
                "qref_trellis_hash": (u32, [u32]),
                "qref_norm_ppf": (d, [d]),
                "qref_codebook_v16": (None, [P]),
                "qref_codebook_v8": (None, [P, P]),
                "qref_trellis_states": (None, [P, P, i32, i32, P]),
                "qref_trellis_decode_f32": (None, [P, P, P, i32, i32, P]),
                "qref_trellis_decode_i8": (None, [P, P, P, i32, i32, i32, P, P]),
                "qref_viterbi": (i32, [i32, P, P, P, i32, P, P]),
                "qref_trellis_rms_scale": (u16, [P]),
                "qref_trellis_encode": (i32, [P, i32, i32, P, P, P, P, P]),
                "qref_kv_row_bytes": (i64, [i32, i32]),
                "qref_kv_quant": (i32, [i32, P, i64, i32, P, P]),
                "qref_kv_dequant": (i32, [i32, P, P, i64, i32, P]),
                "qref_attn_decode": (i32, [i32, P, i32, i32, i32, i32, i64, P, P, P, P, P, P]),
                "qref_gemv": (i32, [i32, P, P, P, i32, i32, P, P, i32, P, P, P]),
                "qref_fwht256": (None, [P]),
                "qref_hadamard_quant": (None, [P, i32, i32, P, i32, P, P, P]),
                "qref_gemm_i8": (None, [P, P, i32, P, P, i32, i32, i32, P, P]),
            }
            for name, (res, args) in sig.items():
                f = getattr(lib, name)
                f.restype = res
                f.argtypes = args
            _lib = lib
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


# -- threads (timing records only) ------------------------------------------------

def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return _L().qref_threads()


def set_threads(n: int) -> None:
    _L().qref_set_threads(int(n))


# -- geometry -----------------------------------------------------------------

def scale_block(fmt: int) -> int:
    return _L().qref_scale_block(fmt)


def packed_row_bytes(fmt: int, K: int) -> int:
    return _L().qref_packed_row_bytes(fmt, K)


def row_stride(fmt: int, K: int) -> int:
    return _L().qref_row_stride(fmt, K)


def f64_to_f16_bits(x: float) -> int:
    return _L().qref_f64_to_f16(float(x))


def f16_bits_to_f64(h: int) -> float:
    return _L().qref_f16_to_f64(int(h))


# -- activation Q8 ------------------------------------------------------------

def act_quant(x, qblock: int = 32):
    """x [B][K] fp32 -> (q int8 [B][K], d fp32 [B][K/qblock], qsum int32 [B][K/qblock])."""
    x = _c(np.atleast_2d(x), np.float32)
    B, K = x.shape
    assert K % qblock == 0
    q = np.empty((B, K), np.int8)
    d = np.empty((B, K // qblock), np.float32)
    s = np.empty((B, K // qblock), np.int32)
    _L().qref_act_quant(_p(x), B, K, qblock, _p(q), _p(d), _p(s))
    return q, d, s


def act_planes(q):
    """q int8 [B][K] -> 4-bit planes uint32 [B][K/32][8] (lo words of the four
    8-value groups, then hi words; value n of a group in nibble n)."""
    q = _c(np.atleast_2d(q), np.int8)
    B, K = q.shape
    assert K % 32 == 0
    out = np.empty((B, K // 32, 8), np.uint32)
    _L().qref_act_planes(_p(q), B, K, _p(out))
    return out


def q8_block(v):
    v = _c(v, np.float32).ravel()
    q = np.empty(v.size, np.int8)
    d = np.empty(1, np.float32)
    s = np.empty(1, np.int32)
    _L().qref_q8_block(_p(v), v.size, _p(q), _p(d), _p(s))
    return q, float(d[0]), int(s[0])


# -- weight quantizers and packing ----------------------------------------------

def quantize(fmt: int, w):
    """w [N][K] fp32 -> (codes int8 [N][K], scales uint16 (fp16 bits) [N][K/block])."""
    w = _c(np.atleast_2d(w), np.float32)
    N, K = w.shape
    blk = scale_block(fmt)
    assert K % blk == 0
    c = np.empty((N, K), np.int8)
    s = np.empty((N, K // blk), np.uint16)
    fn = {TERN_B3: "qref_quant_tern", INT2: "qref_quant_int2", SIGN1: "qref_quant_sign1",
          INT4: "qref_quant_int4"}[fmt]
    getattr(_L(), fn)(_p(w), N, K, _p(c), _p(s))
    return c, s


def pack(fmt: int, codes):
    codes = _c(np.atleast_2d(codes), np.int8)
    N, K = codes.shape
    out = np.empty((N, row_stride(fmt, K)), np.uint8)
    rc = _L().qref_pack(fmt, _p(codes), N, K, _p(out))
    assert rc == 0
    return out


def unpack(fmt: int, packed, K: int):
    packed = _c(np.atleast_2d(packed), np.uint8)
    N = packed.shape[0]
    assert packed.shape[1] == row_stride(fmt, K)
    out = np.empty((N, K), np.int8)
    rc = _L().qref_unpack(fmt, _p(packed), N, K, _p(out))
    assert rc == 0
    return out


# -- trellis ------------------------------------------------------------------------

def trellis_hash(state: int) -> int:
    return _L().qref_trellis_hash(int(state))


def norm_ppf(p: float) -> float:
    return _L().qref_norm_ppf(float(p))


def codebook_v16():
    v = np.empty(256, np.uint16)
    _L().qref_codebook_v16(_p(v))
    return v


def codebook_v8():
    v = np.empty(256, np.int8)
    g = ctypes.c_double()
    _L().qref_codebook_v8(_p(v), ctypes.byref(g))
    return v, g.value


def trellis_states(packed, seeds, K: int):
    packed = _c(np.atleast_2d(packed), np.uint8)
    seeds = _c(seeds, np.uint16)
    N = packed.shape[0]
    st = np.empty((N, K), np.uint16)
    _L().qref_trellis_states(_p(packed), _p(seeds), N, K, _p(st))
    return st


def trellis_decode_f32(packed, seeds, scales, K: int):
    packed = _c(np.atleast_2d(packed), np.uint8)
    seeds = _c(seeds, np.uint16)
    scales = _c(np.atleast_2d(scales), np.uint16)
    N = packed.shape[0]
    w = np.empty((N, K), np.float32)
    _L().qref_trellis_decode_f32(_p(packed), _p(seeds), _p(scales), N, K, _p(w))
    return w


def trellis_decode_i8(packed, seeds, scales, K: int, oblock: int = 256):
    packed = _c(np.atleast_2d(packed), np.uint8)
    seeds = _c(seeds, np.uint16)
    scales = _c(np.atleast_2d(scales), np.uint16)
    N = packed.shape[0]
    wq = np.empty((N, K), np.int8)
    dw = np.empty((N, K // oblock), np.float32)
    _L().qref_trellis_decode_i8(_p(packed), _p(seeds), _p(scales), N, K, oblock, _p(wq), _p(dw))
    return wq, dw


def viterbi(L: int, val, w, sc):
    """Viterbi over an L-bit bit-shift trellis: (state path uint32 [K], fp32 cost)."""
    val = _c(val, np.float32)
    w = _c(w, np.float32)
    sc = _c(sc, np.float32)
    K = w.shape[0]
    assert val.shape[0] == 1 << L and sc.shape[0] == K
    st = np.empty(K, np.uint32)
    cost = ctypes.c_float()
    rc = _L().qref_viterbi(L, _p(val), _p(w), _p(sc), K, _p(st), ctypes.byref(cost))
    assert rc == 0, rc
    return st, np.float32(cost.value)


def trellis_rms_scale(w64) -> int:
    w64 = _c(w64, np.float32)
    assert w64.shape == (64,)
    return int(_L().qref_trellis_rms_scale(_p(w64)))


def trellis_encode(w, scales_in=None):
    """Trellis encoder: w [N][K] fp32 -> (packed, seeds, scales row-major, cost [N] fp32)."""
    w = _c(np.atleast_2d(w), np.float32)
    N, K = w.shape
    packed = np.zeros((N, row_stride(TRELLIS2, K)), np.uint8)
    seeds = np.empty(N, np.uint16)
    scales = np.empty((N, K // 64), np.uint16)
    cost = np.empty(N, np.float32)
    si = None if scales_in is None else _c(np.atleast_2d(scales_in), np.uint16)
    rc = _L().qref_trellis_encode(_p(w), N, K, None if si is None else _p(si), _p(packed), _p(seeds),
                                  _p(scales), _p(cost))
    assert rc == 0, rc
    return packed, seeds, scales, cost


# -- KV cache and decode attention ---------------------------------------------------

KV_Q4, KV_Q8 = 4, 8


def kv_row_bytes(fmt: int, D: int) -> int:
    return int(_L().qref_kv_row_bytes(fmt, D))


def kv_quant(fmt: int, x):
    """x [..., D] fp32 -> (codes uint8 [..., row bytes], scales fp16 bits [..., D/32])."""
    x = _c(x, np.float32)
    D = x.shape[-1]
    rows = int(np.prod(x.shape[:-1]))
    codes = np.empty(x.shape[:-1] + (kv_row_bytes(fmt, D),), np.uint8)
    scales = np.empty(x.shape[:-1] + (D // 32,), np.uint16)
    rc = _L().qref_kv_quant(fmt, _p(x), rows, D, _p(codes), _p(scales))
    assert rc == 0, rc
    return codes, scales


def kv_dequant(fmt: int, codes, scales, D: int):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint16)
    rows = int(np.prod(codes.shape[:-1]))
    x = np.empty(codes.shape[:-1] + (D,), np.float64)
    rc = _L().qref_kv_dequant(fmt, _p(codes), _p(scales), rows, D, _p(x))
    assert rc == 0, rc
    return x


def attn_decode(fmt: int, q, kc, ks, vc, vs, T: int):
    """q [n_kv * G][D] fp32; kc, vc [n_kv][t_cap][row bytes]; ks, vs [n_kv][t_cap][D/32].
    Returns (out fp64 [n_kv * G][D], bound fp64 [n_kv * G][D])."""
    q = _c(q, np.float32)
    kc, vc = _c(kc, np.uint8), _c(vc, np.uint8)
    ks, vs = _c(ks, np.uint16), _c(vs, np.uint16)
    n_kv, t_cap = kc.shape[0], kc.shape[1]
    D = q.shape[1]
    G = q.shape[0] // n_kv
    out = np.empty(q.shape, np.float64)
    bound = np.empty(q.shape, np.float64)
    rc = _L().qref_attn_decode(fmt, _p(q), n_kv, G, D, T, t_cap, _p(kc), _p(ks), _p(vc), _p(vs), _p(out),
                               _p(bound))
    assert rc == 0, rc
    return out, bound


# -- GEMV / rotation / GEMM ---------------------------------------------------------

def gemv(fmt: int, packed, scales, seeds, K: int, q, d, want_I: bool = False):
    """Returns (y fp64 [B][N], absT fp64 [B][N], I int64 [B][N][K/32] or None)."""
    packed = _c(np.atleast_2d(packed), np.uint8)
    scales = _c(np.atleast_2d(scales), np.uint16)
    q = _c(np.atleast_2d(q), np.int8)
    d = _c(np.atleast_2d(d), np.float32)
    N = packed.shape[0]
    B = q.shape[0]
    assert q.shape[1] == K and d.shape == (B, K // 32)
    seeds_a = None if seeds is None else _c(seeds, np.uint16)
    y = np.empty((B, N), np.float64)
    a = np.empty((B, N), np.float64)
    I = np.empty((B, N, K // 32), np.int64) if want_I else None
    rc = _L().qref_gemv(fmt, _p(packed), _p(scales), _p(seeds_a), N, K, _p(q), _p(d), B,
                        _p(I), _p(y), _p(a))
    assert rc == 0
    return y, a, I


def fwht256(u):
    u = _c(u, np.float32).copy()
    assert u.size == 256
    _L().qref_fwht256(_p(u))
    return u


def hadamard_quant(x, sign_bits, qblock: int = 256):
    x = _c(np.atleast_2d(x), np.float32)
    B, K = x.shape
    sign_bits = _c(sign_bits, np.uint32)
    assert sign_bits.size == K // 32
    q = np.empty((B, K), np.int8)
    d = np.empty((B, K // qblock), np.float32)
    s = np.empty((B, K // qblock), np.int32)
    _L().qref_hadamard_quant(_p(x), B, K, _p(sign_bits), qblock, _p(q), _p(d), _p(s))
    return q, d, s


def gemm_i8(xq, dx, wq, dw, kblock: int = 256):
    xq = _c(np.atleast_2d(xq), np.int8)
    wq = _c(np.atleast_2d(wq), np.int8)
    dx = _c(np.atleast_2d(dx), np.float32)
    dw = _c(np.atleast_2d(dw), np.float32)
    M, K = xq.shape
    N = wq.shape[0]
    y = np.empty((M, N), np.float64)
    a = np.empty((M, N), np.float64)
    _L().qref_gemm_i8(_p(xq), _p(dx), M, _p(wq), _p(dw), N, K, kblock, _p(y), _p(a))
    return y, a
