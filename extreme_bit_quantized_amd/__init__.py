"""Python binding of libqgemv: extreme low-bit GEMV/GEMM on AMD MI355X (gfx950).

Argument marshalling only.  Every function here has the name of the C entry
point it calls (include/qgemv.h); tensors are passed as device pointers, the
stream defaults to torch's current stream, and a negative return code raises
QError.  All computation happens in the HIP kernels of libqgemv.so; if the
library has not been built this module refuses to load rather than fall back to
anything else.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqgemv.so")

QFMT_TERN_B3, QFMT_INT2, QFMT_SIGN1, QFMT_INT4, QFMT_TRELLIS2 = 1, 2, 3, 4, 5
FORMAT_NAMES = {QFMT_TERN_B3: "tern_b3", QFMT_INT2: "int2", QFMT_SIGN1: "sign1", QFMT_INT4: "int4",
                QFMT_TRELLIS2: "trellis2"}
QERR = {0: "QERR_OK", -1: "QERR_INVALID_ARG", -2: "QERR_UNSUPPORTED_FMT", -3: "QERR_SHAPE",
        -4: "QERR_ALIGNMENT", -5: "QERR_HIP", -6: "QERR_BUFFER", -7: "QERR_TOO_LARGE"}
QGEMV_STATIC_PLAN_BYTES = 1 << 20


class QError(RuntimeError):
    def __init__(self, code: int, func: str):
        self.code = code
        msg = _lib.qstrerror(code).decode() if _lib is not None else "?"
        if code == -5 and _lib is not None:
            msg += ": " + _lib.qhip_error_name().decode()
        super().__init__("%s failed: %s (%s)" % (func, QERR.get(code, code), msg))


class qweight_t(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("block", ctypes.c_int32), ("codes", ctypes.c_void_p), ("row_bytes", ctypes.c_int64),
                ("scales", ctypes.c_void_p), ("seeds", ctypes.c_void_p)]


class qgemv_item_t(ctypes.Structure):
    _fields_ = [("w", qweight_t), ("q", ctypes.c_void_p), ("planes", ctypes.c_void_p), ("d", ctypes.c_void_p),
                ("qsum", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class qact_job_t(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("B", ctypes.c_int32), ("K", ctypes.c_int32), ("q", ctypes.c_void_p),
                ("planes", ctypes.c_void_p), ("d", ctypes.c_void_p), ("qsum", ctypes.c_void_p)]


QACT_BATCH_MAX = 16

_lib = None


def load(path: str = LIB_PATH):
    """Load libqgemv.so (raises if it is missing: there is no other backend)."""
    global _lib
    if _lib is not None:
        return _lib
    # torch first: it carries its own copy of the HIP runtime under the same
    # soname as the system one the library links against.  Loaded in this order
    # the library binds to torch's copy and both share one runtime; loaded the
    # other way round, the library's launches failed with hipErrorNoDevice.
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise ImportError("libqgemv.so is not built at %s; run `python -m extreme_bit_quantized_amd.build`" % path)
    lib = ctypes.CDLL(path)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    W = ctypes.POINTER(qweight_t)
    sig = {
        "qstrerror": (ctypes.c_char_p, [ctypes.c_int]),
        "qhip_error_name": (ctypes.c_char_p, []),
        "qfmt_scale_block": (i32, [i32]),
        "qfmt_packed_row_bytes": (i64, [i32, i32]),
        "qfmt_row_bytes": (i64, [i32, i32]),
        "qweight_check": (ctypes.c_int, [W]),
        "qfmt_scale_group": (i32, [i32]),
        "qfmt_scales_bytes": (i64, [i32, i32, i32]),
        "qweight_set_scales": (ctypes.c_int, [W, P, P]),
        "qweight_get_scales": (ctypes.c_int, [W, P, P]),
        "qweight_quantize": (ctypes.c_int, [i32, P, i32, i32, P, i64, P, P]),
        "qweight_pack": (ctypes.c_int, [i32, P, i32, i32, P, i64, P]),
        "qact_quant_i8": (ctypes.c_int, [P, i32, i32, i32, P, P, P, P]),
        "qact_hadamard_quant_i8": (ctypes.c_int, [P, i32, i32, P, i32, P, P, P, P]),
        "qact_planes": (ctypes.c_int, [P, i32, i32, P, P]),
        "qact_quant_batch": (ctypes.c_int, [ctypes.POINTER(qact_job_t), i32, P]),
        "qgemv": (ctypes.c_int, [W, P, P, P, P, i32, P, P]),
        "qgemv_blockdots": (ctypes.c_int, [W, P, P, P, P, P]),
        "qgemv_grouped_plan_bytes": (i64, [ctypes.POINTER(qgemv_item_t), i32, i32]),
        "qgemv_grouped_plan": (ctypes.c_int, [ctypes.POINTER(qgemv_item_t), i32, i32, P, i64]),
        "qgemv_grouped_run": (ctypes.c_int, [P, P, P]),
        "qgemv_grouped_run_static": (ctypes.c_int, [P, P]),
        "qtrellis_decode_i8": (ctypes.c_int, [W, i32, P, P, P]),
        "qtrellis_encode_workspace_bytes": (i64, [i32, i32, i32]),
        "qkv_row_bytes": (i64, [i32]),
        "qkv_quant": (ctypes.c_int, [i32, P, i64, P, P, P]),
        "qattn_decode_workspace_bytes": (i64, [i32, i32, i32]),
        "qattn_decode": (ctypes.c_int, [i32, P, i32, i32, i32, i32, i64, P, P, P, P, P, P, i64, P]),
        "qtrellis_encode": (ctypes.c_int, [P, i32, i32, P, P, i64, P, P, P, i32, P, i64, P]),
        "qweight_unpack_i8": (ctypes.c_int, [W, P, P, P]),
        "qgemm_i8": (ctypes.c_int, [P, P, i32, P, P, i32, i32, i32, P, P]),
        "qcalib_mfma_i8": (ctypes.c_int, [i32, i32, P, P, P]),
        "qcalib_hbm_read": (ctypes.c_int, [P, i64, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, func: str):
    if rc < 0:
        raise QError(rc, func)
    return rc


# ---- geometry (host) ------------------------------------------------------------------------

def qfmt_scale_block(fmt: int) -> int:
    return load().qfmt_scale_block(fmt)


def qfmt_packed_row_bytes(fmt: int, cols: int) -> int:
    return _check(load().qfmt_packed_row_bytes(fmt, cols), "qfmt_packed_row_bytes")


def qfmt_row_bytes(fmt: int, cols: int) -> int:
    return _check(load().qfmt_row_bytes(fmt, cols), "qfmt_row_bytes")


class PackedWeight:
    """Device tensors of one packed matrix plus its C descriptor."""

    def __init__(self, fmt: int, rows: int, cols: int, codes, scales, seeds=None, row_bytes: int | None = None):
        self.fmt, self.rows, self.cols = fmt, rows, cols
        self.codes, self.scales, self.seeds = codes, scales, seeds
        self.row_bytes = row_bytes if row_bytes is not None else qfmt_row_bytes(fmt, cols)
        self.desc = qweight_t(fmt, rows, cols, qfmt_scale_block(fmt), _ptr(codes), self.row_bytes,
                              _ptr(scales), _ptr(seeds))

    @classmethod
    def empty(cls, fmt: int, rows: int, cols: int, device="cuda"):
        import torch

        rb = qfmt_row_bytes(fmt, cols)
        codes = torch.empty((rows, rb), dtype=torch.uint8, device=device)
        scales = torch.zeros((qfmt_scales_bytes(fmt, rows, cols) // 2,), dtype=torch.int16, device=device)
        seeds = torch.empty((rows,), dtype=torch.int16, device=device) if fmt == QFMT_TRELLIS2 else None
        return cls(fmt, rows, cols, codes, scales, seeds, rb)

    @property
    def nbytes(self) -> int:
        """Algorithmic bytes: codes, one fp16 per scale block, seeds (no padding)."""
        n = self.rows * self.row_bytes + self.rows * (self.cols // qfmt_scale_block(self.fmt)) * 2
        return n + (2 * self.rows if self.seeds is not None else 0)


# ---- device calls ---------------------------------------------------------------------------------

def qweight_check(w: PackedWeight) -> int:
    return load().qweight_check(ctypes.byref(w.desc))


def qweight_quantize(fmt: int, w, out: PackedWeight, stream=None):
    rows, cols = w.shape
    _check(load().qweight_quantize(fmt, _ptr(w), rows, cols, _ptr(out.codes), out.row_bytes, _ptr(out.scales),
                                   _stream(stream)), "qweight_quantize")
    return out


def qfmt_scale_group(fmt: int) -> int:
    return load().qfmt_scale_group(fmt)


def qfmt_scales_bytes(fmt: int, rows: int, cols: int) -> int:
    n = load().qfmt_scales_bytes(fmt, rows, cols)
    _check(n if n < 0 else 0, "qfmt_scales_bytes")
    return n


def qweight_set_scales(w: PackedWeight, rowmajor, stream=None):
    """rowmajor: device fp16 bits [rows][cols/block] (int16 or uint16 tensor)."""
    _check(load().qweight_set_scales(ctypes.byref(w.desc), _ptr(rowmajor), _stream(stream)), "qweight_set_scales")
    return w


def qweight_get_scales(w: PackedWeight, rowmajor, stream=None):
    _check(load().qweight_get_scales(ctypes.byref(w.desc), _ptr(rowmajor), _stream(stream)), "qweight_get_scales")
    return rowmajor


def qweight_pack(fmt: int, levels, out: PackedWeight, stream=None):
    rows, cols = levels.shape
    _check(load().qweight_pack(fmt, _ptr(levels), rows, cols, _ptr(out.codes), out.row_bytes, _stream(stream)),
           "qweight_pack")
    return out


def qact_quant_i8(x, qblock, q, d, qsum, stream=None):
    B, K = x.shape
    _check(load().qact_quant_i8(_ptr(x), B, K, qblock, _ptr(q), _ptr(d), _ptr(qsum), _stream(stream)),
           "qact_quant_i8")


def qact_hadamard_quant_i8(x, sign_bits, qblock, q, d, qsum, stream=None):
    B, K = x.shape
    _check(load().qact_hadamard_quant_i8(_ptr(x), B, K, _ptr(sign_bits), qblock, _ptr(q), _ptr(d), _ptr(qsum),
                                         _stream(stream)), "qact_hadamard_quant_i8")


def qact_planes(q, planes, stream=None):
    B, K = q.shape
    _check(load().qact_planes(_ptr(q), B, K, _ptr(planes), _stream(stream)), "qact_planes")


def qact_quant_batch(jobs, stream=None):
    """jobs: (x [B][K] fp32, q or None, planes or None, d, qsum) per input; one launch."""
    arr = (qact_job_t * max(1, len(jobs)))()
    for i, (x, q, planes, d, qsum) in enumerate(jobs):
        B, K = x.shape
        arr[i] = qact_job_t(_ptr(x), B, K, _ptr(q), _ptr(planes), _ptr(d), _ptr(qsum))
    _check(load().qact_quant_batch(arr, len(jobs), _stream(stream)), "qact_quant_batch")


def qgemv(w: PackedWeight, q, planes, d, qsum, B: int, y, stream=None):
    _check(load().qgemv(ctypes.byref(w.desc), _ptr(q), _ptr(planes), _ptr(d), _ptr(qsum), B, _ptr(y),
                        _stream(stream)), "qgemv")


def qgemv_blockdots(w: PackedWeight, q, planes, qsum, out, stream=None):
    _check(load().qgemv_blockdots(ctypes.byref(w.desc), _ptr(q), _ptr(planes), _ptr(qsum), _ptr(out),
                                  _stream(stream)), "qgemv_blockdots")


def make_items(entries):
    """entries: iterable of (PackedWeight, q, planes, d, qsum, y) -> ctypes array of qgemv_item_t."""
    entries = list(entries)
    arr = (qgemv_item_t * len(entries))()
    for i, (w, q, pl, d, qs, y) in enumerate(entries):
        arr[i] = qgemv_item_t(w.desc, _ptr(q), _ptr(pl), _ptr(d), _ptr(qs), _ptr(y))
    return arr


def qgemv_grouped_plan_bytes(items, B: int) -> int:
    return _check(load().qgemv_grouped_plan_bytes(items, len(items), B), "qgemv_grouped_plan_bytes")


def qgemv_grouped_plan(items, B: int, host_plan) -> None:
    """host_plan: a 16-byte aligned host buffer (e.g. a CPU torch uint8 tensor)."""
    _check(load().qgemv_grouped_plan(items, len(items), B, _ptr(host_plan), host_plan.numel()),
           "qgemv_grouped_plan")


def qgemv_grouped_run(host_plan, dev_plan, stream=None):
    _check(load().qgemv_grouped_run(_ptr(host_plan), _ptr(dev_plan), _stream(stream)), "qgemv_grouped_run")


def qgemv_grouped_run_static(host_plan, stream=None):
    """Run a host plan from the library's static device plan storage (no allocation)."""
    _check(load().qgemv_grouped_run_static(_ptr(host_plan), _stream(stream)), "qgemv_grouped_run_static")


class GroupedPlan:
    """A plan built on the host and copied to the device.

    The plan stores the device addresses of every entry's tensors; the plan
    object keeps those tensors (and the PackedWeights) referenced for as long as
    it lives, so none of them can be freed and reused while the plan may run."""

    def __init__(self, entries, B: int, device="cuda"):
        import torch

        self._entries = [tuple(e) for e in entries]
        self.items = make_items(self._entries)
        self.B = B
        nb = qgemv_grouped_plan_bytes(self.items, B)
        # 16-byte aligned host buffer
        raw = torch.empty(nb + 16, dtype=torch.uint8)
        off = (-raw.data_ptr()) % 16
        self.host = raw[off:off + nb]
        self._raw = raw
        qgemv_grouped_plan(self.items, B, self.host)
        self.dev = self.host.to(device)

    def run(self, stream=None):
        qgemv_grouped_run(self.host, self.dev, stream)

    def run_static(self, stream=None):
        """The same launch from the library's static plan storage (allocates nothing)."""
        qgemv_grouped_run_static(self.host, stream)


def qtrellis_decode_i8(w: PackedWeight, oblock: int, wq, dw, stream=None):
    _check(load().qtrellis_decode_i8(ctypes.byref(w.desc), oblock, _ptr(wq), _ptr(dw), _stream(stream)),
           "qtrellis_decode_i8")


def qtrellis_encode_workspace_bytes(rows: int, cols: int, rows_per_pass: int) -> int:
    n = load().qtrellis_encode_workspace_bytes(rows, cols, rows_per_pass)
    _check(n if n < 0 else 0, "qtrellis_encode_workspace_bytes")
    return n


def qtrellis_encode(w, out: PackedWeight, workspace, rows_per_pass: int, scales_in=None, cost=None, stream=None):
    """w: fp32 [rows][cols] (device); out: an empty TRELLIS2 PackedWeight of the same
    shape; workspace: a device tensor of at least qtrellis_encode_workspace_bytes."""
    rows, cols = w.shape
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().qtrellis_encode(_ptr(w), rows, cols, _ptr(scales_in), _ptr(out.codes), out.row_bytes,
                                  _ptr(out.seeds), _ptr(out.scales), _ptr(cost), rows_per_pass, _ptr(workspace),
                                  ws_bytes, _stream(stream)), "qtrellis_encode")
    return out


QKV_Q4, QKV_Q8, QATTN_HEAD_DIM = 4, 8, 256


def qkv_row_bytes(fmt: int) -> int:
    n = load().qkv_row_bytes(fmt)
    _check(n if n < 0 else 0, "qkv_row_bytes")
    return n


def qkv_quant(fmt: int, x, codes, scales, stream=None):
    """x: fp32 [..., 256] (device) -> codes uint8 [..., row bytes], scales int16 [..., 8]."""
    rows = x.numel() // QATTN_HEAD_DIM
    _check(load().qkv_quant(fmt, _ptr(x), rows, _ptr(codes), _ptr(scales), _stream(stream)), "qkv_quant")


def qattn_decode_workspace_bytes(n_kv: int, group: int, T: int) -> int:
    n = load().qattn_decode_workspace_bytes(n_kv, group, T)
    _check(n if n < 0 else 0, "qattn_decode_workspace_bytes")
    return n


def qattn_decode(fmt: int, q, kcodes, kscales, vcodes, vscales, T: int, out, workspace, heads_per_block=None,
                 stream=None):
    """q [n_kv * group][256] fp32; caches [n_kv][t_cap][...] (device tensors)."""
    n_kv, t_cap = kcodes.shape[0], kcodes.shape[1]
    group = q.shape[0] // n_kv
    hpb = group if heads_per_block is None else heads_per_block
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().qattn_decode(fmt, _ptr(q), n_kv, group, hpb, T, t_cap, _ptr(kcodes), _ptr(kscales), _ptr(vcodes),
                               _ptr(vscales), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)), "qattn_decode")
    return out


def qweight_unpack_i8(w: PackedWeight, wq, dw, stream=None):
    _check(load().qweight_unpack_i8(ctypes.byref(w.desc), _ptr(wq), _ptr(dw), _stream(stream)),
           "qweight_unpack_i8")


def qgemm_i8(xq, dx, wq, dw, kblock: int, y, stream=None):
    M, K = xq.shape
    N = wq.shape[0]
    _check(load().qgemm_i8(_ptr(xq), _ptr(dx), M, _ptr(wq), _ptr(dw), N, K, kblock, _ptr(y), _stream(stream)),
           "qgemm_i8")


def qcalib_mfma_i8(blocks: int, iters: int, clocks, sink, stream=None):
    """clocks: int64 tensor of 4 * blocks entries, sink: int32 tensor (both on the device)."""
    _check(load().qcalib_mfma_i8(blocks, iters, _ptr(clocks), _ptr(sink), _stream(stream)), "qcalib_mfma_i8")


def qcalib_hbm_read(buf, sink, nbytes: int | None = None, stream=None):
    """buf: any device tensor (its first nbytes bytes are read, all by default),
    sink: an int32 device tensor."""
    n = buf.numel() * buf.element_size() if nbytes is None else nbytes
    _check(load().qcalib_hbm_read(_ptr(buf), n, _ptr(sink), _stream(stream)), "qcalib_hbm_read")
