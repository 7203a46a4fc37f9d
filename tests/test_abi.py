"""Host-only checks of the C ABI: the library loads, exports what the header
declares, and rejects bad arguments before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemv.h")


@pytest.fixture(scope="module")
def ebq():
    import extreme_bit_quantized_amd as ebq

    if not os.path.exists(ebq.LIB_PATH):
        from extreme_bit_quantized_amd import build

        build.build()
    ebq.load()
    return ebq


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([a-z][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol(ebq):
    names = _declared_functions()
    assert len(names) >= 17, names
    lib = ctypes.CDLL(ebq.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def _declared_arity():
    """name -> number of parameters, from the prototypes in the header."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    out = {}
    for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([a-z][a-z0-9_]*)\s*\(([^)]*)\)\s*;",
                         src, flags=re.M):
        params = " ".join(m.group(2).split())
        out[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_signatures_match_header(ebq):
    """Every ctypes prototype the binding sets has the header's parameter count."""
    arity = _declared_arity()
    lib = ebq.load()
    checked = 0
    for name, n in arity.items():
        f = getattr(lib, name)
        if f.argtypes is None:
            continue
        assert len(f.argtypes) == n, (name, len(f.argtypes), n)
        checked += 1
    assert checked >= 15, checked


def test_scale_storage_geometry(ebq, qref):
    """Scale groups are one GEMV segment; sizes follow the tiled formula and
    equal the plain [rows][cols/block] size when nothing is padded."""
    seg = {ebq.QFMT_TERN_B3: 1024, ebq.QFMT_INT2: 512, ebq.QFMT_SIGN1: 1024, ebq.QFMT_INT4: 256,
           ebq.QFMT_TRELLIS2: 512}
    for fmt in qref.FORMATS:
        blk = qref.scale_block(fmt)
        G = ebq.qfmt_scale_group(fmt)
        assert G * blk == seg[fmt]
        for N, K in ((1, 256), (64, 5120), (100, 1280), (17408, 5120), (5120, 17408), (6144, 5120)):
            if K % blk:
                continue
            nsb = K // blk
            tiled = -(-N // 64) * -(-nsb // G) * 64 * G * 2
            assert ebq.qfmt_scales_bytes(fmt, N, K) == tiled
            if N % 64 == 0 and nsb % G == 0:
                assert tiled == N * nsb * 2
    assert ebq.load().qfmt_scales_bytes(9, 64, 256) == -2
    assert ebq.load().qfmt_scales_bytes(ebq.QFMT_INT2, 64, 48) == -3


def test_geometry_agrees_with_oracle(ebq, qref):
    for fmt in qref.FORMATS:
        assert ebq.qfmt_scale_block(fmt) == qref.scale_block(fmt)
        blk = qref.scale_block(fmt)
        for K in (blk, 2 * blk, 256, 1024, 1280, 5120, 6144, 17408):
            if K % blk or K % 32:
                continue
            assert ebq.qfmt_packed_row_bytes(fmt, K) == qref.packed_row_bytes(fmt, K)
            assert ebq.qfmt_row_bytes(fmt, K) == qref.row_stride(fmt, K)
    assert ebq.load().qfmt_row_bytes(9, 256) == -2
    assert ebq.load().qfmt_row_bytes(ebq.QFMT_INT2, 48) == -3


def _desc(ebq, fmt=3, rows=64, cols=1024, block=None, codes=4096, row_bytes=None, scales=8192, seeds=None):
    if block is None:
        block = ebq.qfmt_scale_block(fmt) if fmt in (1, 2, 3, 4, 5) else 32
    if row_bytes is None:
        row_bytes = ebq.load().qfmt_row_bytes(fmt, cols) if fmt in (1, 2, 3, 4, 5) else 16
    return ebq.qweight_t(fmt, rows, cols, block, codes, row_bytes, scales, seeds)


def test_weight_validation(ebq):
    L = ebq.load()
    chk = lambda d: L.qweight_check(ctypes.byref(d))
    assert chk(_desc(ebq)) == 0
    assert chk(_desc(ebq, fmt=7)) == -2
    assert chk(_desc(ebq, block=64)) == -3
    assert chk(_desc(ebq, cols=1000)) == -3
    assert chk(_desc(ebq, rows=-1)) == -1
    assert chk(_desc(ebq, codes=4104)) == -4
    assert chk(_desc(ebq, scales=8193)) == -4
    assert chk(_desc(ebq, codes=None)) == -1
    assert chk(_desc(ebq, row_bytes=64)) == -3          # below the packed size
    assert chk(_desc(ebq, row_bytes=136)) == -3         # not a multiple of 16
    assert chk(_desc(ebq, fmt=5, cols=512)) == -1       # trellis without seeds
    assert chk(_desc(ebq, fmt=5, cols=512, seeds=12288)) == 0
    assert chk(_desc(ebq, rows=0, codes=None, scales=None)) == 0  # empty matrix


def test_call_validation_without_gpu(ebq):
    L = ebq.load()
    d = _desc(ebq)
    w = ctypes.byref(d)
    A = 1 << 20  # fake, aligned "device" addresses: every call below is rejected before launch
    assert L.qgemv(w, A, A, A, A, 65, A, None) == -1
    assert L.qgemv(w, A, A, A, A, -1, A, None) == -1
    assert L.qgemv(w, A, A, A, A, 0, A, None) == 0         # empty batch: no-op
    # 1-bit reads the activation planes (32-byte aligned); q is not needed
    assert L.qgemv(w, A, A + 16, A, A, 1, A, None) == -4
    assert L.qgemv(w, A, None, A, A, 1, A, None) == -1
    assert L.qgemv(w, None, A, A, A, 1, A + 2, None) == -4
    assert L.qgemv(w, None, A, None, A, 1, A, None) == -1
    # ternary reads q (16-byte aligned); planes are not needed
    t = ctypes.byref(_desc(ebq, fmt=1))
    assert L.qgemv(t, A + 4, None, A, A, 1, A, None) == -4
    assert L.qgemv(t, None, A, A, A, 1, A, None) == -1
    assert L.qgemv(t, A, None, A, A, 1, A + 2, None) == -4
    assert L.qgemv_blockdots(w, A, None, A, A, None) == -1
    assert L.qgemv_blockdots(t, A, None, A, A + 2, None) == -4
    assert L.qact_planes(A, 1, 48, A, None) == -3
    assert L.qact_planes(A, 1, 64, A + 16, None) == -4
    assert L.qact_planes(A + 2, 1, 64, A, None) == -4
    assert L.qact_planes(A, 0, 64, A, None) == 0
    assert L.qact_planes(None, 1, 64, A, None) == -1
    assert L.qact_quant_i8(A, 1, 1024, 64, A, A, A, None) == -1
    assert L.qact_quant_i8(A, 1, 48, 32, A, A, A, None) == -3
    assert L.qact_quant_i8(A, 0, 1024, 32, A, A, A, None) == 0
    assert L.qact_quant_i8(A + 4, 1, 1024, 32, A, A, A, None) == -4
    assert L.qact_hadamard_quant_i8(A, 1, 1000, A, 256, A, A, A, None) == -3
    assert L.qact_hadamard_quant_i8(A, 1, 1024, None, 256, A, A, A, None) == -1
    assert L.qgemm_i8(A, A, 16, A, A, 16, 96, 32, A, None) == -3
    assert L.qgemm_i8(A, A, 16, A, A, 16, 256, 64, A, None) == -1
    assert L.qgemm_i8(A, A, 0, A, A, 16, 256, 256, A, None) == 0
    # one scale per row: kblock = K (any multiple of 64); other block sizes rejected
    assert L.qgemm_i8(A, A, 16, A, A, 16, 192, 96, A, None) == -1
    assert L.qgemm_i8(A, A, 16, A, A, 16, 160, 160, A, None) == -3     # K % 64
    assert L.qgemm_i8(A + 4, A, 16, A, A, 16, 192, 192, A, None) == -4
    assert L.qgemm_i8(A, A, 0, A, A, 16, 192, 192, A, None) == 0
    # rotation + Q8 per token row: qblock = K, at most 32768
    assert L.qact_hadamard_quant_i8(A, 1, 1024, A, 512, A, A, A, None) == -1
    assert L.qact_hadamard_quant_i8(A, 1, 33024, A, 33024, A, A, A, None) == -3
    assert L.qact_hadamard_quant_i8(A, 0, 5120, A, 5120, A, A, A, None) == 0
    assert L.qtrellis_decode_i8(w, 256, A, A, None) == -2   # not a trellis matrix
    tr = ctypes.byref(_desc(ebq, fmt=5, cols=5120, seeds=12288))
    assert L.qtrellis_decode_i8(tr, 512, A, A, None) == -1  # block neither 32, 256 nor the row
    assert L.qtrellis_decode_i8(tr, 5120, A + 2, A, None) == -4
    big = ctypes.byref(_desc(ebq, fmt=5, cols=33024, seeds=12288))
    assert L.qtrellis_decode_i8(big, 33024, A, A, None) == -3  # one scale per row: at most 32768
    assert L.qweight_quantize(5, A, 4, 256, A, 64, A, None) == -2
    assert L.qweight_pack(2, A, 4, 48, A, 16, None) == -3
    assert L.qgemv_grouped_run(None, A, None) == -1
    J = ebq.qact_job_t
    def jobs(*js):
        arr = (J * max(1, len(js)))(*js)
        return arr, len(js)
    ok = J(A, 2, 64, A, A, A, A)
    assert L.qact_quant_batch(jobs(ok)[0], 17, None) == -1
    assert L.qact_quant_batch(jobs(ok)[0], -1, None) == -1
    assert L.qact_quant_batch(None, 0, None) == 0
    assert L.qact_quant_batch(*jobs(J(A, 2, 48, A, A, A, A)), None) == -3
    assert L.qact_quant_batch(*jobs(ok, J(A + 4, 2, 64, A, A, A, A)), None) == -4
    assert L.qact_quant_batch(*jobs(J(A, 2, 64, A, A + 16, A, A)), None) == -4
    assert L.qact_quant_batch(*jobs(J(A, 2, 64, None, None, A, A)), None) == -1
    assert L.qact_quant_batch(*jobs(J(A, 2, 64, A, None, None, A)), None) == -1
    assert L.qact_quant_batch(*jobs(J(A, 0, 64, None, None, None, None)), None) == 0   # empty input: no launch
    assert L.qcalib_mfma_i8(-1, 10, A, A, None) == -1
    assert L.qcalib_mfma_i8(0, 10, A, A, None) == 0
    assert L.qcalib_mfma_i8(2, 10, None, A, None) == -1
    assert L.qcalib_mfma_i8(2, 10, A + 4, A, None) == -4
    assert ebq.load().qstrerror(-4).decode().startswith("pointer")
    assert L.qcalib_hbm_read(A, -16, A, None) == -1
    assert L.qcalib_hbm_read(A, 0, A, None) == 0
    assert L.qcalib_hbm_read(None, 16, A, None) == -1
    assert L.qcalib_hbm_read(A, 24, A, None) == -3
    assert L.qcalib_hbm_read(A + 8, 16, A, None) == -4


def test_grouped_plan_on_host(ebq):
    import torch

    A = 1 << 20
    shapes = [(3, 5120, 1024), (1, 1024, 5120), (3, 100, 1024), (4, 17408, 512)]
    descs = [_desc(ebq, fmt=f, rows=n, cols=k, codes=A, scales=A) for f, n, k in shapes]
    items = (ebq.qgemv_item_t * len(descs))()
    for i, d in enumerate(descs):
        items[i] = ebq.qgemv_item_t(d, A, A, A, A, A)
    nb = ebq.qgemv_grouped_plan_bytes(items, 2)
    raw = torch.zeros(nb + 16, dtype=torch.uint8)
    off = (-raw.data_ptr()) % 16
    host = raw[off:off + nb]
    ebq.qgemv_grouped_plan(items, 2, host)
    h = host.numpy()
    hdr = np.frombuffer(h[:64].tobytes(), dtype=np.int32)
    assert hdr[0] == 0x50564751 and hdr[2] == 4 and hdr[4] == 2
    ntiles = sum((n + 63) // 64 for _, n, _ in shapes)
    assert hdr[3] == ntiles
    tiles_off = int(np.frombuffer(h[32:40].tobytes(), dtype=np.int64)[0])
    tiles = np.frombuffer(h[tiles_off:tiles_off + 8 * ntiles].tobytes(), dtype=np.uint32).reshape(-1, 2)
    got = sorted(map(tuple, tiles.tolist()))
    want = sorted((i, r) for i, (_, n, _) in enumerate(shapes) for r in range(0, n, 64))
    assert got == want
    # tiles are grouped by format: format f owns [fmt_begin[f], fmt_begin[f + 1])
    fmt_of = [s[0] for s in shapes]
    fb = np.frombuffer(h[48:80].tobytes(), dtype=np.int32)
    assert fb[1] == 0 and fb[6] == ntiles
    for k, (i, r) in enumerate(tiles.tolist()):
        assert fb[fmt_of[i]] <= k < fb[fmt_of[i] + 1]
    # inside a format the tiles are dealt to 256 lists, stored list by list:
    # longest first inside a list, and the lists' byte totals differ by at most
    # one tile (each tile, longest first, went to the list with the fewest bytes)
    nwk = int(np.frombuffer(h[80:84].tobytes(), dtype=np.int32)[0])
    workers_off = int(np.frombuffer(h[88:96].tobytes(), dtype=np.int64)[0])
    assert nwk == 256
    wb_all = np.frombuffer(h[workers_off:workers_off + 4 * 6 * (nwk + 1)].tobytes(), dtype=np.int32)
    cost = lambda i, r: min(64, shapes[i][1] - r) * (descs[i].row_bytes + shapes[i][2] // descs[i].block * 2)
    tl = tiles.tolist()
    for f in set(fmt_of):
        wb = wb_all[f * (nwk + 1):(f + 1) * (nwk + 1)]
        assert wb[0] == fb[f] and wb[-1] == fb[f + 1] and (np.diff(wb) >= 0).all()
        loads = []
        for w in range(nwk):
            c = [cost(*tl[k]) for k in range(wb[w], wb[w + 1])]
            assert c == sorted(c, reverse=True)
            loads.append(sum(c))
        fcosts = [cost(i, r) for i, r in tl if fmt_of[i] == f]
        assert max(loads) - min(loads) <= max(fcosts)
    # too small a buffer is refused
    assert ebq.load().qgemv_grouped_plan(items, 4, 2, host.data_ptr(), nb - 16) == -6
    # batches up to 64 (above 6 the launch runs on the matrix cores)
    assert ebq.load().qgemv_grouped_plan_bytes(items, 4, 64) > 0
    assert ebq.load().qgemv_grouped_plan_bytes(items, 4, 65) == -1
    assert ebq.load().qgemv_grouped_plan_bytes(items, 4, 0) == -1


def test_grouped_plan_keeps_its_tensors(ebq):
    """The plan stores raw device addresses, so the Python plan object holds every
    tensor of every entry (and the PackedWeights) for its own lifetime: dropping
    the caller's references frees nothing.  Host tensors stand in for device ones
    (building a plan is host work; nothing runs)."""
    import gc
    import weakref

    import torch

    def aligned(n):
        """n zero bytes on the host, 64-byte aligned."""
        raw = torch.zeros(n + 64, dtype=torch.uint8)
        off = (-raw.data_ptr()) % 64
        return raw[off:off + n]

    fmt, N, K = 3, 70, 1024
    codes = aligned(N * ebq.qfmt_row_bytes(fmt, K)).view(N, -1)
    scales = aligned(ebq.qfmt_scales_bytes(fmt, N, K)).view(torch.int16)
    pw = ebq.PackedWeight(fmt, N, K, codes, scales)
    planes = aligned(4 * 8 * K // 32).view(torch.int32)
    d = aligned(4 * K // 32).view(torch.float32)
    qs = aligned(4 * K // 32).view(torch.int32)
    y = aligned(4 * N).view(torch.float32)
    refs = [weakref.ref(t) for t in (codes, scales, planes, d, qs, y)] + [weakref.ref(pw)]
    plan = ebq.GroupedPlan([(pw, None, planes, d, qs, y)], 1, device="cpu")
    del codes, scales, pw, planes, d, qs, y
    gc.collect()
    assert all(r() is not None for r in refs)
    del plan
    gc.collect()
    assert all(r() is None for r in refs)


def test_static_plan_size_limit(ebq):
    """qgemv_grouped_run_static refuses a plan larger than its static storage
    before any HIP call (so this runs without a GPU)."""
    import torch

    A = 1 << 20
    rows = 64 * 140000                     # 140000 tiles of 8 bytes: more than 1 MiB of plan
    d = _desc(ebq, fmt=3, rows=rows, cols=1024, codes=A, scales=A)
    items = (ebq.qgemv_item_t * 1)()
    items[0] = ebq.qgemv_item_t(d, A, A, A, A, A)
    nb = ebq.qgemv_grouped_plan_bytes(items, 1)
    assert nb > ebq.QGEMV_STATIC_PLAN_BYTES
    raw = torch.zeros(nb + 16, dtype=torch.uint8)
    off = (-raw.data_ptr()) % 16
    host = raw[off:off + nb]
    ebq.qgemv_grouped_plan(items, 1, host)
    L = ebq.load()
    assert L.qgemv_grouped_run_static(host.data_ptr(), None) == -7
    assert L.qgemv_grouped_run_static(None, None) == -1
    assert L.qgemv_grouped_run_static(host.data_ptr() + 4, None) == -4
    junk = torch.zeros(256, dtype=torch.uint8)
    o2 = (-junk.data_ptr()) % 16
    assert L.qgemv_grouped_run_static(junk[o2:].data_ptr(), None) == -6
    assert "static plan" in L.qstrerror(-7).decode()


def test_trellis_encode_validation_without_gpu(ebq):
    """The encoder's argument checks run on the host before any HIP call."""
    L = ebq.load()
    A = 1 << 20
    need = L.qtrellis_encode_workspace_bytes(4, 256, 2)
    # scales of all rows, (state, cost) per pass row, 4 KB of choices per pass row and step
    assert need == 2048 // 2048 * 256 + 256 + 2 * 255 * 4096
    assert L.qtrellis_encode_workspace_bytes(4, 256, 9) == L.qtrellis_encode_workspace_bytes(4, 256, 4)
    assert L.qtrellis_encode_workspace_bytes(4, 96, 2) == -3
    assert L.qtrellis_encode_workspace_bytes(0, 256, 2) == -1
    assert L.qtrellis_encode_workspace_bytes(4, 256, 0) == -1

    def enc(w=A, rows=4, cols=256, si=None, codes=A, rb=64, seeds=A, sc=A, cost=None, per=2, ws=A, wsb=need):
        return L.qtrellis_encode(w, rows, cols, si, codes, rb, seeds, sc, cost, per, ws, wsb, None)

    assert enc(rows=0) == 0
    assert enc(rows=-1) == -1
    assert enc(per=0) == -1
    assert enc(cols=96) == -3
    assert enc(cols=32) == -3
    assert enc(cols=(1 << 20) + 64) == -3
    assert enc(rb=48) == -3             # below the 64 packed bytes of 256 symbols
    assert enc(rb=72) == -3             # not a multiple of 16
    assert enc(w=None) == -1 and enc(codes=None) == -1 and enc(seeds=None) == -1
    assert enc(sc=None) == -1 and enc(ws=None) == -1
    assert enc(w=A + 2) == -4 and enc(codes=A + 8) == -4 and enc(seeds=A + 1) == -4
    assert enc(sc=A + 8) == -4 and enc(si=A + 1) == -4 and enc(cost=A + 2) == -4 and enc(ws=A + 128) == -4
    assert enc(wsb=need - 1) == -6


def test_attention_validation_without_gpu(ebq):
    L = ebq.load()
    A = 1 << 20
    assert L.qkv_row_bytes(8) == 256 and L.qkv_row_bytes(4) == 128 and L.qkv_row_bytes(5) == -2
    assert L.qkv_quant(5, A, 4, A, A, None) == -2
    assert L.qkv_quant(8, A, 0, A, A, None) == 0
    assert L.qkv_quant(8, A, -1, A, A, None) == -1
    assert L.qkv_quant(8, None, 4, A, A, None) == -1
    assert L.qkv_quant(8, A + 4, 4, A, A, None) == -4
    assert L.qkv_quant(4, A, 4, A + 8, A, None) == -4
    # partial sums of 256-token chunks: [rows][chunks][256 values + max + sum] fp32
    assert L.qattn_decode_workspace_bytes(4, 6, 65536) == 24 * 256 * 258 * 4
    assert L.qattn_decode_workspace_bytes(4, 9, 100) == -1
    need = L.qattn_decode_workspace_bytes(2, 6, 300)

    def att(fmt=8, q=A, n_kv=2, group=6, hpb=6, T=300, t_cap=512, kc=A, ks=A, vc=A, vs=A, out=A, ws=A, wsb=need):
        return L.qattn_decode(fmt, q, n_kv, group, hpb, T, t_cap, kc, ks, vc, vs, out, ws, wsb, None)

    assert att(fmt=5) == -2
    assert att(group=0) == -1 and att(group=9, hpb=9) == -1
    assert att(hpb=3) == -1 and att(hpb=1, T=0) == -3
    assert att(T=0) == -3 and att(t_cap=299) == -3
    assert att(q=None) == -1 and att(kc=None) == -1 and att(vs=None) == -1 and att(ws=None) == -1
    assert att(q=A + 4) == -4 and att(kc=A + 8) == -4 and att(ks=A + 1) == -4 and att(out=A + 2) == -4
    assert att(ks=A + 2) == -4 and att(vs=A + 8) == -4  # scale rows are read 16 bytes at a time
    assert att(wsb=need - 1) == -6
