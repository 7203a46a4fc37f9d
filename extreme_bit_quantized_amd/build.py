"""Build libqgemv.so in-tree with hipcc for gfx950.

    python -m extreme_bit_quantized_amd.build [--jobs N]

Every source under csrc/ is compiled to an object under _build/ (the GEMV
instantiation file once per batch size), then linked into
extreme_bit_quantized_amd/libqgemv.so.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqgemv.so")
ARCH = "gfx950"
MAX_B = 6          # lane-per-row dot4 GEMV batch sizes (one object each)
MAX_TG = 4         # matrix-core GEMV token groups of 16 (batches up to 64)

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++20", "-fPIC",
    # packed fp32 VALU ops stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-ffp-contract=fast-honor-pragmas",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I" + os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libqgemv")


def _units():
    units = []
    for name in sorted(os.listdir(CSRC)):
        if not name.endswith(".hip"):
            continue
        src = os.path.join(CSRC, name)
        if name == "gemv_inst.hip":
            for b in range(1, MAX_B + 1):
                units.append((src, os.path.join(BUILD, "gemv_b%d.o" % b), ["-DQGEMV_NB=%d" % b]))
        elif name == "gemv_mfma_inst.hip":
            for t in range(1, MAX_TG + 1):
                units.append((src, os.path.join(BUILD, "gemv_mfma_tg%d.o" % t), ["-DQGEMV_TG=%d" % t]))
        else:
            units.append((src, os.path.join(BUILD, name[:-4] + ".o"), []))
    return units


def _scratch_users(remarks: str):
    """Kernels whose resource-usage remark reports scratch memory (bytes/lane > 0)."""
    users, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)) > 0:
            users.append((name, int(m.group(1))))
    return users


# MFMAs written as inline asm are opaque to the compiler: it inserts no wait
# states after them, so a read of an MFMA's result (or a write to its
# destination) that the compiler schedules right behind it sees the old value.
# Sources with such MFMAs have their device assembly checked: every access to
# an MFMA destination register by another instruction must come at least
# MFMA_WAIT_STATES wait states (instructions; s_nop n counts n + 1) after it.
# Straight-line approximation: a label does not reset the count.
MFMA_WAIT_STATES = 18
_ASM_MFMA = re.compile(r'"\s*v_mfma|"v_mfma_\w+ %|QG_MF\(')
_REG = re.compile(r"\b([av])(?:\[(\d+):(\d+)\]|(\d+)\b)")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(4) is not None:
            out.add((m.group(1), int(m.group(4))))
        else:
            out.update((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def mfma_result_hazards(asm: str, wait_states: int = MFMA_WAIT_STATES):
    """(function, distance, instruction) for each access to an MFMA destination
    register fewer than wait_states wait states after that MFMA (another MFMA
    accumulating into exactly that destination is the hardware's own chain)."""
    found, fn, pending, n = [], None, {}, 0
    for line in asm.splitlines():
        t = line.split(";")[0].strip()
        if re.match(r"^[A-Za-z_.$][\w.$]*:$", t):
            if not t.startswith("."):
                fn, pending, n = t[:-1], {}, 0
            continue
        if not t or t.startswith("."):
            continue
        op = t.split()[0]
        if op == "s_nop":
            n += int(t.split()[1], 0) + 1
            continue
        n += 1
        args = t[len(op):]
        mfma = op.startswith("v_mfma")
        parts = [x.strip() for x in args.split(",")]
        used = _regs(",".join(parts[1:3])) if mfma else _regs(args)
        near = [n - pending[r] for r in used if r in pending and n - pending[r] < wait_states]
        if near:
            found.append((fn, min(near), t))
        if mfma:
            for r in _regs(parts[0]):
                pending[r] = n
        else:
            for r in used:
                pending.pop(r, None)
    return found


def _check_asm_mfma(hipcc, src, extra):
    with open(src) as f:
        if not _ASM_MFMA.search(f.read()):
            return
    out = os.path.join(BUILD, os.path.basename(src)[:-4] + "".join(extra).replace("=", "") + ".s")
    cmd = [hipcc] + FLAGS + extra + ["--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc -S failed for %s:\n%s" % (os.path.basename(src), r.stderr))
    with open(out) as f:
        bad = mfma_result_hazards(f.read())
    if bad:
        raise RuntimeError("%s: MFMA results accessed too early: %s" % (os.path.basename(src), bad[:4]))


def _compile(hipcc, src, obj, extra):
    cmd = [hipcc] + FLAGS + extra + ["-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line,
    # and the per-kernel resource remarks (checked below)
    lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
    err = "\n".join(l for l in lines if "kernel-resource-usage" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (os.path.basename(obj), err))
    # A kernel in scratch memory means a register array indexed at run time or a
    # spill: an order of magnitude slower, and never intended here.
    users = _scratch_users(r.stderr)
    if users:
        raise RuntimeError("%s: kernels using scratch memory: %s" % (os.path.basename(obj), users))
    return err


def build(jobs: int | None = None, verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    units = _units()
    jobs = jobs or min(len(units), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_compile, hipcc, s, o, e) for s, o, e in units]
        futs += [ex.submit(_check_asm_mfma, hipcc, s, e) for s, _, e in units]
        for f in futs:
            msg = f.result()
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + [o for _, o, _ in units]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.v))
