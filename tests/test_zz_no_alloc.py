"""The no-allocation grouped launch (qgemv_grouped_run_static) against the
launch it is a variant of (qgemv_grouped_run with the caller's device copy of
the plan): bit-identical outputs, and both within the oracle's tolerance, on
two calls in a row, the second with a smaller plan (the static storage keeps
the first call's plan until the second overwrites it)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import INT2, INT4, NAMES, SIGN1, TERN, TRELLIS, assert_close_terms, gpu_act_planes, gpu_weight, \
    host, oracle_weight, raw_weight

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import extreme_bit_quantized_amd as ebq  # noqa: E402


def _plan(specs, B, seed):
    entries, refs = [], []
    for i, (fmt, N, K) in enumerate(specs):
        raw = raw_weight(fmt, N, K, seed + i)
        pw = gpu_weight(fmt, raw, N, K)
        rp, rs, rseeds = oracle_weight(fmt, raw)
        x = synth.gauss([seed + i, 9], (B, K))
        q, pl, d, s = gpu_act_planes(x)
        y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
        entries.append((pw, q, pl, d, s, y))
        rq, rd, _ = oracle.act_quant(x)
        refs.append(oracle.gemv(fmt, rp, rs, rseeds, K, rq, rd))
    return ebq.GroupedPlan(entries, B), entries, refs


def test_static_plan_matches_device_plan():
    ebq.load()
    big = [(SIGN1, 300, 5120), (TERN, 200, 2048), (INT4, 130, 1280), (INT2, 90, 2560), (TRELLIS, 70, 1536),
           (SIGN1, 65, 17408)]
    small = [(INT4, 65, 1024), (SIGN1, 1, 1024), (TERN, 70, 1280)]  # one token: the matrix-core ternary kernel
    for call, (B, specs, seed) in enumerate(((3, big, 600), (1, small, 620))):
        plan, entries, refs = _plan(specs, B, seed)
        assert plan.host.numel() <= ebq.QGEMV_STATIC_PLAN_BYTES
        plan.run()
        torch.cuda.synchronize()
        want = [host(e[5]).copy() for e in entries]
        for e in entries:
            e[5].fill_(float("nan"))
        plan.run_static()
        torch.cuda.synchronize()
        for (fmt, N, K), e, w, (yr, absT, _) in zip(specs, entries, want, refs):
            got = host(e[5])
            assert (got.view(np.uint32) == w.view(np.uint32)).all(), "call %d %s" % (call, NAMES[fmt])
            assert_close_terms(got, yr, absT, what="static plan, call %d %s" % (call, NAMES[fmt]))
