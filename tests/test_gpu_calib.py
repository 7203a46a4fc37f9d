"""The matrix-core calibration entry point runs and its counters advance."""
import pytest

pytestmark = pytest.mark.gpu


def test_mfma_calibration_counters():
    import torch
    import extreme_bit_quantized_amd as ebq

    blocks, iters = 8, 200
    clocks = torch.zeros(4 * blocks, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ebq.qcalib_mfma_i8(blocks, iters, clocks, sink)
    torch.cuda.synchronize()
    c = clocks.view(blocks, 4).cpu()
    # 200 x 16 MFMAs of >= 16 cycles each per wave: the cycle counter moves by far more than that
    assert bool(((c[:, 1] - c[:, 0]) > 200 * 16 * 16).all())
    assert bool(((c[:, 3] - c[:, 2]) > 0).all())
    assert int(sink[0]) == 0


def test_hbm_read_calibration_runs():
    """The streaming-read calibration reads the whole buffer (a ragged size too)
    and leaves the sink alone for data that does not fold to its constant."""
    import torch
    import extreme_bit_quantized_amd as ebq

    buf = torch.zeros((1 << 24) + 48, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ebq.qcalib_hbm_read(buf, sink)
    ebq.qcalib_hbm_read(buf, sink, nbytes=16)
    torch.cuda.synchronize()
    assert int(sink[0]) == 0
