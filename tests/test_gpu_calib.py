"""The roofline calibration kernels run on the device and leave their sink untouched (the
folded value never hits the improbable constant that would store it)."""
import pytest

from gpu_util import lib_or_fail, torch_or_skip

pytestmark = pytest.mark.gpu


def test_calibration_kernels_run():
    torch = torch_or_skip()
    mx = lib_or_fail()
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    buf = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
    for ctas in (1, 3, 512):  # grid smaller and larger than the 16-byte words per round
        mx.mx_calib_read(buf, ctas, sink)
    mx.mx_calib_read(buf[:4112], 2, sink)  # a ragged tail after the unrolled rounds
    mx.mx_calib_mfma(8, 16, sink)
    ops = torch.randint(0, 256, (3 * 16384 + 100,), dtype=torch.uint8, device="cuda")
    for ctas in (1, 5):  # 4 and 20 waves over the 3 whole windows of the buffer
        mx.mx_calib_mfma_operands(ops, ctas, 16, sink)
    clocks = torch.full((8 * 5 + 2,), -1, dtype=torch.int64, device="cuda")
    mx.mx_calib_mfma_operands_clock(ops, 5, 4096, sink, clocks)
    torch.cuda.synchronize()
    assert sink.cpu().tolist() == [7, 7, 7, 7]
    c = clocks.cpu().tolist()
    assert c[40:] == [-1, -1], "nothing written past the 20 waves' pairs"
    for w in range(20):
        ticks, rt = c[2 * w], c[2 * w + 1]
        assert ticks > 0 and rt > 0, (w, ticks, rt)
        # 4096 rounds of 64 MFMAs hold the pipe at least 16 cycles each; the clock lies
        # between 0.5 and 3 GHz
        assert ticks >= 4096 * 64 * 16, (w, ticks)
        assert 0.5e9 < ticks / (rt / 100e6) < 3e9, (w, ticks, rt)
    with pytest.raises(mx.MxError):
        mx.mx_calib_read(buf[:1000], 8, sink)
