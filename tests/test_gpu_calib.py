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
    torch.cuda.synchronize()
    assert sink.cpu().tolist() == [7, 7, 7, 7]
    with pytest.raises(mx.MxError):
        mx.mx_calib_read(buf[:1000], 8, sink)
