"""Weight preparation from a caller-quantized weight (packed E2M1 codes and E8M0 scales,
preshuffled once: "[gfx950][FlyDSL] Add direct dense A4W4 MXFP4 GEMM", Scope).

- The oracle's quantization of a seeded weight, prepared this way, unprepares to itself
  and yields the same blob as preparing the bf16 weight.
- Arbitrary bytes (every E2M1 code, scale bytes 0..254) survive the round trip unchanged.
- A GEMM against a weight of random codes and scales (never produced by this library's
  quantizer) matches the oracle's exact product of the same MXFP4 operands, on the
  streaming kernel (M = 1, 8) and the tiled kernel (M = 37, 300), with ragged M tails."""
import numpy as np
import pytest

import workloads as W
from oracle import mx_oracle as O

from gpu_util import check_gemm, dev_bf16, host_bits, host_u8, lib_or_fail, torch_or_skip

pytestmark = pytest.mark.gpu


def _dev_u8(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).cuda()


def test_packed_oracle_weight_round_trip_and_matches_bf16_prepare():
    torch = torch_or_skip()
    mx = lib_or_fail()
    N, K = 768, 4224  # three quads of column groups, 33 K steps
    w = W.dense_weight(N, K, seed=31)
    qw, sw = O.quantize_mx(w)
    wp = mx.mx_prepare_weight_packed(_dev_u8(qw), _dev_u8(sw))
    q, s = mx.mx_unprepare_weight(wp, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(q), qw)
    assert np.array_equal(host_u8(s), sw)
    wp2 = mx.mx_prepare_weight(dev_bf16(w))
    torch.cuda.synchronize()
    assert torch.equal(wp, wp2)


def test_packed_arbitrary_bytes_round_trip():
    torch = torch_or_skip()
    mx = lib_or_fail()
    N, K = 512, 256
    rng = np.random.default_rng(41)
    qw = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    sw = rng.integers(0, 255, size=(N, K // 32), dtype=np.uint8)
    wp = mx.mx_prepare_weight_packed(_dev_u8(qw), _dev_u8(sw))
    assert wp.numel() == mx.mx_prepared_weight_bytes(N, K)
    q, s = mx.mx_unprepare_weight(wp, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(q), qw)
    assert np.array_equal(host_u8(s), sw)


@pytest.mark.parametrize("M", [1, 8, 37, 300])
def test_gemm_on_caller_packed_weight(M):
    torch = torch_or_skip()
    mx = lib_or_fail()
    N, K = 768, 768
    rng = np.random.default_rng(51)
    qw = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)           # every E2M1 code, both signs
    sw = rng.integers(127 - 9, 127 + 10, size=(N, K // 32), dtype=np.uint8)  # scales 2^-9 .. 2^9
    a = W.dense_activation(300, K, "plain", seed=52)[:M]
    qa, sa = O.quantize_mx(a)
    exact = O.gemm_from_mx(qa, sa, qw, sw)
    wp = mx.mx_prepare_weight_packed(_dev_u8(qw), _dev_u8(sw))
    c = host_bits(mx.mx_a4w4_gemm(dev_bf16(a), wp, N))
    torch.cuda.synchronize()
    check_gemm(c, exact, what=f"packed weight M={M} ({mx.mx_a4w4_gemm_plan(M, N, K)})")


def test_packed_shape_errors():
    torch = torch_or_skip()
    mx = lib_or_fail()
    q = torch.zeros((256, 100), dtype=torch.uint8, device="cuda")    # K = 200: not a multiple of 128
    s = torch.zeros((256, 6), dtype=torch.uint8, device="cuda")
    with pytest.raises(mx.MxError):
        mx.mx_prepare_weight_packed(q, s)
    with pytest.raises(ValueError):
        mx.mx_prepare_weight_packed(torch.zeros((256, 128), dtype=torch.uint8, device="cuda"), s)
