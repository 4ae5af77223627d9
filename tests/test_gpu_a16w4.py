"""GPU parity of the A16WFP4 variant (bf16 activations x decoded MXFP4 weight on the bf16
MFMA) against the oracle (oracle/mx_oracle.py: gemm_a16w4_ref), within the GEMM tolerance
|gpu - exact| <= 2^-7 |exact| + 1e-3 rms(exact): every output for ragged M over several
64-row tiles and K = 256 .. 4224 (2 to 33 steps), each tile width of the tiled form, the decode form (M <= 32) over its launch
shapes, sampled rows at the headline shape
(N = 7168, K = 768, M = 2048, the launch the bench times); a one-hot activation probe that
must reproduce the decoded weight bit for bit; canary rows past M left untouched."""
import numpy as np
import pytest

import workloads as W
from oracle import mx_oracle as O

from gpu_util import check_gemm, dev_bf16, host_bits, lib_or_fail, sample_rows, torch_or_skip

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K", [256, 768, 1024, 4224])
@pytest.mark.parametrize("M", [1, 37, 64, 100, 300])
def test_a16w4_matches_oracle(M, K):
    torch = torch_or_skip()
    mx = lib_or_fail()
    N = 768
    a = W.dense_activation(300, K, "plain", seed=71)[:M]
    w = W.dense_weight(N, K, seed=72)
    wp = mx.mx_prepare_weight(dev_bf16(w))
    out = torch.full((M + 3, N), 5.0, dtype=torch.bfloat16, device="cuda")
    mx.mx_a16w4_gemm(dev_bf16(a), wp, N, out=out[:M])
    c = host_bits(out)
    torch.cuda.synchronize()
    assert np.all(O.bf16_to_f64(c[M:]) == 5.0)
    check_gemm(c[:M], O.gemm_a16w4_ref(a, w), what=f"a16w4 M={M} K={K}")


@pytest.mark.parametrize("N,K,M", [(768, 768, 1), (768, 768, 16), (768, 4224, 5), (8192, 256, 3),
                                   (256, 9216, 2), (8192, 768, 16), (768, 768, 17), (768, 4224, 32),
                                   (8192, 768, 32), (256, 9216, 20)])
def test_a16w4_decode_form_matches_oracle(N, K, M):
    """The decode form (M <= 32, one or two 16-row tiles): one and two column groups per
    CTA, four and eight waves, a K share of 1 to 9 steps per wave (9216 = 72 steps: two
    prefetch chunks of 8, or three of 4 with two row tiles), rows past M neither read as
    real rows nor written."""
    torch = torch_or_skip()
    mx = lib_or_fail()
    assert mx.mx_a16w4_gemm_plan(M, N, K).startswith("k_gemm_a16w4_stream<")
    a = W.dense_activation(32, K, "plain", seed=74)[:M]
    w = W.dense_weight(N, K, seed=75)
    wp = mx.mx_prepare_weight(dev_bf16(w))
    out = torch.full((M + 3, N), 5.0, dtype=torch.bfloat16, device="cuda")
    mx.mx_a16w4_gemm(dev_bf16(a), wp, N, out=out[:M])
    c = host_bits(out)
    torch.cuda.synchronize()
    assert np.all(O.bf16_to_f64(c[M:]) == 5.0)
    check_gemm(c[:M], O.gemm_a16w4_ref(a, w), what=f"a16w4 decode N={N} K={K} M={M}")


@pytest.mark.parametrize("M,ngw", [(100, 1), (256, 2), (300, 2), (512, 4), (520, 4)])
def test_a16w4_tile_widths_match_oracle(M, ngw):
    """The tiled form at N = 7168, K = 1024 (8 steps, loads two steps ahead) in each of its tile
    widths, 64 x 64 NGW, every output against the oracle, ragged last row tiles, canary rows
    past M. (K = 256, 768, 1024 and 4224 in the test above give 2, 6, 8 and 33 steps: an odd
    count takes the loop's remainder path.)"""
    torch = torch_or_skip()
    mx = lib_or_fail()
    N, K = 7168, 1024
    plan = mx.mx_a16w4_gemm_plan(M, N, K)
    assert plan == f"k_gemm_a16w4<{ngw}, 2> (64 x {64 * ngw} tiles)", plan
    a = W.dense_activation(M, K, "outlier_channels", seed=76)
    w = W.dense_weight(N, K, seed=77)
    wp = mx.mx_prepare_weight(dev_bf16(w))
    out = torch.full((M + 3, N), 5.0, dtype=torch.bfloat16, device="cuda")
    mx.mx_a16w4_gemm(dev_bf16(a), wp, N, out=out[:M])
    c = host_bits(out)
    torch.cuda.synchronize()
    assert np.all(O.bf16_to_f64(c[M:]) == 5.0)
    check_gemm(c[:M], O.gemm_a16w4_ref(a, w), what=f"a16w4 tiles 64x{64 * ngw} M={M}")


def test_a16w4_headline_shape_sampled():
    torch = torch_or_skip()
    mx = lib_or_fail()
    N, K, ms, st = W.DENSE_CONFIGS["n7168_k768"]
    M = max(ms)
    a = W.dense_activation(M, K, st)
    w = W.dense_weight(N, K)
    c = host_bits(mx.mx_a16w4_gemm(dev_bf16(a), mx.mx_prepare_weight(dev_bf16(w)), N))
    torch.cuda.synchronize()
    rows = sample_rows(M, n=32, seed=9)
    check_gemm(c[rows], O.gemm_a16w4_ref(a[rows], w), what="a16w4 7168x768 M=2048")


def test_a16w4_one_hot_reproduces_decoded_weight():
    torch = torch_or_skip()
    mx = lib_or_fail()
    N, K = 512, 256
    w = W.dense_weight(N, K, seed=73)
    qw, sw = O.quantize_mx(w)
    deq = O.dequantize_mx(qw, sw)
    ks = np.array([0, 1, 31, 32, 100, 128, 200, 255])
    a = np.zeros((ks.size, K), dtype=np.uint16)
    a[np.arange(ks.size), ks] = 0x3F80                        # bf16 1.0
    c = host_bits(mx.mx_a16w4_gemm(dev_bf16(a), mx.mx_prepare_weight(dev_bf16(w)), N))
    torch.cuda.synchronize()
    assert np.array_equal(O.bf16_to_f64(c), deq[:, ks].T)     # one exact product per output
