"""Exact probes through every kernel family, each forced with the library's tuning override.

* One-hot weight: W[n, k0 + n] = 1.0 (its block decodes to exactly 1.0), every other weight 0.
  Then C[m, n] = the decoded activation Q(A)[m, k0 + n], a single exact product, which bf16
  holds exactly: the inline (or once-only) quantization, the LDS operand layout, the scale
  op_sel plumbing and the output mapping of the kernel are checked bit for bit.
* Constant: A = 1 and W = 1 everywhere give C = K exactly (768, 4224 and 7168 are bf16 values).

The dense families: the weight-streaming kernel (with and without K slices), the tiled
kernel's 64 x 256, 128 x 512 and 64 x 64 tiles (and K slices), the short-K sweep kernel and
the quantize-once kernel's 256 x 256 and 128 x 128 tiles. The grouped families: the streaming
and the tiled grouped kernels, rows gathered by token over a ragged segment table."""
import os

import numpy as np
import pytest

import workloads as W
from oracle import mx_oracle as O

from gpu_util import dev_bf16, host_bits, lib_or_fail, torch_or_skip

pytestmark = pytest.mark.gpu

ONE = 0x3F80  # bf16 1.0
N_P = 512

# (override, K, rows, workspace bytes(M, K) or None)
DENSE = [
    ("s,1,1,4,1", 4224, (1, 7, 16), None),
    ("s,2,4,8,3", 4224, (17, 30), lambda M, K: 3 * M * N_P * 4),
    ("t,1,4,4,4,2,8,2", 4224, (1, 37, 300), None),
    ("t,1,8,8,4,1,8,2", 4224, (1, 37, 300), None),
    ("t,1,4,4,1,2,8,2", 4224, (1, 37, 300), None),
    ("t,1,4,4,4,2,8,2,4", 4224, (37, 130), lambda M, K: 4 * M * N_P * 4),
    ("k,4,8", 768, (1, 37, 300), None),
    ("q,2,4,8,4,4,2,8", 4224, (37, 300), lambda M, K: (M + 63) // 64 * 64 * K * 17 // 32),
    ("q,2,2,4,4,4,2,8", 7168, (37, 300), lambda M, K: (M + 63) // 64 * 64 * K * 17 // 32),
    ("r,8,8,2,8", 7168, (37, 300), lambda M, K: (M + 63) // 64 * 64 * K * 17 // 32),
    ("r,8,9,1,8", 4224, (37, 300), lambda M, K: (M + 63) // 64 * 64 * K * 17 // 32),
    ("x,8,8,2,8", 4224, (37, 300), lambda M, K: (M + 63) // 64 * 64 * K * 17 // 32),
    ("x,8,9,1,8", 4224, (37, 300), lambda M, K: (M + 63) // 64 * 64 * K * 17 // 32),
    ("x,8,7,2,8", 4224, (37, 300), lambda M, K: (M + 63) // 64 * 64 * K * 17 // 32),
    ("x,8,6,2,8", 4224, (37, 300), lambda M, K: (M + 63) // 64 * 64 * K * 17 // 32),
    ("x,8,3,4,1", 4224, (37, 300), lambda M, K: (M + 63) // 64 * 64 * K * 17 // 32),
    ("x,8,8,2,8,3", 7168, (37, 300),
     lambda M, K: ((M + 63) // 64 * 64 * K * 17 // 32 + 255) // 256 * 256 + 3 * M * N_P * 4),
]


def _one_hot_weight(N, K, k0):
    w = np.zeros((N, K), dtype=np.uint16)
    w[np.arange(N), k0 + np.arange(N)] = ONE
    return w


def _run_dense(mx, torch, cfg, a, wp, N, K, ws_fn):
    M = a.shape[0]
    out = torch.full((M + 3, N), -3.0, dtype=torch.bfloat16, device="cuda")
    ws = False if ws_fn is None else torch.empty(ws_fn(M, K), dtype=torch.uint8, device="cuda")
    os.environ["MX_GEMM_CONFIG"] = cfg
    try:
        mx.mx_a4w4_gemm(dev_bf16(a), wp, N, out=out[:M], workspace=ws)
    finally:
        del os.environ["MX_GEMM_CONFIG"]
    torch.cuda.synchronize()
    c = host_bits(out)
    assert np.all(O.bf16_to_f64(c[M:]) == -3.0), f"{cfg} M={M}: rows past M were written"
    return c[:M]


@pytest.mark.parametrize("cfg,K,ms,ws_fn", DENSE, ids=[d[0] for d in DENSE])
def test_one_hot_weight_probe_every_dense_family(cfg, K, ms, ws_fn):
    torch = torch_or_skip()
    mx = lib_or_fail()
    k0 = 128 if K == 768 else 992
    wp = mx.mx_prepare_weight(dev_bf16(_one_hot_weight(N_P, K, k0)))
    a_all = W.dense_activation(max(ms), K, "outlier_channels", seed=31)
    for M in ms:
        a = a_all[:M]
        c = _run_dense(mx, torch, cfg, a, wp, N_P, K, ws_fn)
        qa, sa = O.quantize_mx(a)
        want = O.dequantize_mx(qa, sa)[:, k0:k0 + N_P]
        got = O.bf16_to_f64(c)
        if not np.array_equal(got, want):
            i = np.argwhere(got != want)[0]
            raise AssertionError(f"{cfg} M={M} K={K}: {int((got != want).sum())} elements differ; first {tuple(i)}: "
                                 f"gpu {got[tuple(i)]!r} want {want[tuple(i)]!r}")


@pytest.mark.parametrize("cfg,K,ms,ws_fn", DENSE, ids=[d[0] for d in DENSE])
def test_constant_probe_every_dense_family(cfg, K, ms, ws_fn):
    torch = torch_or_skip()
    mx = lib_or_fail()
    wp = mx.mx_prepare_weight(dev_bf16(np.full((N_P, K), ONE, dtype=np.uint16)))
    for M in ms:
        c = _run_dense(mx, torch, cfg, np.full((M, K), ONE, dtype=np.uint16), wp, N_P, K, ws_fn)
        assert np.all(O.bf16_to_f64(c) == K), f"{cfg} M={M} K={K}"


GROUPED = ["gs,1,1", "gs,1,4", "gs,2,1", "gs,2,4", "gt,1,4,4,4,1,2", "gt,2,4,4,4,1,1", "gt,1,4,4,4,2,2",
           "gt,1,8,8,4,1,2"]


@pytest.mark.parametrize("cfg", GROUPED)
def test_one_hot_weight_probe_every_grouped_family(cfg, monkeypatch):
    """Every expert holds the one-hot weight, so output row r is the decoded activation row of
    token row_token[r] at columns k0 .. k0 + N - 1, exactly; segments of 0, 1, 63, 64, 130 and
    200 rows with tokens in a scrambled order."""
    torch = torch_or_skip()
    mx = lib_or_fail()
    N, K, k0, E, T = N_P, 4224, 640, 6, 150
    counts = np.array([0, 1, 63, 64, 130, 200])
    offs = np.zeros(E + 1, dtype=np.int32)
    offs[1:] = np.cumsum(counts)
    R = int(offs[-1])
    row_token = np.random.default_rng(5).integers(0, T, size=R).astype(np.int32)
    a = W.dense_activation(T, K, "outlier_channels", seed=33)
    wp1 = mx.mx_prepare_weight(dev_bf16(_one_hot_weight(N, K, k0)))
    wst = torch.cat([wp1] * E)
    monkeypatch.setenv("MX_GROUPED_CONFIG", cfg)
    out = torch.full((R + 2, N), -3.0, dtype=torch.bfloat16, device="cuda")
    mx.mx_a4w4_gemm_grouped(dev_bf16(a), torch.from_numpy(row_token).cuda(), torch.from_numpy(offs).cuda(), E, R,
                            wst, N, rows_hint=40, out=out[:R])
    torch.cuda.synchronize()
    c = host_bits(out)
    assert np.all(O.bf16_to_f64(c[R:]) == -3.0), f"{cfg}: rows past R were written"
    qa, sa = O.quantize_mx(a)
    want = O.dequantize_mx(qa, sa)[row_token][:, k0:k0 + N]
    got = O.bf16_to_f64(c[:R])
    assert np.array_equal(got, want), f"{cfg}: {int((got != want).sum())} elements differ"
