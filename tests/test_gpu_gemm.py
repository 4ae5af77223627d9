"""GPU parity of the dense A4W4 GEMM against the CPU oracle, at every workload point,
plus exact probes and invariants.

Tolerance (per element): |gpu - exact| <= 2^-7 |exact| + 1e-3 rms(exact). At full size
the oracle computes a sample of rows (first, last and a spread) over every column; rms is
taken over those sampled rows.
"""
import numpy as np
import pytest

import workloads as W
from oracle import mx_oracle as O

from gpu_util import (check_gemm, dense_activation_cached, dense_weight_cached, dev_bf16, host_bits,
                      lib_or_fail, sample_rows, torch_or_skip)

pytestmark = pytest.mark.gpu

POINTS = [("smoke_16x256x256", 16)]
for _name, (_N, _K, _ms, _s) in W.DENSE_CONFIGS.items():
    if _name != "smoke_16x256x256":
        POINTS += [(_name, m) for m in _ms]

_prepared = {}


def prepared(name):
    mx = lib_or_fail()
    if name not in _prepared:
        w, _, _ = dense_weight_cached(name)
        _prepared[name] = mx.mx_prepare_weight(dev_bf16(w))
    return _prepared[name]


def run_gemm(a_bits, wp, N):
    mx = lib_or_fail()
    return mx.mx_a4w4_gemm(dev_bf16(a_bits), wp, N)


@pytest.mark.parametrize("name,M", POINTS, ids=[f"{n}-M{m}" for n, m in POINTS])
def test_gemm_matches_oracle(name, M):
    torch = torch_or_skip()
    N, K, _, _ = W.DENSE_CONFIGS[name]
    a = dense_activation_cached(name, M)
    _, qw, sw = dense_weight_cached(name)
    c = host_bits(run_gemm(a, prepared(name), N))
    torch.cuda.synchronize()
    rows = sample_rows(M)
    qa, sa = O.quantize_mx(a[rows])
    exact = O.gemm_from_mx(qa, sa, qw, sw)
    check_gemm(c[rows], exact, what=f"{name} M={M}")


def test_one_hot_weight_probe_is_exact():
    """W[n, k0 + n] = 1 (decodes to exactly 1.0) makes C[:, n] the decoded activation at
    column k0 + n: the inline quantization is checked bit for bit through the GEMM."""
    torch = torch_or_skip()
    mx = lib_or_fail()
    N, K, k0 = 256, 768, 320
    for M in (1, 7, 32, 100):
        a = dense_activation_cached("n7168_k768", 2048)[:M]
        w = np.zeros((N, K), dtype=np.uint16)
        w[np.arange(N), k0 + np.arange(N)] = 0x3F80
        c = host_bits(mx.mx_a4w4_gemm(dev_bf16(a), mx.mx_prepare_weight(dev_bf16(w)), N))
        torch.cuda.synchronize()
        qa, sa = O.quantize_mx(a)
        want = O.dequantize_mx(qa, sa)[:, k0:k0 + N]
        assert np.array_equal(O.bf16_to_f64(c), want), M


def test_one_hot_activation_probe_is_exact():
    """A[m, k0 + m] = 1 makes C[m, :] the decoded weight column k0 + m: prepare, the
    preshuffle and the weight-scale plumbing are checked without knowing the layout."""
    torch = torch_or_skip()
    mx = lib_or_fail()
    name = "n7168_k4224"
    N, K, _, _ = W.DENSE_CONFIGS[name]
    _, qw, sw = dense_weight_cached(name)
    w_hat = O.dequantize_mx(qw, sw)
    for M, k0 in ((16, 4096), (48, 1000 - 1000 % 32), (3, 0)):
        a = np.zeros((M, K), dtype=np.uint16)
        a[np.arange(M), k0 + np.arange(M)] = 0x3F80
        c = host_bits(mx.mx_a4w4_gemm(dev_bf16(a), prepared(name), N))
        torch.cuda.synchronize()
        assert np.array_equal(O.bf16_to_f64(c), w_hat[:, k0:k0 + M].T), (M, k0)


@pytest.mark.parametrize("K", [768, 4224, 7168])
def test_constant_probe(K):
    torch = torch_or_skip()
    mx = lib_or_fail()
    N = 256
    wp = mx.mx_prepare_weight(dev_bf16(np.full((N, K), 0x3F80, dtype=np.uint16)))
    for M in (1, 33, 130):
        c = host_bits(mx.mx_a4w4_gemm(dev_bf16(np.full((M, K), 0x3F80, dtype=np.uint16)), wp, N))
        torch.cuda.synchronize()
        assert np.all(O.bf16_to_f64(c) == K), (K, M)


@pytest.mark.parametrize("M", [1, 17, 100, 512])
def test_scaling_negation_and_determinism(M):
    torch = torch_or_skip()
    mx = lib_or_fail()
    name = "n1536_k7168"
    N = 1536
    a = dense_activation_cached(name, 2048)[:M]
    wp = prepared(name)
    base = host_bits(mx.mx_a4w4_gemm(dev_bf16(a), wp, N))
    again = host_bits(mx.mx_a4w4_gemm(dev_bf16(a), wp, N))
    assert np.array_equal(base, again), "run-to-run bitwise determinism"
    neg = host_bits(mx.mx_a4w4_gemm(dev_bf16(a ^ np.uint16(0x8000)), wp, N))
    assert np.array_equal(neg, base ^ np.uint16(0x8000)) or np.array_equal(
        O.bf16_to_f64(neg), -O.bf16_to_f64(base)), "negation"
    # x * 2^3: exponent field + 3 for every nonzero input (no input is near overflow)
    ab = a.astype(np.uint32)
    nz = (ab & 0x7F80) != 0
    scaled = np.where(nz, ab + (3 << 7), ab).astype(np.uint16)
    sc = host_bits(mx.mx_a4w4_gemm(dev_bf16(scaled), wp, N))
    torch.cuda.synchronize()
    assert np.array_equal(O.bf16_to_f64(sc), 8.0 * O.bf16_to_f64(base)), "power-of-two scaling"


def test_m_tail_prefix_and_canary():
    """Rows >= M are never written, and a prefix of the input gives a prefix of the output
    (for M values served by the same kernel family)."""
    torch = torch_or_skip()
    mx = lib_or_fail()
    name = "n7168_k4224"
    N, K, _, _ = W.DENSE_CONFIGS[name]
    wp = prepared(name)
    a_all = dense_activation_cached(name, 2048)
    outs = {}
    for M in (3, 17, 32, 100, 128, 512):
        c = torch.full((M + 5, N), -7.0, dtype=torch.bfloat16, device="cuda")
        mx.mx_a4w4_gemm(dev_bf16(a_all[:M]), wp, N, out=c[:M])
        cb = host_bits(c)
        assert np.all(cb[M:] == host_bits(torch.full((1,), -7.0, dtype=torch.bfloat16))[0]), M
        outs[M] = cb[:M]
    assert np.array_equal(outs[17][:3], outs[3])
    assert np.array_equal(outs[32][:17], outs[17])
    assert np.array_equal(outs[128][:100], outs[100])
    assert np.array_equal(outs[512][:128], outs[128])


def test_all_zero_and_negative_zero_blocks():
    torch = torch_or_skip()
    mx = lib_or_fail()
    name = "n1536_k7168"
    N, K, _, _ = W.DENSE_CONFIGS[name]
    a = np.zeros((2, K), dtype=np.uint16)
    a[1] = 0x8000
    c = host_bits(mx.mx_a4w4_gemm(dev_bf16(a), prepared(name), N))
    torch.cuda.synchronize()
    assert np.all(O.bf16_to_f64(c) == 0.0)


# Shapes off the benchmark sweep that take the size-dependent choices: 17..32 rows against many
# column groups at a K whose slices are uneven (N=8192, K=4096: five slices of 7, 7, 7, 7 and
# 4 steps), and the four-wave 128 x 48 tiles over two and three row tiles.
OFF_SWEEP = [
    (24, 8192, 4096, "k_gemm_tile<1, 4, 4, 4, 2, 2> GM=8 S=5 + k_splitk_reduce"),
    (200, 4096, 4224, "k_prepare + k_gemm_qk<8, 3, 4> GM=2"),
    (384, 2048, 7168, "k_prepare + k_gemm_qk<8, 3, 4> GM=3"),
]


@pytest.mark.parametrize("M,N,K,plan", OFF_SWEEP, ids=[f"{m}x{n}x{k}" for m, n, k, _ in OFF_SWEEP])
def test_size_dependent_plans_match_oracle(M, N, K, plan):
    torch = torch_or_skip()
    mx = lib_or_fail()
    assert mx.mx_a4w4_gemm_plan(M, N, K) == plan
    w = W.dense_weight(N, K)
    a = W.dense_activation(M, K, "zero_blocks")
    c = host_bits(mx.mx_a4w4_gemm(dev_bf16(a), mx.mx_prepare_weight(dev_bf16(w)), N))
    torch.cuda.synchronize()
    rows = sample_rows(M)
    qa, sa = O.quantize_mx(a[rows])
    qw, sw = O.quantize_mx(w)
    check_gemm(c[rows], O.gemm_from_mx(qa, sa, qw, sw), what=f"{M}x{N}x{K}")
