"""Pins of the A16WFP4 oracle (oracle/mx_oracle.py: gemm_a16w4_ref) to facts outside it:
it reduces exactly to the (separately pinned) A4W4 oracle when the activations are already
MXFP4 values; a brute-force sum in exact rationals decoded from bit fields; a one-hot
activation row reproduces the decoded weight column; power-of-two scaling and negation."""
from fractions import Fraction

import numpy as np

import workloads as W
from oracle import mx_oracle as O


def _bf16_exact(bits: int) -> Fraction:
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0:
        return sign * Fraction(m, 1 << 7) * Fraction(2) ** -126
    return sign * (1 + Fraction(m, 1 << 7)) * Fraction(2) ** (e - 127)


def test_reduces_to_a4w4_when_activations_are_mxfp4():
    K, N, M = 256, 64, 8
    w = W.dense_weight(N, K, seed=61)
    qa, sa = W.mx_bytes(M, K, seed=62, scale_lo=120, scale_hi=130)
    a_vals = O.dequantize_mx(qa, sa)                       # representable in bf16 at these scales
    a_bits = W.f32_to_bf16_bits(a_vals.astype(np.float32))
    assert np.array_equal(O.bf16_to_f64(a_bits), a_vals)
    qw, sw = O.quantize_mx(w)
    assert np.array_equal(O.gemm_a16w4_ref(a_bits, w), O.gemm_from_mx(qa, sa, qw, sw))


def test_brute_force_rational():
    K, N, M = 64, 3, 2
    a = W.dense_activation(M, K, "plain", seed=63)
    w = W.dense_weight(N, K, seed=64)
    qw, sw = O.quantize_mx(w)
    codes = O.unpack_codes(qw)
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
    got = O.gemm_a16w4_ref(a, w)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for k in range(K):
                c = int(codes[n, k])
                wv = mags[c & 7] * Fraction(2) ** (int(sw[n, k // 32]) - 127) * (-1 if c & 8 else 1)
                tot += _bf16_exact(int(a[m, k])) * wv
            assert got[m, n] == float(tot)


def test_one_hot_scaling_negation():
    K, N = 128, 32
    w = W.dense_weight(N, K, seed=65)
    qw, sw = O.quantize_mx(w)
    deq = O.dequantize_mx(qw, sw)
    onehot = np.zeros((3, K), dtype=np.uint16)
    for i, k in enumerate((0, 57, 127)):
        onehot[i, k] = 0x3F80                              # bf16 1.0
    assert np.array_equal(O.gemm_a16w4_ref(onehot, w), deq[:, [0, 57, 127]].T)
    a = W.dense_activation(4, K, "plain", seed=66)
    c = O.gemm_a16w4_ref(a, w)
    a8 = (a.astype(np.uint32) + (3 << 7)).astype(np.uint16)   # x 2^3 (normal values, no overflow)
    assert np.array_equal(O.gemm_a16w4_ref(a8, w), 8.0 * c)
    assert np.array_equal(O.gemm_a16w4_ref(a ^ 0x8000, w), -c)
