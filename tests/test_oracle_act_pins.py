"""Pins of the fused-activation oracle (oracle/mx_act_oracle.py) to facts outside itself:
closed forms and identities of SiLU, the gate/up column convention of SwiGLU on a one-hot
output, agreement of the value quantizer with the (separately pinned) bf16 quantizer on
bf16-representable values, a brute-force GEMM1 row in exact rational arithmetic, and the
validity check accepting the exact quantization while rejecting planted mistakes."""
from fractions import Fraction
import math

import numpy as np
import pytest

import workloads as W
from oracle import mx_act_oracle as A
from oracle import mx_oracle as O


def test_silu_closed_forms():
    assert A.silu(0.0) == 0.0
    assert A.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)   # 0.7310585786300049
    assert A.silu(1.0) == pytest.approx(0.7310585786300049, rel=1e-15)
    x = np.random.default_rng(1).normal(0, 4, 1000)
    # SiLU(x) - SiLU(-x) = x (sigmoid(x) + sigmoid(-x) = 1)
    assert np.allclose(A.silu(x) - A.silu(-x), x, rtol=0, atol=1e-12)
    assert A.silu(60.0) == pytest.approx(60.0, rel=1e-15)
    assert abs(A.silu(-60.0)) < 1e-24


def test_silu_minimum_constant():
    x = A.SILU_ARGMIN
    sig = 1.0 / (1.0 + math.exp(-x))
    assert abs(1.0 + x * (1.0 - sig)) < 1e-14                   # stationary point
    grid = np.linspace(-10, 10, 200001)
    assert A.silu(x) <= A.silu(grid).min() + 1e-15               # the global minimum
    assert A.silu(x) == pytest.approx(-0.2784645427610738, rel=1e-12)


def test_swiglu_column_convention_one_hot():
    N = 256
    c = np.zeros((2, N))
    c[0, 3] = 2.0            # gate column 3
    c[0, N // 2 + 3] = 5.0   # its up column
    c[1, N // 2 + 7] = 9.0   # up without gate: silu(0) * 9 = 0
    h = A.activation(c, A.ACT_SWIGLU)
    assert h.shape == (2, N // 2)
    assert h[0, 3] == pytest.approx(5.0 * 2.0 / (1.0 + math.exp(-2.0)), rel=1e-15)
    h[0, 3] = 0.0
    assert np.all(h == 0.0)
    g = np.random.default_rng(2).normal(size=(3, N // 2))
    assert np.array_equal(A.activation(np.hstack([g, np.ones_like(g)]), A.ACT_SWIGLU), A.silu(g))
    assert np.array_equal(A.activation(g, A.ACT_SILU), A.silu(g))


def test_value_quantizer_matches_bf16_quantizer():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 1 << 16, size=(64, 256), dtype=np.uint16)
    bits = bits[~np.any(((bits >> 7) & 0xFF) == 0xFF, axis=1)]       # finite rows only
    special = np.zeros((4, 256), dtype=np.uint16)
    special[1, :32] = 0x8000                                          # all -0.0
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, -0.25, -2.5, -5.0], dtype=np.float32)
    special[2, :ties.size] = (ties.view(np.uint32) >> 16).astype(np.uint16)
    special[3, :] = 0x0001                                            # bf16 subnormals
    bits = np.vstack([bits, special])
    vals = O.bf16_to_f64(bits)
    vals = np.where((bits & 0x8000) != 0, np.copysign(np.abs(vals), -1.0), vals)   # keep -0.0
    q1, s1 = O.quantize_mx(bits)
    q2, s2 = A.quantize_mx_values(vals)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def _brute_row(a_bits_row, w_bits):
    """One GEMM1 output row from first principles: decode both operands to Fractions."""
    qa, sa = O.quantize_mx(a_bits_row[None, :])
    qw, sw = O.quantize_mx(w_bits)
    ca, cw = O.unpack_codes(qa)[0], O.unpack_codes(qw)
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]

    def val(code, s):
        v = mags[code & 7] * (Fraction(2) ** (int(s) - 127))
        return -v if code & 8 else v
    K = a_bits_row.size
    av = [val(ca[k], sa[0, k // 32]) for k in range(K)]
    return [float(sum(av[k] * val(cw[n, k], sw[n, k // 32]) for k in range(K))) for n in range(w_bits.shape[0])]


def test_grouped_act_ref_brute_force_and_intervals():
    K, N, E = 128, 64, 3
    a = W.dense_activation(5, K, "plain", seed=7)
    ws = {e: W.dense_weight(N, K, seed=70 + e) for e in range(E)}
    offs = np.array([0, 2, 2, 5], dtype=np.int32)      # expert 1 has no rows
    row_token = np.array([4, 0, 1, 3, 2], dtype=np.int32)
    h, lo, hi = A.grouped_gemm1_act_ref(a, row_token, offs, lambda e: ws[e], A.ACT_SWIGLU)
    assert h.shape == (5, N // 2)
    expert = [0, 0, 2, 2, 2]
    for r in range(5):
        c = np.array(_brute_row(a[row_token[r]], ws[expert[r]]))
        assert np.allclose(h[r], A.silu(c[:N // 2]) * c[N // 2:], rtol=1e-14, atol=1e-300)
    assert np.all(lo <= h) and np.all(h <= hi)
    assert np.all(hi - lo <= 1e-2 * np.abs(h) + 1e-3 * np.sqrt(np.mean(h * h)))   # tight enough to mean something
    hs, los, his = A.grouped_gemm1_act_ref(a, row_token, offs, lambda e: ws[e], A.ACT_SILU, rows=[1, 3])
    assert hs.shape == (2, N) and np.all(los <= hs) and np.all(hs <= his)


def test_quantization_valid_accepts_exact_and_rejects_mistakes():
    rng = np.random.default_rng(5)
    h = rng.normal(0, 3, size=(8, 128))
    lo, hi = h - 1e-9 * np.abs(h), h + 1e-9 * np.abs(h)
    q, s = A.quantize_mx_values(h)
    so, co = A.quantization_valid(q, s, lo, hi)
    assert so.all() and co.all()
    # a flipped sign on a large element
    i = np.unravel_index(np.argmax(np.abs(h)), h.shape)
    q2 = q.copy()
    q2[i[0], i[1] // 2] ^= 0x8 << (4 * (i[1] % 2))
    assert not A.quantization_valid(q2, s, lo, hi)[1].all()
    # a scale one too large for a block whose amax is far from a power of two
    s2 = s.copy()
    s2[0, 0] += 1
    assert not A.quantization_valid(q, s2, lo, hi)[0].all()
    # gate and up swapped
    c = rng.normal(0, 2, size=(8, 256))
    hw = A.activation(np.hstack([c[:, 128:], c[:, :128]]), A.ACT_SWIGLU)
    hr = A.activation(c, A.ACT_SWIGLU)
    qw, sw = A.quantize_mx_values(hw)
    so, co = A.quantization_valid(qw, sw, hr - 1e-9 * np.abs(hr), hr + 1e-9 * np.abs(hr))
    assert co.mean() < 0.7
    # an interval straddling a rounding tie admits both neighbours: 1.25 lies between codes 1.0 and 1.5
    t = np.zeros((1, 32))
    t[0, 0], t[0, 1] = 1.25, 4.0                   # amax 4 -> scale 2^0
    qa_, sa_ = A.quantize_mx_values(t)             # 1.25 -> 1.0 (tie to even)
    tl, th = t.copy(), t.copy()
    tl[0, 0], th[0, 0] = 1.2, 1.3
    assert A.quantization_valid(qa_, sa_, tl, th)[1].all()
    up = qa_.copy()
    up[0, 0] = (up[0, 0] & 0xF0) | 3               # code 3 = 1.5: the other neighbour
    assert A.quantization_valid(up, sa_, tl, th)[1].all()
    far = qa_.copy()
    far[0, 0] = (far[0, 0] & 0xF0) | 4             # 2.0 lies outside [1.2, 1.3]
    assert not A.quantization_valid(far, sa_, tl, th)[1].all()
