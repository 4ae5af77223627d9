"""Pins for the CPU oracle: checks against what the format definition and the
mathematics fix, never against the oracle's own formulas retyped.

Format: MXFP4 = E2M1 elements with one E8M0 scale per 32 elements ("[gfx950]
[FlyDSL] Add direct dense A4W4 MXFP4 GEMM", Summary), block exponent
floor(log2 amax) - 2 with round-to-nearest-even, saturating element conversion
(OCP Microscaling v1.0 conversion of a block of scalars).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import mx_oracle as O
from workloads import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")


# ------------------------------------------------------------------ helpers written from the definition

def e2m1_value_from_bitfields(code: int) -> Fraction:
    """E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is subnormal."""
    s = (code >> 3) & 1
    E = (code >> 1) & 3
    m = code & 1
    if E == 0:
        mag = Fraction(m, 2)
    else:
        mag = Fraction(2) ** (E - 1) * (1 + Fraction(m, 2))
    return -mag if s else mag


def threshold_code(mag: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even onto {0,.5,1,1.5,2,3,4,6} via its decision thresholds.

    Midpoints between neighbours are 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5; at a
    midpoint the even code wins, so the comparison is strict where the lower
    neighbour has the even code and inclusive where the upper one does.
    """
    m = np.asarray(mag, dtype=np.float64)
    return ((m > 0.25).astype(np.int64) + (m >= 0.75) + (m > 1.25) + (m >= 1.75)
            + (m > 2.5) + (m >= 3.5) + (m > 5.0))


def bits_of(values):
    out = []
    for v in values:
        if v == "-0":
            out.append(0x8000)
        else:
            f = np.float32(v)
            b = int(f32_to_bf16_bits(np.array([f]))[0])
            assert float(O.bf16_to_f64(np.array([b], dtype=np.uint16))[0]) == float(v), v
            out.append(b)
    return out


def all_finite_bf16() -> np.ndarray:
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (b >> 7) & 0xFF
    return b[exp != 0xFF]


# ------------------------------------------------------------------ E2M1 decode table

def test_e2m1_table_matches_bitfield_definition():
    codes = np.arange(16, dtype=np.uint8)
    got = O.e2m1_decode(codes)
    for c in range(16):
        assert Fraction(float(got[c])) == e2m1_value_from_bitfields(c), c
    # the eight magnitudes, and code 8 is negative zero
    assert [float(x) for x in got[:8]] == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert math.copysign(1.0, float(got[8])) == -1.0


# ------------------------------------------------------------------ hand-worked blocks

def _golden_blocks():
    with open(GOLDEN) as f:
        return json.load(f)["blocks"]


@pytest.mark.parametrize("blk", _golden_blocks(), ids=lambda b: b["name"])
def test_hand_worked_blocks(blk):
    if "bits" in blk:
        head = [int(x, 16) for x in blk["bits"]]
    else:
        head = bits_of(blk["values"])
    bits = np.zeros((1, 32), dtype=np.uint16)
    bits[0, :len(head)] = head
    q, s = O.quantize_mx(bits)
    assert int(s[0, 0]) == blk["scale"]
    codes = O.unpack_codes(q)[0]
    assert [int(c) for c in codes[:len(blk["codes_head"])]] == blk["codes_head"]
    assert np.all(codes[max(len(head), len(blk["codes_head"])):] == 0)
    if "payload_hex" in blk:
        assert q[0].tobytes().hex() == blk["payload_hex"]


# ------------------------------------------------------------------ exhaustive encoder

def test_element_encoder_exhaustive_against_thresholds():
    """Every finite bf16 value at every unclamped block exponent."""
    xb = all_finite_bf16()
    x = O.bf16_to_f64(xb)
    neg = (xb & 0x8000) != 0
    for e in range(-127, 126):
        q = np.ldexp(x, -e)
        got = O.encode_e2m1(q, neg)
        want = threshold_code(np.abs(q)) | (neg.astype(np.int64) << 3)
        assert np.array_equal(got.astype(np.int64), want), e


def test_quantizer_exhaustive_with_anchor_blocks():
    """Whole quantizer (amax, exponent, scaling, rounding, packing).

    Every finite bf16 x with |x| < 2^(e+3) is placed in a block whose last
    element is the anchor 2^(e+2), so the block exponent must be e; the code of
    x must then be the threshold rounding of x * 2^-e.
    """
    xb = all_finite_bf16()
    x = O.bf16_to_f64(xb)
    for e in range(-127, 126, 3):
        sel = np.abs(x) < 2.0 ** (e + 3)
        xs, xsb = x[sel], xb[sel]
        n = xs.size
        nblk = -(-n // 31)
        blocks = np.zeros((nblk, 32), dtype=np.uint16)
        flat = np.zeros(nblk * 31, dtype=np.uint16)
        flat[:n] = xsb
        blocks[:, :31] = flat.reshape(nblk, 31)
        anchor = f32_to_bf16_bits(np.array([2.0 ** (e + 2)], dtype=np.float32))[0]
        blocks[:, 31] = anchor
        q, s = O.quantize_mx(blocks)
        assert np.all(s[:, 0] == e + 127), e
        codes = O.unpack_codes(q)[:, :31].reshape(-1)[:n].astype(np.int64)
        want = threshold_code(np.abs(np.ldexp(xs, -e))) | (((xsb & 0x8000) != 0).astype(np.int64) << 3)
        assert np.array_equal(codes, want), e
        # the anchor itself is 4.0 -> code 6
        assert np.all(O.unpack_codes(q)[:, 31] == 6)


# ------------------------------------------------------------------ scale rule and invariants

def _random_wide_blocks(rng, nblk):
    """Blocks with a wide spread of magnitudes (exponents -140..+125) and random zeros."""
    mant = rng.standard_normal((nblk, 32)).astype(np.float32)
    expo = rng.integers(-135, 120, size=(nblk, 1))
    spread = rng.integers(0, 12, size=(nblk, 32))
    x = np.ldexp(mant, (expo - spread).astype(np.int32)).astype(np.float32)
    x[rng.random((nblk, 32)) < 0.1] = 0.0
    return f32_to_bf16_bits(x)


def test_scale_is_unique_exponent_putting_amax_in_4_to_8():
    rng = np.random.default_rng(7)
    bits = _random_wide_blocks(rng, 4000)
    q, s = O.quantize_mx(bits)
    vals = O.bf16_to_f64(bits)
    codes = O.unpack_codes(q)
    for i in range(bits.shape[0]):
        amax = Fraction(float(np.max(np.abs(vals[i]))))
        e = int(s[i, 0]) - 127
        if amax == 0:
            assert e == -127
            continue
        if amax >= Fraction(2) ** -125:
            # unclamped: amax * 2^-e in [4, 8), and the largest code is 4 or 6
            assert Fraction(4) <= amax * Fraction(2) ** (-e) < Fraction(8), i
            assert int((codes[i] & 7).max()) in (6, 7), i
        else:
            assert e == -127, i
    dec = O.dequantize_mx(q, s)
    assert np.all(np.abs(dec) <= 6.0 * np.ldexp(1.0, (s.astype(np.int64) - 127)).repeat(32, axis=1))


def test_decoded_value_is_nearest_representable():
    """Brute force over all 16 codes with exact arithmetic (ties to even code)."""
    rng = np.random.default_rng(11)
    bits = _random_wide_blocks(rng, 300)
    q, s = O.quantize_mx(bits)
    codes = O.unpack_codes(q)
    vals = O.bf16_to_f64(bits)
    table = [e2m1_value_from_bitfields(c) for c in range(16)]
    for i in range(bits.shape[0]):
        scale = Fraction(2) ** (int(s[i, 0]) - 127)
        for k in range(32):
            v = Fraction(float(vals[i, k]))
            neg = bool(bits[i, k] & 0x8000)
            cands = [c for c in range(16) if bool(c & 8) == neg]
            dist = {c: abs(v - table[c] * scale) for c in cands}
            dmin = min(dist.values())
            best = [c for c in cands if dist[c] == dmin]
            want = min(best, key=lambda c: ((c & 7) % 2, c))
            assert int(codes[i, k]) == want, (i, k, float(v))


def test_roundtrip_of_representable_blocks_is_exact():
    rng = np.random.default_rng(3)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    for _ in range(200):
        e = int(rng.integers(-120, 120))
        v = mags[rng.integers(0, 8, 32)] * np.where(rng.random(32) < 0.5, -1, 1)
        v[rng.integers(0, 32)] = rng.choice([4.0, 6.0])  # amax in [4, 8)
        x = np.ldexp(v, e).astype(np.float32)
        bits = f32_to_bf16_bits(x)[None, :]
        q, s = O.quantize_mx(bits)
        assert int(s[0, 0]) == e + 127
        assert np.array_equal(O.dequantize_mx(q, s)[0], np.ldexp(v, e))


def test_power_of_two_scaling_and_negation():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    bits = f32_to_bf16_bits(x)
    q, s = O.quantize_mx(bits)
    for j in (-9, -1, 1, 13):
        q2, s2 = O.quantize_mx(f32_to_bf16_bits(np.ldexp(x, j).astype(np.float32)))
        assert np.array_equal(q2, q)
        assert np.array_equal(s2.astype(int), s.astype(int) + j)
    qn, sn = O.quantize_mx(bits ^ np.uint16(0x8000))
    assert np.array_equal(sn, s)
    assert np.array_equal(O.unpack_codes(qn), O.unpack_codes(q) ^ 8)


def test_nonfinite_rejected():
    bits = np.zeros((1, 32), dtype=np.uint16)
    bits[0, 3] = 0x7F80  # +inf
    with pytest.raises(ValueError):
        O.quantize_mx(bits)


# ------------------------------------------------------------------ GEMM

def _fraction_gemm_from_codes(qa, sa, qw, sw):
    """Exact sum of products, decoding each element from its bit fields."""
    ca, cw = O.unpack_codes(qa), O.unpack_codes(qw)
    M, K = ca.shape
    N = cw.shape[0]
    table = [e2m1_value_from_bitfields(c) for c in range(16)]
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                sa_ = Fraction(2) ** (int(sa[m, k // 32]) - 127)
                sw_ = Fraction(2) ** (int(sw[n, k // 32]) - 127)
                acc += table[ca[m, k]] * sa_ * table[cw[n, k]] * sw_
            out[m][n] = acc
    return out


@pytest.mark.parametrize("seed,wide", [(0, False), (1, True)])
def test_gemm_matches_exact_fraction_sum(seed, wide):
    rng = np.random.default_rng(seed)
    M, N, K = 3, 5, 128
    a = rng.standard_normal((M, K)).astype(np.float32)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    if wide:
        a = np.ldexp(a, rng.integers(-20, 20, size=(M, K // 32)).repeat(32, axis=1)).astype(np.float32)
    ab, wb = f32_to_bf16_bits(a), f32_to_bf16_bits(w)
    got = O.gemm_ref(ab, wb)
    qa, sa = O.quantize_mx(ab)
    qw, sw = O.quantize_mx(wb)
    want = _fraction_gemm_from_codes(qa, sa, qw, sw)
    for m in range(M):
        for n in range(N):
            assert Fraction(float(got[m, n])) == want[m][n]


def test_gemm_wide_spread_takes_exact_path():
    """Exponent spread beyond float64's exact range: result still exact."""
    a = np.zeros((1, 64), dtype=np.float32)
    a[0, 0] = 2.0 ** 100
    a[0, 32] = 2.0 ** -100
    w = np.ones((1, 64), dtype=np.float32)
    qa, sa = O.quantize_mx(f32_to_bf16_bits(a))
    qw, sw = O.quantize_mx(f32_to_bf16_bits(w))
    assert not O._assert_exact(qa, sa, qw, sw, 64)
    got = O.gemm_ref(f32_to_bf16_bits(a), f32_to_bf16_bits(w))
    # both nonzero blocks are exactly representable; the sum is rounded once
    assert float(got[0, 0]) == float(Fraction(2) ** 100 + Fraction(2) ** -100)


@pytest.mark.parametrize("K", [256, 768, 4224])
def test_constant_probe(K):
    """A = 1, W = 1: every block has amax 1 -> exact, so C = K."""
    ones_a = np.full((2, K), 0x3F80, dtype=np.uint16)
    ones_w = np.full((256, K), 0x3F80, dtype=np.uint16)
    c = O.gemm_ref(ones_a, ones_w)
    assert np.all(c == K)


def test_one_hot_weight_probe_selects_quantized_activation_columns():
    """W[n, k0 + n] = 1 makes C[:, n] the decoded A element at column k0 + n."""
    rng = np.random.default_rng(2)
    M, N, K, k0 = 5, 256, 512, 128
    ab = f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = np.zeros((N, K), dtype=np.float32)
    w[np.arange(N), k0 + np.arange(N)] = 1.0
    c = O.gemm_ref(ab, f32_to_bf16_bits(w))
    qa, sa = O.quantize_mx(ab)
    ca = O.unpack_codes(qa)
    for m in range(M):
        for n in range(N):
            k = k0 + n
            want = e2m1_value_from_bitfields(int(ca[m, k])) * Fraction(2) ** (int(sa[m, k // 32]) - 127)
            assert Fraction(float(c[m, n])) == want


def test_one_hot_activation_probe_selects_weight_rows():
    """A[m, k0 + m] = 1 makes C[m, :] the decoded W elements at column k0 + m."""
    rng = np.random.default_rng(4)
    M, N, K, k0 = 16, 256, 256, 64
    wb = f32_to_bf16_bits((0.02 * rng.standard_normal((N, K))).astype(np.float32))
    a = np.zeros((M, K), dtype=np.float32)
    a[np.arange(M), k0 + np.arange(M)] = 1.0
    c = O.gemm_ref(f32_to_bf16_bits(a), wb)
    qw, sw = O.quantize_mx(wb)
    cw = O.unpack_codes(qw)
    for m in range(M):
        k = k0 + m
        want = [e2m1_value_from_bitfields(int(cw[n, k])) * Fraction(2) ** (int(sw[n, k // 32]) - 127)
                for n in range(N)]
        assert [Fraction(float(x)) for x in c[m]] == want


def test_gemm_scaling_and_negation_are_exact():
    rng = np.random.default_rng(9)
    a = rng.standard_normal((4, 256)).astype(np.float32)
    wb = f32_to_bf16_bits((0.02 * rng.standard_normal((256, 256))).astype(np.float32))
    c = O.gemm_ref(f32_to_bf16_bits(a), wb)
    c2 = O.gemm_ref(f32_to_bf16_bits(np.ldexp(a, 5).astype(np.float32)), wb)
    assert np.array_equal(c2, 32.0 * c)
    cn = O.gemm_ref(f32_to_bf16_bits(-a), wb)
    assert np.array_equal(cn, -c)


def test_sampled_gemm_equals_full():
    rng = np.random.default_rng(12)
    ab = f32_to_bf16_bits(rng.standard_normal((9, 256)).astype(np.float32))
    wb = f32_to_bf16_bits((0.02 * rng.standard_normal((256, 256))).astype(np.float32))
    full = O.gemm_ref(ab, wb)
    rows, cols = [0, 4, 8], [3, 100, 255]
    assert np.array_equal(O.gemm_ref_sampled(ab, wb, rows, cols), full[np.ix_(rows, cols)])


def test_grouped_reference_by_brute_force():
    rng = np.random.default_rng(13)
    T, E, topk, N, K = 3, 5, 2, 256, 128
    ab = f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    ws = {e: f32_to_bf16_bits((0.02 * rng.standard_normal((N, K))).astype(np.float32)) for e in range(E)}
    pairs = [(t, e) for t in range(T) for e in rng.choice(E, topk, replace=False)]
    pairs.sort(key=lambda p: p[1])
    row_token = np.array([t for t, _ in pairs], dtype=np.int32)
    counts = np.bincount([e for _, e in pairs], minlength=E)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    got = O.grouped_gemm_ref(ab, row_token, offs, lambda e: ws[e])
    for r, (t, e) in enumerate(pairs):
        assert np.array_equal(got[r], O.gemm_ref(ab[t:t + 1], ws[e])[0])


def test_prepared_size_matches_page_figure():
    """The page gives 32,169,984 bytes for one 8448 x 7168 MXFP4 weight
    ("[gfx950][FlyDSL] Add direct dense A4W4 MXFP4 GEMM", Model validation)."""
    assert O.prepared_weight_bytes(8448, 7168) == 32_169_984
    # and 2.786 GiB over 93 layers
    assert abs(93 * 32_169_984 / 2 ** 30 - 2.786) < 5e-4


def _bf16_fraction(bits: int) -> Fraction:
    """A bf16 bit pattern decoded from its fields (sign, 8-bit exponent, 7-bit fraction)."""
    sign = -1 if bits & 0x8000 else 1
    e, f = (bits >> 7) & 0xFF, bits & 0x7F
    if e == 0:
        return sign * Fraction(f, 128) * Fraction(2) ** -126
    return sign * (1 + Fraction(f, 128)) * Fraction(2) ** (e - 127)


def test_bf16_exact_product_against_fraction_sums():
    """gemm_bf16_exact (the unquantized reference of the relative-L2 context metric) equals
    the exact rational sum of products of the bf16 inputs decoded from their bit fields, on
    inputs whose float64 sums are exact (exponents within a narrow range, K = 32) and on a
    hand-worked case."""
    rng = np.random.default_rng(11)
    a = (rng.integers(0x3E00, 0x4080, size=(3, 32)) | (rng.integers(0, 2, size=(3, 32)) << 15)).astype(np.uint16)
    w = (rng.integers(0x3E00, 0x4080, size=(4, 32)) | (rng.integers(0, 2, size=(4, 32)) << 15)).astype(np.uint16)
    got = O.gemm_bf16_exact(a, w)
    for m in range(3):
        for n in range(4):
            want = sum((_bf16_fraction(int(x)) * _bf16_fraction(int(y)) for x, y in zip(a[m], w[n])), Fraction(0))
            assert Fraction(got[m, n]) == want
    # [1.5, -2] . [0.25, 3] = 0.375 - 6 = -5.625 (0x3FC0 = 1.5, 0xC000 = -2, 0x3E80 = 0.25, 0x4040 = 3)
    hand = O.gemm_bf16_exact(np.array([[0x3FC0, 0xC000]], dtype=np.uint16), np.array([[0x3E80, 0x4040]], dtype=np.uint16))
    assert hand.tolist() == [[-5.625]]
    # a transposed operand would not even have the right shape
    assert O.gemm_bf16_exact(a, w).shape == (3, 4)


def test_relative_l2_hand_values():
    """rel_l2(x, ref) = ||x - ref||_2 / ||ref||_2: hand-worked values, the argument order, and the
    zero-reference convention."""
    assert O.rel_l2(np.array([3.6, 4.8]), np.array([3.0, 4.0])) == pytest.approx(0.2, abs=1e-15)
    assert O.rel_l2(np.zeros(4), np.array([1.0, 0.0, 0.0, 0.0])) == 1.0
    assert O.rel_l2(np.array([2.0, 0.0]), np.array([1.0, 0.0])) == 1.0
    assert O.rel_l2(np.array([1.0, 0.0]), np.array([2.0, 0.0])) == 0.5   # not symmetric
    assert O.rel_l2(np.ones(3), np.zeros(3)) == 0.0                      # zero reference: defined as 0
