"""CPU oracle for the inline-quantized A4W4 MXFP4 GEMM.

TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the bench's
CPU-baseline leg are the only callers; the product library never imports,
links or runs anything here, and this package imports nothing from it.

What is computed, and where it is stated:

* "[gfx950][FlyDSL] Add direct dense A4W4 MXFP4 GEMM", Summary: BF16
  activations are quantized to MXFP4 (E2M1 elements with E8M0 scales) and
  multiplied against MXFP4 weights (packed E2M1 with E8M0 scales).
* Same page, Scope: N divisible by 256, K divisible by 128.
* "[gfx1250] Fuse A4W4 stage1 FP4 quantization", Summary: the E8M0 scale is
  computed from the value itself.
* The block-scale and element-conversion rules come from the OCP Microscaling
  (MX) v1.0 conversion of a block of scalars: shared exponent
  floor(log2(amax)) minus the largest exponent of the element format (2 for
  E2M1), elements converted with round-to-nearest-even and saturation.

The pages leave several steps open; the readings taken are:

1. Scale rule: e = floor(log2 amax) - 2, clamped to [-127, 127]; the page's
   "ceil-based scale accounting" is read as ceil-division sizing of scale
   buffers, not a ceil exponent rule.
2. An all-zero block gets e = -127 (scale byte 0).
3. The sign bit of an element is the sign bit of the input, so -0.0 and
   negative values that round to zero encode as 0x8.
4. Ties go to the even code; magnitudes at or above 6 saturate to 6.
5. Nibble order: the element at even k is the low nibble of its byte.
6. Weights are quantized with the same rule as activations, blocks along K.
7. Non-finite inputs are outside the contract and raise ValueError.

The GEMM result is the exact real sum of the dequantized products, evaluated
in float64 (exact under the exponent-spread guard in ``_assert_exact``).

The MoE layer's second GEMM and combine ("[HIP] [CK] [FlyDSL] [Kernel] Extend
MXFP4 GEMM1 replacement to A4W4", Summary: the stage-2 GEMM that follows GEMM1)
are read as follows, the pages giving no more than that stage's existence:

8. GEMM2 takes its activation rows already in MXFP4 (canonical payload and
   scales, as GEMM1's fused epilogue or the standalone quantizer emit them), in
   expert-sorted order, and multiplies row r by the quantized weight of the
   expert whose segment holds r; there is no inline quantization.
9. The combine sums each token's top-k GEMM2 rows weighted by its routing
   weights: out[t] = sum_k weights[t, k] * y[row of (t, k)]; a row index outside
   the rows contributes nothing.
10. The A16WFP4 variant ("[gfx950][FlyDSL] Add direct dense A4W4 MXFP4 GEMM",
    CI Guide: named as outside that change) keeps the activations in bf16 and
    multiplies them by the MXFP4 weight decoded to real values (no activation
    quantization).

Nothing here is blocked, fused or reordered beyond the definition: quantize
each 32-element block, decode, then one float64 matrix product.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

BLOCK = 32
# Magnitudes of E2M1 codes 0..7 (code | 8 is the negative of the same magnitude).
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E8M0_BIAS = 127
E_MIN, E_MAX = -127, 127
ELEM_EMAX = 2  # exponent of the largest E2M1 magnitude (6 = 1.5 * 2^2)


# ----------------------------------------------------------------------------- bf16

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns exactly: a bfloat16 is the top half of a float32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- E2M1 / E8M0

def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each 4-bit E2M1 code (bit 3 sign, bits 2:0 magnitude index)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def block_exponent(amax: np.ndarray) -> np.ndarray:
    """Shared block exponent e = floor(log2 amax) - 2, clamped to [-127, 127].

    floor(log2 amax) is taken exactly from frexp (amax = f * 2^p with
    f in [0.5, 1) gives floor(log2 amax) = p - 1); no floating log is used.
    amax == 0 gives -127.
    """
    a = np.asarray(amax, dtype=np.float64)
    _, p = np.frexp(a)
    e = (p.astype(np.int64) - 1) - ELEM_EMAX
    e = np.where(a == 0.0, E_MIN, e)
    return np.clip(e, E_MIN, E_MAX)


def encode_e2m1(q: np.ndarray, negative: np.ndarray) -> np.ndarray:
    """E2M1 code of scaled values q: the nearest magnitude, ties to the even code.

    Magnitudes at or above 6 first saturate to 6; the nearest of the eight
    magnitudes is then found by enumeration. ``negative`` sets bit 3.
    """
    mag = np.minimum(np.abs(np.asarray(q, dtype=np.float64)), 6.0)   # saturate
    d = np.abs(mag[..., None] - E2M1_MAGNITUDES)              # [..., 8]
    dmin = d.min(axis=-1, keepdims=True)
    best = d == dmin
    even = best & ((np.arange(8) % 2) == 0)
    pick_even = even.any(axis=-1)
    code = np.where(pick_even, np.argmax(even, axis=-1), np.argmax(best, axis=-1))
    return (code | (np.asarray(negative, dtype=bool).astype(np.int64) << 3)).astype(np.uint8)


def quantize_mx(bits: np.ndarray, chunk_rows: int | None = None):
    """Quantize bf16 rows [R, K] to MXFP4 along K.

    Returns (payload uint8 [R, K/2], scales uint8 [R, K/32]) in the canonical
    layout: row-major, low nibble = even k, one E8M0 byte per 32-element block.
    """
    b = np.asarray(bits, dtype=np.uint16)
    if b.ndim != 2 or b.shape[1] % BLOCK != 0:
        raise ValueError("expected [R, K] with K a multiple of 32")
    R, K = b.shape
    nb = K // BLOCK
    payload = np.empty((R, K // 2), dtype=np.uint8)
    scales = np.empty((R, nb), dtype=np.uint8)
    if chunk_rows is None:
        chunk_rows = max(1, (1 << 20) // max(K, 1))
    for r0 in range(0, R, chunk_rows):
        v = bf16_to_f64(b[r0:r0 + chunk_rows])
        if not np.all(np.isfinite(v)):
            raise ValueError("non-finite input is outside the MXFP4 quantizer's contract")
        neg = (b[r0:r0 + chunk_rows] & 0x8000) != 0
        vb = v.reshape(v.shape[0], nb, BLOCK)
        amax = np.abs(vb).max(axis=-1)                        # step: block amax
        e = block_exponent(amax)                              # step: shared exponent
        q = np.ldexp(vb, -e[..., None])                       # step: scale (exact)
        codes = encode_e2m1(q, neg.reshape(vb.shape))         # step: RNE + saturate
        codes = codes.reshape(v.shape[0], K)
        payload[r0:r0 + chunk_rows] = codes[:, 0::2] | (codes[:, 1::2] << 4)
        scales[r0:r0 + chunk_rows] = (e + E8M0_BIAS).astype(np.uint8)
    return payload, scales


def unpack_codes(payload: np.ndarray) -> np.ndarray:
    """Split packed bytes [R, K/2] into codes [R, K] (low nibble first)."""
    p = np.asarray(payload, dtype=np.uint8)
    codes = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    codes[:, 0::2] = p & 0x0F
    codes[:, 1::2] = p >> 4
    return codes


def dequantize_mx(payload: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode MXFP4 rows to float64: value(code) * 2^(scale - 127)."""
    codes = unpack_codes(payload)
    R, K = codes.shape
    s = np.asarray(scales, dtype=np.int64).reshape(R, K // BLOCK)
    if np.any(s == 255):
        raise ValueError("E8M0 code 255 (NaN) is never produced by the quantizer")
    vals = e2m1_decode(codes).reshape(R, K // BLOCK, BLOCK)
    return np.ldexp(vals, (s - E8M0_BIAS)[..., None]).reshape(R, K)


# ----------------------------------------------------------------------------- GEMM

def _nonzero_block_exponent_range(payload: np.ndarray, scales: np.ndarray):
    codes = unpack_codes(payload)
    R, K = codes.shape
    nz = ((codes & 7) != 0).reshape(R, K // BLOCK, BLOCK).any(axis=-1)
    if not nz.any():
        return None
    s = np.asarray(scales, dtype=np.int64)[nz]
    return int(s.min()), int(s.max())


def _assert_exact(qa, sa, qw, sw, K: int) -> bool:
    """True when every float64 partial sum of the product is exact.

    Each product of two decoded elements is an integer multiple of
    2^(ea + eb - 2) with magnitude at most 36 * 2^(ea + eb); the sum over K
    terms is exact in float64 when K * 144 * 2^spread <= 2^53, where spread is
    the range of ea + eb over nonzero blocks.
    """
    ra = _nonzero_block_exponent_range(qa, sa)
    rw = _nonzero_block_exponent_range(qw, sw)
    if ra is None or rw is None:
        return True
    spread = (ra[1] - ra[0]) + (rw[1] - rw[0])
    return K * 144 * (2.0 ** spread) <= 2.0 ** 53


def _fraction_matmul(a_hat: np.ndarray, w_hat: np.ndarray) -> np.ndarray:
    M, K = a_hat.shape
    N = w_hat.shape[0]
    out = np.empty((M, N), dtype=np.float64)
    for m in range(M):
        for n in range(N):
            out[m, n] = float(sum((Fraction(float(x)) * Fraction(float(y))
                                   for x, y in zip(a_hat[m], w_hat[n])), Fraction(0)))
    return out


def gemm_from_mx(qa, sa, qw, sw) -> np.ndarray:
    """C[m, n] = sum_k Ahat[m, k] * What[n, k] for MXFP4 operands, in float64."""
    a_hat = dequantize_mx(qa, sa)
    w_hat = dequantize_mx(qw, sw)
    K = a_hat.shape[1]
    if _assert_exact(qa, sa, qw, sw, K):
        return a_hat @ w_hat.T
    if a_hat.shape[0] * w_hat.shape[0] * K > 1 << 22:
        raise ValueError("exponent spread too wide for an exact float64 sum at this size")
    return _fraction_matmul(a_hat, w_hat)


def gemm_ref(a_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """The A4W4 GEMM: quantize A [M,K] and W [N,K] to MXFP4, then the exact product [M,N]."""
    qa, sa = quantize_mx(a_bits)
    qw, sw = quantize_mx(w_bits)
    return gemm_from_mx(qa, sa, qw, sw)


def gemm_ref_sampled(a_bits: np.ndarray, w_bits: np.ndarray, rows, cols) -> np.ndarray:
    """Selected outputs C[rows[i], cols[j]] of ``gemm_ref``.

    Quantization acts on each row of A and of W independently, so quantizing
    only the selected rows gives the same operands as quantizing everything.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    return gemm_ref(np.asarray(a_bits)[rows], np.asarray(w_bits)[cols])


def gemm_bf16_exact(a_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """Unquantized product of the bf16 inputs in float64 (context metric only)."""
    return bf16_to_f64(a_bits) @ bf16_to_f64(w_bits).T


def grouped_gemm_ref(a_bits: np.ndarray, row_token: np.ndarray, expert_offsets: np.ndarray,
                     expert_weight, rows=None) -> np.ndarray:
    """Grouped GEMM1 over expert segments.

    Output row r (in expert-sorted order) is quantized A[row_token[r]] times
    the quantized weight of the expert e whose segment
    expert_offsets[e] <= r < expert_offsets[e+1] holds r. ``expert_weight(e)``
    returns W_e [N, K] as bf16 bits. ``rows`` selects a subset of output rows.
    """
    offs = np.asarray(expert_offsets, dtype=np.int64)
    tok = np.asarray(row_token, dtype=np.int64)
    R = int(offs[-1])
    rows = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    expert_of = np.searchsorted(offs, rows, side="right") - 1
    out = None
    for e in np.unique(expert_of):
        sel = np.flatnonzero(expert_of == e)
        c = gemm_ref(np.asarray(a_bits)[tok[rows[sel]]], expert_weight(int(e)))
        if out is None:
            out = np.empty((rows.size, c.shape[1]), dtype=np.float64)
        out[sel] = c
    if out is None:
        out = np.empty((0, 0), dtype=np.float64)
    return out


def gemm_a16w4_ref(a_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """A16WFP4: the bf16 activations A [M, K], unquantized, times the MXFP4-quantized
    weight W [N, K] decoded to real values; one float64 matrix product. Each product of a
    bf16 value and a decoded E2M1 value is exact; the float64 sum's rounding (at most
    K 2^-53 sum |a w|) is negligible against any bf16-output tolerance."""
    qw, sw = quantize_mx(w_bits)
    return bf16_to_f64(a_bits) @ dequantize_mx(qw, sw).T


def grouped_gemm_mx_ref(a_payload: np.ndarray, a_scales: np.ndarray, expert_offsets: np.ndarray,
                        expert_weight, rows=None) -> np.ndarray:
    """Grouped GEMM on already-quantized rows (the second MoE GEMM).

    Output row r (expert-sorted order) is the exact product of MXFP4 row r of A
    (canonical payload and scales) and the quantized weight of the expert e with
    expert_offsets[e] <= r < expert_offsets[e+1]. ``rows`` selects output rows.
    """
    offs = np.asarray(expert_offsets, dtype=np.int64)
    R = int(offs[-1])
    rows = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    expert_of = np.searchsorted(offs, rows, side="right") - 1
    out = None
    for e in np.unique(expert_of):
        sel = np.flatnonzero(expert_of == e)
        qw, sw = quantize_mx(expert_weight(int(e)))
        c = gemm_from_mx(np.asarray(a_payload)[rows[sel]], np.asarray(a_scales)[rows[sel]], qw, sw)
        if out is None:
            out = np.empty((rows.size, c.shape[1]), dtype=np.float64)
        out[sel] = c
    return np.empty((0, 0)) if out is None else out


def combine_ref(y: np.ndarray, token_rows: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """Top-k weighted combine: out[t] = sum_k weights[t, k] * y[token_rows[t, k]], float64;
    a row index outside [0, len(y)) contributes nothing."""
    y = np.asarray(y, dtype=np.float64)
    tr = np.asarray(token_rows, dtype=np.int64)
    w = np.asarray(weights, dtype=np.float64)
    T, topk = tr.shape
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for k in range(topk):
        ok = (tr[:, k] >= 0) & (tr[:, k] < y.shape[0])
        out[ok] += w[ok, k:k + 1] * y[tr[ok, k]]
    return out


# ----------------------------------------------------------------------------- sizes

def prepared_weight_bytes(N: int, K: int) -> int:
    """Bytes of an MXFP4 weight: N*K/2 payload + N*K/32 scales = N*K*17/32."""
    return N * K // 2 + N * K // BLOCK


def rel_l2(x: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    den = math.sqrt(float(np.sum(ref * ref)))
    return math.sqrt(float(np.sum((np.asarray(x, dtype=np.float64) - ref) ** 2))) / den if den else 0.0
