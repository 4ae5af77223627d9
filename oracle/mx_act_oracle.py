"""CPU oracle for grouped GEMM1 with a fused activation + MXFP4 quantization epilogue.

TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the bench's
CPU-baseline leg are the only callers; the product library never imports,
links or runs anything here.

What is computed, and where it is stated:

* "[gfx1250] Fuse A4W4 stage1 FP4 quantization", Summary: the grouped GEMM1
  epilogue applies the activation (SiLU or SwiGLU) to the GEMM1 output and
  emits packed MXFP4 (E2M1 payload plus E8M0 scales) for the second GEMM,
  with each E8M0 scale computed directly from the FP32 activation value.
* The GEMM1 output itself is mx_oracle.grouped_gemm_ref: the exact product of
  the MXFP4-quantized routed activation rows and the expert's MXFP4 weight.

Readings taken where the pages are silent:

1. SiLU(x) = x / (1 + exp(-x)).
2. SwiGLU on a gate+up output of N columns: h[:, j] = SiLU(c[:, j]) * c[:, N/2 + j]
   for j < N/2 (gate columns first, up columns second); h has N/2 columns.
3. SiLU without gating: h = SiLU(c) on all N columns.
4. h is quantized along its columns in 32-element blocks with the rule of
   mx_oracle.quantize_mx applied to the real value of h. The gfx1250 page rounds
   h to BF16 before packing only because its 8-wide pack instruction takes BF16;
   gfx950 converts FP32 directly, so h is quantized once.
5. SiTUv2 is not defined on the pages and is not implemented.

Checking a GPU result. The GPU forms h in FP32 from FP32 accumulators, so at a
rounding boundary its code or scale may legitimately differ from the exact one.
``grouped_gemm1_act_ref`` therefore returns, besides the exact h, an interval
[h_lo, h_hi] that provably holds the GPU's FP32 value: each accumulator lies
within gamma_K * sum_k |a_k w_k| of the exact sum (the standard bound for K
floating-point additions of exactly representable products, gamma_K =
1.01 K 2^-24), the interval is carried through the activation exactly (SiLU's
one minimum included), and widened for the FP32 evaluation of the activation
itself: (|g| + 16) 2^-23 |h|, with |g| the largest gate magnitude in the
interval, covers an exponential and a reciprocal of 1 ulp each (the hardware
v_exp_f32 and v_rcp_f32), the rounding of the exponential's argument
-|g| log2(e) (relative error |g| 2^-24 in exp(-|g|)) and three roundings of
products and sums; 2^-100 max|up| more covers an exponential that underflows
to zero (|g| > 87, where the exact SiLU is below 2^-120). ``quantization_valid`` accepts a GPU scale byte only if
it is the rule's scale of some block amax inside the intervals, and a GPU code
only if it is the rule's code, at that scale, of some value in the element's
interval. Where an interval holds a single code and scale, this is bit-exact
agreement with the oracle's own quantization of the exact h.
"""
from __future__ import annotations

import numpy as np

from . import mx_oracle as O

ACT_SILU = 0
ACT_SWIGLU = 1

# SiLU's only stationary point: the root of 1 + x (1 - sigmoid(x)) = 0 (a minimum).
SILU_ARGMIN = -1.2784645427610738
FP32_UNIT = 2.0 ** -24


def silu(x):
    """x * sigmoid(x) = x / (1 + exp(-x)), in float64."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def activation(c: np.ndarray, act: int) -> np.ndarray:
    """h from a GEMM1 output c [R, N] (readings 1-3)."""
    c = np.asarray(c, dtype=np.float64)
    if act == ACT_SILU:
        return silu(c)
    if act == ACT_SWIGLU:
        half = c.shape[1] // 2
        return silu(c[:, :half]) * c[:, half:]
    raise ValueError(f"unknown activation {act}")


def quantize_mx_values(v: np.ndarray):
    """Quantize real rows [R, K] to MXFP4 along K (the rule of quantize_mx, on values).

    The sign bit of an element is the sign of its value (negative zero included).
    Returns (payload uint8 [R, K/2], scales uint8 [R, K/32]), canonical layout.
    """
    v = np.asarray(v, dtype=np.float64)
    if v.ndim != 2 or v.shape[1] % O.BLOCK != 0:
        raise ValueError("expected [R, K] with K a multiple of 32")
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite input is outside the MXFP4 quantizer's contract")
    R, K = v.shape
    vb = v.reshape(R, K // O.BLOCK, O.BLOCK)
    e = O.block_exponent(np.abs(vb).max(axis=-1))                 # step: shared exponent
    q = np.ldexp(vb, -e[..., None])                               # step: scale (exact)
    codes = O.encode_e2m1(q, np.signbit(vb)).reshape(R, K)        # step: RNE + saturate
    return codes[:, 0::2] | (codes[:, 1::2] << 4), (e + O.E8M0_BIAS).astype(np.uint8)


def _silu_range(lo: np.ndarray, hi: np.ndarray):
    """Exact range of SiLU over [lo, hi] (elementwise)."""
    a, b = silu(lo), silu(hi)
    rlo, rhi = np.minimum(a, b), np.maximum(a, b)
    inside = (lo <= SILU_ARGMIN) & (SILU_ARGMIN <= hi)
    return np.where(inside, np.minimum(rlo, silu(SILU_ARGMIN)), rlo), rhi


def _product_range(alo, ahi, blo, bhi):
    corners = np.stack([alo * blo, alo * bhi, ahi * blo, ahi * bhi])
    return corners.min(axis=0), corners.max(axis=0)


def grouped_gemm1_act_ref(a_bits: np.ndarray, row_token: np.ndarray, expert_offsets: np.ndarray,
                          expert_weight, act: int, rows=None):
    """Exact h and an interval holding the GPU's FP32 h, for selected output rows.

    Row r (expert-sorted order) of the GEMM1 output is the exact product of the
    quantized activation row A[row_token[r]] and the quantized weight of the
    expert whose segment holds r (mx_oracle.grouped_gemm_ref); h follows from
    ``activation``. Returns (h, h_lo, h_hi), each [len(rows), N_h] float64.
    """
    offs = np.asarray(expert_offsets, dtype=np.int64)
    tok = np.asarray(row_token, dtype=np.int64)
    R = int(offs[-1])
    rows = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    expert_of = np.searchsorted(offs, rows, side="right") - 1
    c = cabs = None
    for e in np.unique(expert_of):
        sel = np.flatnonzero(expert_of == e)
        qa, sa = O.quantize_mx(np.asarray(a_bits)[tok[rows[sel]]])
        qw, sw = O.quantize_mx(expert_weight(int(e)))
        ce = O.gemm_from_mx(qa, sa, qw, sw)                                   # exact sums
        ae = np.abs(O.dequantize_mx(qa, sa)) @ np.abs(O.dequantize_mx(qw, sw)).T  # sum of |products|
        if c is None:
            c = np.empty((rows.size, ce.shape[1]))
            cabs = np.empty_like(c)
        c[sel], cabs[sel] = ce, ae
    if c is None:
        return (np.empty((0, 0)),) * 3
    K = np.asarray(a_bits).shape[1]
    d = 1.01 * K * FP32_UNIT * cabs * (1.0 + 1e-12) + 1e-300
    lo, hi = c - d, c + d
    h = activation(c, act)
    if act == ACT_SILU:
        glo, ghi = lo, hi
        h_lo, h_hi = _silu_range(lo, hi)
        umax = np.ones_like(h)
    else:
        half = c.shape[1] // 2
        glo, ghi = lo[:, :half], hi[:, :half]
        slo, shi = _silu_range(glo, ghi)
        h_lo, h_hi = _product_range(slo, shi, lo[:, half:], hi[:, half:])
        umax = np.maximum(np.abs(lo[:, half:]), np.abs(hi[:, half:]))
    gmax = np.maximum(np.abs(glo), np.abs(ghi))
    w = (gmax + 16.0) * 2.0 ** -23 * np.maximum(np.abs(h_lo), np.abs(h_hi)) + 2.0 ** -100 * umax + 1e-300
    return h, h_lo - w, h_hi + w


def quantization_valid(payload: np.ndarray, scales: np.ndarray, h_lo: np.ndarray, h_hi: np.ndarray):
    """Per-block and per-element validity of a quantized h against intervals [h_lo, h_hi].

    Returns (scale_ok [R, K/32] bool, code_ok [R, K] bool); see the module notes.
    """
    payload = np.asarray(payload, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    R, K = h_lo.shape
    nb = K // O.BLOCK
    blo = h_lo.reshape(R, nb, O.BLOCK)
    bhi = h_hi.reshape(R, nb, O.BLOCK)
    spans0 = (blo <= 0) & (bhi >= 0)
    amin_el = np.where(spans0, 0.0, np.minimum(np.abs(blo), np.abs(bhi)))
    amax_lo = amin_el.max(axis=-1)
    amax_hi = np.maximum(np.abs(blo), np.abs(bhi)).max(axis=-1)
    s_lo = O.block_exponent(amax_lo) + O.E8M0_BIAS
    s_hi = O.block_exponent(amax_hi) + O.E8M0_BIAS
    scale_ok = (scales.astype(np.int64) >= s_lo) & (scales.astype(np.int64) <= s_hi)

    e = scales.astype(np.int64) - O.E8M0_BIAS                      # the GPU's own scale
    e_el = np.repeat(e, O.BLOCK, axis=1)
    codes = O.unpack_codes(payload)
    value = O.e2m1_decode(codes)                                    # at scale 2^0
    c_lo = O.encode_e2m1(np.ldexp(h_lo, -e_el), np.signbit(h_lo))
    c_hi = O.encode_e2m1(np.ldexp(h_hi, -e_el), np.signbit(h_hi))
    v_lo, v_hi = O.e2m1_decode(c_lo), O.e2m1_decode(c_hi)
    in_range = (value >= v_lo) & (value <= v_hi)
    neg_zero = codes == 0x8
    pos_zero = codes == 0x0
    zero_sign_ok = np.where(neg_zero, h_lo < 0, np.where(pos_zero, h_hi >= 0, True))
    return scale_ok, in_range & zero_sign_ok
