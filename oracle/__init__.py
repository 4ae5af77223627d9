"""CPU oracle (test infrastructure only; never imported by the product library)."""
from .mx_oracle import (  # noqa: F401
    BLOCK, E2M1_MAGNITUDES, E8M0_BIAS, bf16_to_f64, block_exponent, dequantize_mx,
    e2m1_decode, encode_e2m1, gemm_bf16_exact, gemm_from_mx, gemm_ref, gemm_ref_sampled,
    grouped_gemm_ref, grouped_gemm_mx_ref, combine_ref, gemm_a16w4_ref, prepared_weight_bytes, quantize_mx, rel_l2, unpack_codes,
)
