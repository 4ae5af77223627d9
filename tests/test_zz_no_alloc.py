"""The allocation-free dense GEMM (mx_a4w4_gemm_noalloc) against mx_a4w4_gemm with the
workspace that entry point asks for: the same plan runs with the library's own device scratch
array in place of a caller workspace, so the outputs agree bit for bit.

Two calls in a row share the array: the first runs the quantize-once plan (its activations
fill the scratch), the second a smaller call whose plan writes K-slice partial sums over the
same bytes; then the first shape once more. Each output is also checked against the oracle."""
import numpy as np
import pytest

import workloads as W
from oracle import mx_oracle as O

from gpu_util import check_gemm, dev_bf16, host_bits, lib_or_fail, torch_or_skip

pytestmark = pytest.mark.gpu

# (M, N, K): quantize-once plan, then a smaller call whose plan keeps K-slice partials in the
# workspace, then one without a workspace
CASES = [(1024, 2560, 4224), (128, 1536, 7168), (300, 768, 768)]


def test_noalloc_matches_workspace_entry_point():
    torch = torch_or_skip()
    mx = lib_or_fail()
    plans = []
    ws_seen = []
    inputs = {}
    for M, N, K in CASES:
        if (N, K) not in inputs:
            w = W.dense_weight(N, K, seed=61)
            inputs[(N, K)] = (w, mx.mx_prepare_weight(dev_bf16(w)),
                              W.dense_activation(max(m for m, n, k in CASES if (n, k) == (N, K)), K,
                                                 "outlier_channels", seed=62))
    for M, N, K in CASES + CASES[:1]:
        w, wp, a_all = inputs[(N, K)]
        a = a_all[:M]
        need = mx.mx_a4w4_gemm_workspace_bytes(M, N, K)
        assert need <= mx.mx_noalloc_scratch_bytes()
        ws_seen.append(need)
        plans.append(mx.mx_a4w4_gemm_plan(M, N, K, need))
        da = dev_bf16(a)
        ref = mx.mx_a4w4_gemm(da, wp, N)  # allocates `need` bytes of workspace itself
        out = torch.full((M + 2, N), -5.0, dtype=torch.bfloat16, device="cuda")
        mx.mx_a4w4_gemm_noalloc(da, wp, N, out=out[:M])
        torch.cuda.synchronize()
        got = host_bits(out[:M])
        assert np.array_equal(got, host_bits(ref)), f"M={M} N={N} K={K} ({plans[-1]}): differs"
        assert bool((out[M:] == -5.0).all()), f"M={M} N={N} K={K}: rows past M were written"
        qa, sa = O.quantize_mx(a)
        qw, sw = O.quantize_mx(w)
        check_gemm(got, O.gemm_from_mx(qa, sa, qw, sw), what=f"noalloc M={M} N={N} K={K}")
    # the cases exercise both uses of the scratch array and a plan without one
    assert "k_gemm_qo" in plans[0] and ws_seen[0] > 0, plans[0]
    assert "k_splitk_reduce" in plans[1] and ws_seen[1] > 0, plans[1]
    assert ws_seen[2] == 0, plans[2]


def test_noalloc_rejects_plans_beyond_the_scratch():
    torch = torch_or_skip()
    mx = lib_or_fail()
    M, N, K = 16384, 2560, 7168  # quantize-once activations: 16384 * 7168 * 17 / 32 bytes > 32 MiB
    assert mx.mx_a4w4_gemm_workspace_bytes(M, N, K) > mx.mx_noalloc_scratch_bytes()
    a = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    wp = torch.zeros(mx.mx_prepared_weight_bytes(N, K), dtype=torch.uint8, device="cuda")
    out = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mx.MxError, match="WORKSPACE"):
        mx.mx_a4w4_gemm_noalloc(a, wp, N, out=out)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "nothing is launched when the plan does not fit"


def test_noalloc_register_direct_plans():
    """The register-direct plans through the scratch array: 2048 x 8448 at K = 2048 (944 tiles
    of 128 x 144, one wave each), then 2048 x 1536 at K = 7168 (the four-wave kernel) over the
    same bytes; bit for bit against mx_a4w4_gemm with its own workspace, and against the
    oracle. (The register-direct plan with tail K slices needs at least 129 x 4 FP32 partial
    tiles of 64 KiB, more than the array holds, so that plan is refused here.)"""
    torch = torch_or_skip()
    mx = lib_or_fail()
    for M, N, K, kern in ((2048, 8448, 2048, "k_gemm_qr<8, 9, 1>"), (2048, 1536, 7168, "k_gemm_qk")):
        need = mx.mx_a4w4_gemm_workspace_bytes(M, N, K)
        assert 0 < need <= mx.mx_noalloc_scratch_bytes()
        plan = mx.mx_a4w4_gemm_plan(M, N, K, need)
        assert kern in plan, plan
        w = W.dense_weight(N, K, seed=63)
        a = W.dense_activation(M, K, "outlier_channels", seed=64)
        wp = mx.mx_prepare_weight(dev_bf16(w))
        da = dev_bf16(a)
        ref = mx.mx_a4w4_gemm(da, wp, N)
        out = torch.full((M + 2, N), -5.0, dtype=torch.bfloat16, device="cuda")
        mx.mx_a4w4_gemm_noalloc(da, wp, N, out=out[:M])
        torch.cuda.synchronize()
        got = host_bits(out[:M])
        assert np.array_equal(got, host_bits(ref)), f"M={M} N={N} K={K} ({plan}): differs"
        assert bool((out[M:] == -5.0).all()), f"M={M} N={N} K={K}: rows past M were written"
        qa, sa = O.quantize_mx(a)
        qw, sw = O.quantize_mx(w)
        check_gemm(got, O.gemm_from_mx(qa, sa, qw, sw), what=f"noalloc M={M} N={N} K={K}")
