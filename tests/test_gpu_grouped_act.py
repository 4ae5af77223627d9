"""GPU parity of grouped GEMM1 with the fused SiLU / SwiGLU + MXFP4 quantization epilogue
("[gfx1250] Fuse A4W4 stage1 FP4 quantization", Summary) against the oracle
(oracle/mx_act_oracle.py).

The GPU forms h in FP32, so every scale byte and code is checked against the oracle's
rigorous interval for that FP32 value: it must be the quantization rule's result for some
value in the interval (bit-exact wherever the interval holds a single code and scale). The
share of codes identical to the oracle's quantization of the exact h is reported too."""
import numpy as np
import pytest

import workloads as W
from oracle import mx_act_oracle as AO
from oracle import mx_oracle as O

from gpu_util import dev_bf16, host_u8, lib_or_fail, sample_rows, torch_or_skip
from test_gpu_grouped import (CHECK_COLS, _ragged_case, expert_first_rows, expert_gate_up_rows, one_row_per_expert,
                               rows_hint, stacked_weights)

pytestmark = pytest.mark.gpu


def _check(q, s, a, row_token, offs, weight, act, rows, what):
    h, lo, hi = AO.grouped_gemm1_act_ref(a, row_token, offs, weight, act, rows=rows)
    scale_ok, code_ok = AO.quantization_valid(q[rows], s[rows], lo, hi)
    if not scale_ok.all():
        i = np.argwhere(~scale_ok)[0]
        raise AssertionError(f"{what}: {int((~scale_ok).sum())} scale bytes invalid; first row {rows[i[0]]} "
                             f"block {i[1]}: gpu {s[rows[i[0]], i[1]]}")
    if not code_ok.all():
        i = np.argwhere(~code_ok)[0]
        raise AssertionError(f"{what}: {int((~code_ok).sum())} codes invalid; first row {rows[i[0]]} col {i[1]}: "
                             f"interval [{lo[tuple(i)]!r}, {hi[tuple(i)]!r}]")
    hq, _ = AO.quantize_mx_values(h)
    same = float(np.mean(O.unpack_codes(q[rows]) == O.unpack_codes(hq)))
    print(f"{what}: {same:.5f} of codes identical to the exact quantization")
    assert same > 0.99


@pytest.mark.parametrize("T", list(W.MOE_TOKENS))
def test_swiglu_quant_matches_oracle(T):
    torch = torch_or_skip()
    mx = lib_or_fail()
    a = W.moe_activation(T)
    _, offs, row_token = W.moe_routing(T)
    wst = stacked_weights(np.flatnonzero(np.diff(offs) > 0))
    R = int(offs[-1])
    Nh = W.MOE_N // 2
    hq = torch.full((R + 2, Nh // 2), 0xAB, dtype=torch.uint8, device="cuda")
    hs = torch.full((R + 2, Nh // 32), 0xCD, dtype=torch.uint8, device="cuda")
    mx.mx_a4w4_gemm_grouped_act_quant(dev_bf16(a), torch.from_numpy(row_token).cuda(), torch.from_numpy(offs).cuda(),
                                      W.MOE_E, R, wst, W.MOE_N, act=mx.MX_ACT_SWIGLU, rows_hint=rows_hint(T),
                                      h_fp4=hq[:R], h_scale=hs[:R])
    torch.cuda.synchronize()
    q, s = host_u8(hq), host_u8(hs)
    assert np.all(q[R:] == 0xAB) and np.all(s[R:] == 0xCD)       # rows >= R untouched
    rows = sample_rows(R, n=16, seed=100 + T, tile=None)
    _check(q, s, a, row_token, offs, W.moe_expert_weight, AO.ACT_SWIGLU, rows,
           f"swiglu T={T} ({mx.mx_a4w4_gemm_grouped_act_quant_plan(W.MOE_E, R, W.MOE_N, W.MOE_K, 1, rows_hint(T))})")
    # one row of every active expert: its first 32-column block of h (gate columns 0..31 with
    # their up partners 768..799)
    rows = one_row_per_expert(offs, seed=110 + T)
    _check(q[:, :CHECK_COLS // 2], s[:, :CHECK_COLS // 32], a, row_token, offs, expert_gate_up_rows, AO.ACT_SWIGLU,
           rows, f"swiglu T={T}, one row per active expert ({rows.size})")


def test_silu_quant_matches_oracle():
    torch = torch_or_skip()
    mx = lib_or_fail()
    T = 256
    a = W.moe_activation(T)
    _, offs, row_token = W.moe_routing(T)
    wst = stacked_weights(np.flatnonzero(np.diff(offs) > 0))
    R = int(offs[-1])
    hq, hs = mx.mx_a4w4_gemm_grouped_act_quant(dev_bf16(a), torch.from_numpy(row_token).cuda(),
                                               torch.from_numpy(offs).cuda(), W.MOE_E, R, wst, W.MOE_N,
                                               act=mx.MX_ACT_SILU, rows_hint=rows_hint(T))
    torch.cuda.synchronize()
    assert hq.shape == (R, W.MOE_N // 2) and hs.shape == (R, W.MOE_N // 32)
    rows = sample_rows(R, n=16, seed=7, tile=None)
    _check(host_u8(hq), host_u8(hs), a, row_token, offs, W.moe_expert_weight, AO.ACT_SILU, rows, "silu T=256")
    rows = one_row_per_expert(offs, seed=8)  # SiLU: h columns 0..31 from output columns 0..31
    _check(host_u8(hq)[:, :CHECK_COLS // 2], host_u8(hs)[:, :CHECK_COLS // 32], a, row_token, offs,
           expert_first_rows, AO.ACT_SILU, rows, f"silu T=256, one row per active expert ({rows.size})")


ACT_CONFIGS = ["gt,1,4,4,4,2,2", "gt,1,8,8,4,1,2", "gt,1,4,4,2,2,2"]


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("cfg", ACT_CONFIGS)
def test_every_fused_config_on_ragged_segments(cfg, act, monkeypatch):
    """Every fused configuration, both activations, every row of a ragged segment table
    (segments of 0, 1, 63, 64, 130 and 200 rows), N = 1024 so both tile widths divide it."""
    torch = torch_or_skip()
    mx = lib_or_fail()
    E, _, K, T, offs, row_token, a, _ = _ragged_case()
    N = 1024
    ws = [W.dense_weight(N, K, seed=90 + e) for e in range(E)]
    wst = torch.cat([mx.mx_prepare_weight(dev_bf16(w)) for w in ws])
    R = int(offs[-1])
    monkeypatch.setenv("MX_GROUPED_CONFIG", cfg)
    hq, hs = mx.mx_a4w4_gemm_grouped_act_quant(dev_bf16(a), torch.from_numpy(row_token).cuda(),
                                               torch.from_numpy(offs).cuda(), E, R, wst, N, act=act, rows_hint=1)
    torch.cuda.synchronize()
    _check(host_u8(hq), host_u8(hs), a, row_token, offs, lambda e: ws[e], act, np.arange(R),
           f"{cfg} act={act}")


def test_fused_without_tokens_writes_zero():
    torch = torch_or_skip()
    mx = lib_or_fail()
    E, _, K, _, offs, _, _, _ = _ragged_case()
    N = 1024
    wst = torch.zeros(E * mx.mx_prepared_weight_bytes(N, K), dtype=torch.uint8, device="cuda")
    R = int(offs[-1])
    for act in (0, 1):
        Nh = N // 2 if act else N
        hq = torch.full((R, Nh // 2), 0x77, dtype=torch.uint8, device="cuda")
        hs = torch.full((R, Nh // 32), 0x77, dtype=torch.uint8, device="cuda")
        mx.mx_a4w4_gemm_grouped_act_quant(torch.empty((0, K), dtype=torch.bfloat16, device="cuda"),
                                          torch.zeros(R, dtype=torch.int32, device="cuda"),
                                          torch.from_numpy(offs).cuda(), E, R, wst, N, act=act, h_fp4=hq, h_scale=hs)
        torch.cuda.synchronize()
        assert np.all(host_u8(hq) == 0) and np.all(host_u8(hs) == 0)


@pytest.mark.parametrize("bad", ["gt,1,4,4,4,1,2", "gs,1,1", "gt,9"])
def test_fused_unknown_override_fails(bad, monkeypatch):
    torch = torch_or_skip()
    mx = lib_or_fail()
    E, _, K, T, offs, row_token, a, _ = _ragged_case()
    N = 1024
    wst = torch.zeros(E * mx.mx_prepared_weight_bytes(N, K), dtype=torch.uint8, device="cuda")
    monkeypatch.setenv("MX_GROUPED_CONFIG", bad)
    with pytest.raises(mx.MxError):
        mx.mx_a4w4_gemm_grouped_act_quant(dev_bf16(a), torch.from_numpy(row_token).cuda(),
                                          torch.from_numpy(offs).cuda(), E, int(offs[-1]), wst, N)
