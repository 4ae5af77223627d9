"""GPU parity of the MoE second GEMM on MXFP4 rows and of the top-k weighted combine against
the oracle (oracle/mx_oracle.py: grouped_gemm_mx_ref, combine_ref).

- GEMM2 at the layer's shape (E = 896, N = model_dim 3584, K = inter_dim 768) for the routed
  rows of T = 1, 16, 256, 4096 tokens, on sampled rows, in the configuration the library
  picks (the one the bench times); arbitrary MXFP4 rows (every E2M1 code, scales 2^-9..2^2).
- Every configuration (tiled, and the short-K sweep with 4, 7 and 14 column tiles per unit,
  N = 1024 leaving a partial chunk) on a ragged segment table (0, 1, 63, 64, 130, 200 rows),
  all rows.
- The combine, with out-of-range row indices, against the exact weighted sum of the same
  bf16 rows. Its bound follows from the arithmetic: a k-term FP32 sum of FP32 products
  (at most (topk + 2) 2^-24 sum_k |w_k y_k|) and one rounding to bf16, whose 8-bit
  significand leaves at most half an ulp, 2^-8 of the value."""
import numpy as np
import pytest

import workloads as W
from oracle import mx_oracle as O

from gpu_util import check_gemm, dev_bf16, host_bits, lib_or_fail, sample_rows, torch_or_skip
from test_gpu_grouped import _ragged_case

pytestmark = pytest.mark.gpu

_w2 = {"buf": None, "done": set(), "rows": {}}
CHECK_COLS = 32


def stacked_w2(experts):
    """Stacked prepared second-GEMM weights; only the listed experts are filled. Rows 0..31
    of each (the weight of output columns 0..31) are kept for the one-row-per-expert check."""
    torch = torch_or_skip()
    mx = lib_or_fail()
    per = mx.mx_prepared_weight_bytes(W.MOE_N2, W.MOE_K2)
    if _w2["buf"] is None:
        _w2["buf"] = torch.zeros(W.MOE_E * per, dtype=torch.uint8, device="cuda")
    need = sorted(set(int(e) for e in experts) - _w2["done"])
    for e in need:
        w = W.moe_expert_weight2(e)
        mx.mx_prepare_weight(dev_bf16(w), out=_w2["buf"][e * per:(e + 1) * per])
        _w2["rows"][e] = w[:CHECK_COLS].copy()
        _w2["done"].add(e)
    torch.cuda.synchronize()
    return _w2["buf"]


def _u8(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


@pytest.mark.parametrize("T", list(W.MOE_TOKENS))
def test_gemm2_matches_oracle(T):
    torch = torch_or_skip()
    mx = lib_or_fail()
    _, offs, _ = W.moe_routing(T)
    R = int(offs[-1])
    hint = max(1, -(-R // min(W.MOE_E, R)))
    aq, as_ = W.mx_bytes(R, W.MOE_K2, seed=200 + T)
    w2 = stacked_w2(np.flatnonzero(np.diff(offs) > 0))
    out = torch.full((R + 2, W.MOE_N2), 7.0, dtype=torch.bfloat16, device="cuda")
    mx.mx_a4w4_gemm_grouped_mx(_u8(aq), _u8(as_), torch.from_numpy(offs).cuda(), W.MOE_E, R, w2, W.MOE_N2,
                               rows_hint=hint, out=out[:R])
    c = host_bits(out)
    torch.cuda.synchronize()
    assert np.all(O.bf16_to_f64(c[R:]) == 7.0)
    rows = sample_rows(R, n=16, seed=300 + T, tile=None)
    exact = O.grouped_gemm_mx_ref(aq, as_, offs, W.moe_expert_weight2, rows=rows)
    check_gemm(c[rows], exact, what=f"gemm2 T={T} ({mx.mx_a4w4_gemm_grouped_mx_plan(W.MOE_N2, W.MOE_K2, hint)})")
    # one row of every active expert, output columns 0..31
    rng = np.random.default_rng(310 + T)
    rows = np.array([int(offs[e]) + int(rng.integers(0, offs[e + 1] - offs[e]))
                     for e in np.flatnonzero(np.diff(offs) > 0)], dtype=np.int64)
    exact = O.grouped_gemm_mx_ref(aq, as_, offs, lambda e: _w2["rows"][int(e)], rows=rows)
    check_gemm(c[rows, :CHECK_COLS], exact, what=f"gemm2 T={T}, one row per active expert ({rows.size})")


@pytest.mark.parametrize("cfg", ["gt,1,4,4,4,2,2", "gt,1,8,8,4,1,2", "gt,1,4,4,2,2,2", "gk,4", "gk,7", "gk,14"])
def test_gemm2_every_config_on_ragged_segments(cfg, monkeypatch):
    torch = torch_or_skip()
    mx = lib_or_fail()
    E, _, K, _, offs, _, _, _ = _ragged_case()
    N = 1024
    R = int(offs[-1])
    ws = [W.dense_weight(N, K, seed=120 + e) for e in range(E)]
    wst = torch.cat([mx.mx_prepare_weight(dev_bf16(w)) for w in ws])
    aq, as_ = W.mx_bytes(R, K, seed=17)
    monkeypatch.setenv("MX_GROUPED_CONFIG", cfg)
    c = host_bits(mx.mx_a4w4_gemm_grouped_mx(_u8(aq), _u8(as_), torch.from_numpy(offs).cuda(), E, R, wst, N))
    torch.cuda.synchronize()
    check_gemm(c, O.grouped_gemm_mx_ref(aq, as_, offs, lambda e: ws[e]), what=f"gemm2 {cfg}")


def test_gemm2_bad_override_fails(monkeypatch):
    torch = torch_or_skip()
    mx = lib_or_fail()
    E, _, K, _, offs, _, _, _ = _ragged_case()
    N, R = 1024, int(offs[-1])
    wst = torch.zeros(E * mx.mx_prepared_weight_bytes(N, K), dtype=torch.uint8, device="cuda")
    aq, as_ = W.mx_bytes(R, K, seed=18)
    monkeypatch.setenv("MX_GROUPED_CONFIG", "gt,2,4,4,4,1,1")
    with pytest.raises(mx.MxError):
        mx.mx_a4w4_gemm_grouped_mx(_u8(aq), _u8(as_), torch.from_numpy(offs).cuda(), E, R, wst, N)


@pytest.mark.parametrize("T", [1, 16, 256])
def test_combine_matches_oracle(T):
    torch = torch_or_skip()
    mx = lib_or_fail()
    ids, offs, _ = W.moe_routing(T)
    R, N, topk = int(offs[-1]), W.MOE_N2, W.MOE_TOPK
    y = W.normal_bf16((R, N), seed=400 + T, std=3.0)
    tr = W.moe_token_rows(ids)
    tr[0, 3] = -1                      # out of range: contributes nothing
    tr[-1, -1] = R
    wts = W.moe_combine_weights(T)
    out = host_bits(mx.mx_moe_combine(dev_bf16(y), torch.from_numpy(tr).cuda(), torch.from_numpy(wts).cuda()))
    torch.cuda.synchronize()
    yv = O.bf16_to_f64(y)
    exact = O.combine_ref(yv, tr, wts)
    mag = O.combine_ref(np.abs(yv), tr, np.abs(wts))
    got = O.bf16_to_f64(out)
    fp32 = (topk + 2) * 2.0 ** -24 * mag * 1.01
    bound = 2.0 ** -8 * (np.abs(exact) + fp32) + fp32 + 1e-30
    bad = np.abs(got - exact) > bound
    assert not bad.any(), f"{int(bad.sum())} outputs outside the bound; first {np.argwhere(bad)[0]}"


def test_combine_empty_and_errors():
    torch = torch_or_skip()
    mx = lib_or_fail()
    y = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    tr = torch.zeros((0, 2), dtype=torch.int32, device="cuda")
    assert mx.mx_moe_combine(y, tr, torch.zeros((0, 2), dtype=torch.float32, device="cuda")).shape == (0, 64)
    with pytest.raises(mx.MxError):   # N = 60 is not a multiple of 8
        mx.mx_moe_combine(torch.zeros((4, 60), dtype=torch.bfloat16, device="cuda"),
                          torch.zeros((2, 2), dtype=torch.int32, device="cuda"),
                          torch.zeros((2, 2), dtype=torch.float32, device="cuda"))
