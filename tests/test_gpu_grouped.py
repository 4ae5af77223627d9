"""GPU parity of the grouped MoE GEMM1 (E = 896 experts, top-16 uniform routing,
K = 3584, N = 1536) against the oracle, plus malformed-table handling."""
import numpy as np
import pytest

import workloads as W
from oracle import mx_oracle as O

from gpu_util import check_gemm, dev_bf16, host_bits, lib_or_fail, sample_rows, torch_or_skip

pytestmark = pytest.mark.gpu

_stack = {"experts": set(), "buf": None, "rows": {}}
CHECK_COLS = 32  # output columns of the one-row-per-expert checks: one MXFP4 block of h


def stacked_weights(experts):
    """Stacked prepared weights of all E experts; only the listed ones are filled
    (the others are never read by a launch whose table leaves them empty). While each
    expert's weight is at hand, the rows the one-row-per-expert checks need are kept:
    W rows 0..31 (output columns 0..31) and 768..799 (the up columns paired with gate
    columns 0..31)."""
    torch = torch_or_skip()
    mx = lib_or_fail()
    per = mx.mx_prepared_weight_bytes(W.MOE_N, W.MOE_K)
    if _stack["buf"] is None:
        _stack["buf"] = torch.zeros(W.MOE_E * per, dtype=torch.uint8, device="cuda")
    need = sorted(set(int(e) for e in experts) - _stack["experts"])
    half = W.MOE_N // 2
    for e, w in W.moe_expert_weights(need):
        mx.mx_prepare_weight(dev_bf16(w), out=_stack["buf"][e * per:(e + 1) * per])
        _stack["rows"][e] = (w[:CHECK_COLS].copy(), w[half:half + CHECK_COLS].copy())
        _stack["experts"].add(e)
    torch.cuda.synchronize()
    return _stack["buf"]


def expert_first_rows(e):
    """W_e rows 0..31: the weight of output columns 0..31 (kept by stacked_weights)."""
    return _stack["rows"][int(e)][0]


def expert_gate_up_rows(e):
    """W_e rows 0..31 (gate) stacked on rows 768..799 (their up partners): a 64-row weight
    whose SwiGLU output is h columns 0..31."""
    lo, up = _stack["rows"][int(e)]
    return np.concatenate([lo, up])


def per_expert_exact(a, row_token, offs, rows):
    """Exact GEMM1 output columns 0..31 of the given rows (at most one per expert): the same
    steps as the oracle's grouped reference (quantize the token's row and the expert's weight
    rows, exact product), with each expert's quantized weight rows kept across calls."""
    qcache = _stack.setdefault("q", {})
    expert_of = np.searchsorted(np.asarray(offs, dtype=np.int64), rows, side="right") - 1
    out = np.empty((len(rows), CHECK_COLS))
    for i, (r, e) in enumerate(zip(rows, expert_of)):
        if int(e) not in qcache:
            qcache[int(e)] = O.quantize_mx(expert_first_rows(e))
        qa, sa = O.quantize_mx(a[int(row_token[r])][None, :])
        out[i] = O.gemm_from_mx(qa, sa, *qcache[int(e)])[0]
    return out


def one_row_per_expert(offs, seed):
    """A seeded row inside every non-empty segment."""
    rng = np.random.default_rng(seed)
    return np.array([int(offs[e]) + int(rng.integers(0, offs[e + 1] - offs[e]))
                     for e in np.flatnonzero(np.diff(offs) > 0)], dtype=np.int64)


def rows_hint(T):
    R = W.MOE_TOPK * T
    return max(1, -(-R // min(W.MOE_E, R)))


@pytest.mark.parametrize("T", list(W.MOE_TOKENS))
def test_grouped_matches_oracle(T):
    torch = torch_or_skip()
    mx = lib_or_fail()
    a = W.moe_activation(T)
    ids, offs, row_token = W.moe_routing(T)
    active = np.flatnonzero(np.diff(offs) > 0)
    wst = stacked_weights(active)
    R = int(offs[-1])
    out = torch.full((R + 3, W.MOE_N), 5.0, dtype=torch.bfloat16, device="cuda")
    mx.mx_a4w4_gemm_grouped(dev_bf16(a), torch.from_numpy(row_token).cuda(), torch.from_numpy(offs).cuda(),
                            W.MOE_E, R, wst, W.MOE_N, rows_hint=rows_hint(T), out=out[:R])
    c = host_bits(out)
    torch.cuda.synchronize()
    assert np.all(c[R:] == host_bits(torch.full((1,), 5.0, dtype=torch.bfloat16))[0])
    rows = sample_rows(R, n=24, seed=T, tile=None)
    exact = O.grouped_gemm_ref(a, row_token, offs, W.moe_expert_weight, rows=rows)
    check_gemm(c[rows], exact, what=f"grouped T={T}")
    # one row of every active expert (its first 32 output columns): a wrong expert or unit
    # lookup for any segment would show
    rows = one_row_per_expert(offs, seed=10 + T)
    exact = per_expert_exact(a, row_token, offs, rows)
    check_gemm(c[rows, :CHECK_COLS], exact, what=f"grouped T={T}, one row per active expert ({rows.size})")


@pytest.mark.parametrize("hint", [1, 20, 64, 100])
def test_grouped_tiling_hint_only_changes_tiling(hint):
    """The rows-per-expert hint selects the tiling; every choice meets the tolerance."""
    torch = torch_or_skip()
    mx = lib_or_fail()
    T = 256
    a = W.moe_activation(T)
    _, offs, row_token = W.moe_routing(T)
    wst = stacked_weights(np.flatnonzero(np.diff(offs) > 0))
    R = int(offs[-1])
    c = host_bits(mx.mx_a4w4_gemm_grouped(dev_bf16(a), torch.from_numpy(row_token).cuda(),
                                          torch.from_numpy(offs).cuda(), W.MOE_E, R, wst, W.MOE_N,
                                          rows_hint=hint))
    torch.cuda.synchronize()
    rows = sample_rows(R, n=16, seed=hint, tile=None)
    exact = O.grouped_gemm_ref(a, row_token, offs, W.moe_expert_weight, rows=rows)
    check_gemm(c[rows], exact, what=f"grouped hint={hint}")


@pytest.mark.parametrize("hint", [2, 64])
def test_grouped_malformed_table_is_clamped(hint):
    """Out-of-range tokens read as zero rows; segments are clamped to [0, R_max] (both the
    streaming and the tiled kernels)."""
    torch = torch_or_skip()
    mx = lib_or_fail()
    E, N, K, T = 4, 256, 256, 3
    rng = np.random.default_rng(0)
    a = W.f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    ws = [W.dense_weight(N, K, seed=50 + e) for e in range(E)]
    wst = torch.cat([mx.mx_prepare_weight(dev_bf16(w)) for w in ws])
    offs = np.array([0, 2, 2, 5, 9], dtype=np.int32)       # last segment runs past R_max = 6
    row_token = np.array([0, 2, 1, 7, -1, 2], dtype=np.int32)  # 7 and -1 are out of range
    R_max = 6
    c = host_bits(mx.mx_a4w4_gemm_grouped(dev_bf16(a), torch.from_numpy(row_token).cuda(),
                                          torch.from_numpy(offs).cuda(), E, R_max, wst, N, rows_hint=hint))
    torch.cuda.synchronize()
    expert_of = [0, 0, 2, 2, 2, 3]
    for r in range(R_max):
        tok = int(row_token[r])
        if 0 <= tok < T:
            want = O.gemm_ref(a[tok:tok + 1], ws[expert_of[r]])[0]
            check_gemm(c[r:r + 1], want[None, :], what=f"row {r}")
        else:
            assert np.all(O.bf16_to_f64(c[r]) == 0.0), r


GROUPED_CONFIGS = ["gs,1,1", "gs,1,4", "gs,2,1", "gs,2,4",
                   "gt,1,4,4,4,1,2", "gt,2,4,4,4,1,1", "gt,1,4,4,4,2,2",
                   "gt,1,8,8,4,1,2"]


def _ragged_case():
    """Six experts with segments of 0, 1, 63, 64, 130 and 200 rows (ragged tails, segments
    spanning several 64- and 128-row tiles), N = 512, K = 768, tokens drawn from T = 50."""
    E, N, K, T = 6, 512, 768, 50
    sizes = [0, 1, 63, 64, 130, 200]
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rng = np.random.default_rng(7)
    row_token = rng.integers(0, T, size=int(offs[-1])).astype(np.int32)
    a = W.f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    ws = [W.dense_weight(N, K, seed=80 + e) for e in range(E)]
    return E, N, K, T, offs, row_token, a, ws


@pytest.mark.parametrize("cfg", GROUPED_CONFIGS)
def test_grouped_every_config_matches_oracle(cfg, monkeypatch):
    """Each compiled grouped kernel (forced through the tuning override) matches the oracle
    on every row of a ragged segment table."""
    torch = torch_or_skip()
    mx = lib_or_fail()
    E, N, K, T, offs, row_token, a, ws = _ragged_case()
    wst = torch.cat([mx.mx_prepare_weight(dev_bf16(w)) for w in ws])
    R = int(offs[-1])
    monkeypatch.setenv("MX_GROUPED_CONFIG", cfg)
    c = host_bits(mx.mx_a4w4_gemm_grouped(dev_bf16(a), torch.from_numpy(row_token).cuda(),
                                          torch.from_numpy(offs).cuda(), E, R, wst, N, rows_hint=1))
    torch.cuda.synchronize()
    exact = O.grouped_gemm_ref(a, row_token, offs, lambda e: ws[e])
    check_gemm(c, exact, what=f"grouped {cfg}")


@pytest.mark.parametrize("hint", [2, 64])
def test_grouped_without_tokens_writes_zero_rows(hint):
    """T = 0: every output row is Q(0) W^T = 0 (and no activation is read)."""
    torch = torch_or_skip()
    mx = lib_or_fail()
    E, N, K, _, offs, _, _, ws = _ragged_case()
    wst = torch.cat([mx.mx_prepare_weight(dev_bf16(w)) for w in ws])
    R = int(offs[-1])
    row_token = torch.zeros(R, dtype=torch.int32, device="cuda")
    out = torch.full((R, N), 3.0, dtype=torch.bfloat16, device="cuda")
    empty = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    mx.mx_a4w4_gemm_grouped(empty, row_token, torch.from_numpy(offs).cuda(), E, R, wst, N,
                            rows_hint=hint, out=out)
    torch.cuda.synchronize()
    assert np.all(O.bf16_to_f64(host_bits(out)) == 0.0)


@pytest.mark.parametrize("bad", ["gt,1,4,4,4,3,2", "gs,3,1", "gx", "gt,1,4"])
def test_grouped_unknown_override_fails(bad, monkeypatch):
    torch = torch_or_skip()
    mx = lib_or_fail()
    E, N, K, T, offs, row_token, a, ws = _ragged_case()
    wst = torch.cat([mx.mx_prepare_weight(dev_bf16(w)) for w in ws])
    monkeypatch.setenv("MX_GROUPED_CONFIG", bad)
    with pytest.raises(mx.MxError):
        mx.mx_a4w4_gemm_grouped(dev_bf16(a), torch.from_numpy(row_token).cuda(), torch.from_numpy(offs).cuda(),
                                E, int(offs[-1]), wst, N)
