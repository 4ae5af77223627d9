"""Every compiled GEMM configuration (streaming kernel with and without K slices, tiled
kernel with and without masked tail tiles, several tile orders, the short-K sweep kernel and
the quantize-once kernel) against the oracle.

The library's tuning override (environment variable MX_GEMM_CONFIG) forces each
configuration; an override that does not name a compiled, feasible configuration fails
the call, so each case below provably ran the configuration it names."""
import os

import numpy as np
import pytest

import workloads as W
from oracle import mx_oracle as O

from gpu_util import check_gemm, dev_bf16, host_bits, lib_or_fail, torch_or_skip

pytestmark = pytest.mark.gpu

# mirrors MX_STREAM_CONFIGS / MX_TILE_CONFIGS in the kernels
STREAM = [(1, 1, 2), (1, 1, 4), (1, 1, 8), (1, 2, 4), (1, 2, 8), (1, 4, 4), (1, 4, 8),
          (2, 1, 2), (2, 1, 4), (2, 1, 8), (2, 2, 4), (2, 2, 8), (2, 4, 4), (2, 4, 8),
          (4, 1, 4), (4, 1, 8), (4, 2, 4), (4, 4, 4), (8, 1, 4), (8, 2, 4)]
TILE = [(1, 4, 4, 4, 2, 1), (2, 4, 4, 4, 2, 1), (1, 4, 8, 4, 1, 1), (2, 2, 4, 8, 1, 1), (1, 4, 4, 2, 2, 1),
        (1, 4, 4, 4, 1, 2), (1, 4, 4, 4, 2, 2), (2, 4, 4, 4, 1, 1), (1, 4, 4, 2, 2, 2),
        (1, 8, 8, 4, 1, 2), (1, 4, 4, 1, 2, 1), (1, 4, 4, 1, 2, 2)]
# mirrors MX_QO_CONFIGS in mx_gemm_qo.hip: (WM, WN, MT, NG, NBUF, OCC)
QO = [(2, 4, 8, 4, 4, 2), (2, 2, 4, 4, 4, 2), (2, 2, 4, 4, 5, 2), (1, 4, 8, 4, 3, 2)]
# mirrors MX_QR_CONFIGS / MX_QK_CONFIGS in mx_gemm_qo.hip: (MT, NG, D)
QR = [(8, 8, 2), (8, 9, 1), (9, 8, 1)]
QK = [(8, 8, 2), (8, 9, 1), (8, 7, 2), (8, 6, 2), (8, 3, 4)]
SWEEP_K = (256, 512, 768, 1024)  # the short-K sweep kernel's compiled step counts 2, 4, 6, 8
N_TEST = 768          # 3 x 256: tail tiles for BN = 512
K_TESTS = (4224, 768)  # 33 and 6 steps of 128
LDS_MAX = 160 * 1024

_cache = {}


def _case(K):
    if K not in _cache:
        mx = lib_or_fail()
        a = W.dense_activation(600, K, "plain", seed=21)
        w = W.dense_weight(N_TEST, K, seed=22)
        qw, sw = O.quantize_mx(w)
        qa, sa = O.quantize_mx(a)
        exact = O.gemm_from_mx(qa, sa, qw, sw)
        _cache[K] = (a, mx.mx_prepare_weight(dev_bf16(w)), exact)
    return _cache[K]


def _run(cfg, a, wp, ws):
    mx = lib_or_fail()
    os.environ["MX_GEMM_CONFIG"] = cfg
    try:
        return host_bits(mx.mx_a4w4_gemm(dev_bf16(a), wp, N_TEST, workspace=ws))
    finally:
        del os.environ["MX_GEMM_CONFIG"]


def _stream_lds(M, TS, MT, NG, WK):
    R = min(M, 16 * MT)
    return max(R * (TS * 64 + 16) + R * 4 * TS, WK * NG * MT * 1024)


@pytest.mark.parametrize("K", K_TESTS)
@pytest.mark.parametrize("mt,ng,wk", STREAM, ids=[f"s{c}" for c in STREAM])
def test_stream_config(mt, ng, wk, K):
    torch = torch_or_skip()
    a, wp, exact = _case(K)
    T = K // 128
    M = 16 * mt - 3
    ws = torch.empty(16 * M * N_TEST * 4, dtype=torch.uint8, device="cuda")
    splits = [s for s in (1, 3, 16) if s <= T and _stream_lds(M, -(-T // s), mt, ng, wk) <= LDS_MAX]
    assert splits
    for S in splits:
        c = _run(f"s,{mt},{ng},{wk},{S}", a[:M], wp, ws)
        torch.cuda.synchronize()
        check_gemm(c, exact[:M], what=f"stream {mt},{ng},{wk} S={S} K={K}")


@pytest.mark.parametrize("K", K_TESTS)
@pytest.mark.parametrize("cfg", TILE, ids=[f"t{c}" for c in TILE])
def test_tile_config(cfg, K):
    torch = torch_or_skip()
    a, wp, exact = _case(K)
    for M, gm in ((100, 1), (300, 8), (37, 3)):
        c = _run("t," + ",".join(map(str, cfg[:5])) + f",{gm},{cfg[5]}", a[:M], wp, False)
        torch.cuda.synchronize()
        check_gemm(c, exact[:M], what=f"tile {cfg} GM={gm} M={M} K={K}")
    # K slices (FP32 partials in the workspace, reduced in slice order); 4 slices of 6 steps
    # leave an uneven last slice at K = 4224
    for M, S in ((100, 3), (37, 4)):
        ws = torch.empty(S * M * N_TEST * 4, dtype=torch.uint8, device="cuda")
        c = _run("t," + ",".join(map(str, cfg[:5])) + f",8,{cfg[5]},{S}", a[:M], wp, ws)
        torch.cuda.synchronize()
        check_gemm(c, exact[:M], what=f"tile {cfg} S={S} M={M} K={K}")


def test_tile_split_needs_workspace():
    """A sliced tiled override without room for its partials fails instead of running."""
    torch_or_skip()
    mx = lib_or_fail()
    a, wp, _ = _case(4224)
    os.environ["MX_GEMM_CONFIG"] = "t,1,4,4,4,1,8,2,3"
    try:
        with pytest.raises(mx.MxError):
            mx.mx_a4w4_gemm(dev_bf16(a[:64]), wp, N_TEST, workspace=False)
    finally:
        del os.environ["MX_GEMM_CONFIG"]


@pytest.mark.parametrize("K", K_TESTS + (7168,))
@pytest.mark.parametrize("cfg", QO, ids=[f"q{c}" for c in QO])
def test_quantize_once_config(cfg, K):
    """The quantize-once kernel (activations quantized once into the workspace, then two
    prepared operands multiplied) on a ragged last row tile (300 rows: 256 + 44, or 2 x 128 +
    44), a tile of fewer rows than one 64-row quad (37), several tile orders, tail column tiles
    (N = 768 = 3 x 256) and canary rows past M. Its per-element sum runs over K steps in order,
    as in the tiled inline kernel, so the two are also compared bit for bit."""
    torch = torch_or_skip()
    mx = lib_or_fail()
    a, wp, exact = _case(K)
    for M, gm in ((300, 8), (37, 1), (256, 3)):
        full = torch.full((M + 5, N_TEST), -7.0, dtype=torch.bfloat16, device="cuda")
        ws = torch.empty((M + 63) // 64 * 64 * K * 17 // 32, dtype=torch.uint8, device="cuda")
        os.environ["MX_GEMM_CONFIG"] = "q," + ",".join(map(str, cfg)) + f",{gm}"
        try:
            mx.mx_a4w4_gemm(dev_bf16(a[:M]), wp, N_TEST, out=full[:M], workspace=ws)
        finally:
            del os.environ["MX_GEMM_CONFIG"]
        torch.cuda.synchronize()
        got = host_bits(full[:M])
        check_gemm(got, exact[:M], what=f"quantize-once {cfg} GM={gm} M={M} K={K}")
        assert bool((full[M:] == -7.0).all()), f"quantize-once {cfg} M={M} K={K}: rows past M were written"
        inline = _run("t,1,4,4,4,1,8,2", a[:M], wp, False)
        torch.cuda.synchronize()
        assert np.array_equal(got, inline), f"quantize-once {cfg} M={M} K={K}: differs from the inline kernel"


@pytest.mark.parametrize("K", (128, 256, 512) + K_TESTS + (7168,))
@pytest.mark.parametrize("cfg", QR, ids=[f"r{c}" for c in QR])
def test_register_direct_config(cfg, K):
    """The register-direct quantize-once kernel (one wave per 128 x 16 NG tile, operands D
    steps ahead in registers) at every remainder of its ring of two or three steps (T = 1, 2,
    4, 6, 33, 56 steps), on a ragged last row tile, a tile of fewer rows than one 64-row quad,
    several tile orders and canary rows past M. At N = 768 the 128 x 144 tiles start at every
    byte of a weight scale word (first groups 0, 9, 18, 27, ...) and the last one holds 48
    columns; at M = 600 the 144 x 128 tiles start at every byte of an activation scale word
    and the last one holds 24 rows. Compared with the oracle and bit for bit with the inline
    kernel (same per-element K order)."""
    torch = torch_or_skip()
    mx = lib_or_fail()
    a, wp, exact = _case(K)
    for M, gm in ((300, 8), (37, 1), (256, 3), (600, 2)):
        full = torch.full((M + 5, N_TEST), -7.0, dtype=torch.bfloat16, device="cuda")
        ws = torch.empty((M + 63) // 64 * 64 * K * 17 // 32, dtype=torch.uint8, device="cuda")
        os.environ["MX_GEMM_CONFIG"] = "r," + ",".join(map(str, cfg)) + f",{gm}"
        try:
            mx.mx_a4w4_gemm(dev_bf16(a[:M]), wp, N_TEST, out=full[:M], workspace=ws)
        finally:
            del os.environ["MX_GEMM_CONFIG"]
        torch.cuda.synchronize()
        got = host_bits(full[:M])
        check_gemm(got, exact[:M], what=f"register-direct {cfg} GM={gm} M={M} K={K}")
        assert bool((full[M:] == -7.0).all()), f"register-direct {cfg} M={M} K={K}: rows past M were written"
        inline = _run("t,1,4,4,4,1,8,2", a[:M], wp, False)
        torch.cuda.synchronize()
        assert np.array_equal(got, inline), f"register-direct {cfg} M={M} K={K}: differs from the inline kernel"


@pytest.mark.parametrize("K,slices", ((512, 1), (640, 1), (768, 1), (4224, 1), (4224, 2), (4224, 8), (7168, 3)))
@pytest.mark.parametrize("cfg", QK, ids=[f"x{c}" for c in QK])
def test_four_wave_config(cfg, K, slices):
    """Four register-direct waves per 128 x 16 NG tile, each over a quarter of the CTA's K
    range (T = 4, 5 (one wave with no step), 6, 33, 56 steps), added through LDS in wave order,
    with and without K slices across CTAs (FP32 partials added by the split-K reduce); on a
    ragged last row tile, a tile of fewer rows than one 64-row quad, several tile orders and
    canary rows past M. Tile widths 48, 96, 112 and 144 start at every byte offset within a
    weight scale word, and at N = 768 the last 112- and 144-wide tiles are partial. Compared with the
    oracle (the sum order differs from the inline kernel's)."""
    torch = torch_or_skip()
    mx = lib_or_fail()
    a, wp, exact = _case(K)
    for M, gm in ((300, 8), (37, 1), (256, 3)):
        full = torch.full((M + 5, N_TEST), -7.0, dtype=torch.bfloat16, device="cuda")
        act = (M + 63) // 64 * 64 * K * 17 // 32
        ws = torch.empty((act + 255) // 256 * 256 + slices * M * N_TEST * 4, dtype=torch.uint8, device="cuda")
        os.environ["MX_GEMM_CONFIG"] = "x," + ",".join(map(str, cfg)) + f",{gm},{slices}"
        try:
            mx.mx_a4w4_gemm(dev_bf16(a[:M]), wp, N_TEST, out=full[:M], workspace=ws)
        finally:
            del os.environ["MX_GEMM_CONFIG"]
        torch.cuda.synchronize()
        check_gemm(host_bits(full[:M]), exact[:M], what=f"four-wave {cfg} S={slices} GM={gm} M={M} K={K}")
        assert bool((full[M:] == -7.0).all()), f"four-wave {cfg} M={M} K={K}: rows past M were written"


def _logical_tile(logical, tiles_m, tiles_n, gm):
    """(tile row, tile column) of a logical tile: GM tile-rows at a time, rows first (the
    kernels' tile order)."""
    gsize = gm * tiles_n
    grp, rem = divmod(logical, gsize)
    first = grp * gm
    g = min(tiles_m - first, gm)
    return first + rem % g, rem // g


@pytest.mark.parametrize("K,slices", ((512, 4), (640, 4), (768, 4), (768, 3)))
def test_register_direct_tail_slices(K, slices):
    """More 128 x 128 tiles than one wave per SIMD of the chip (1152 > 1024 at M = 1152,
    N = 16384): the last 128 logical tiles run as K slices (with a slice of one step, of a
    remainder, and an empty one at T = 6 over 4 slices) whose FP32 partials are added in slice
    order. Every tile is checked against the oracle; the whole-tile tiles must equal, bit for
    bit, the run without the split."""
    torch = torch_or_skip()
    mx = lib_or_fail()
    M, N, gm = 1152, 16384, 8
    a = W.dense_activation(M, K, "plain", seed=25)
    w = W.dense_weight(N, K, seed=26)
    qa, sa = O.quantize_mx(a)
    qw, sw = O.quantize_mx(w)
    exact = O.gemm_from_mx(qa, sa, qw, sw)
    wp = mx.mx_prepare_weight(dev_bf16(w))
    ad = dev_bf16(a)
    outs = {}
    for sl in (1, slices):
        cfg = f"r,8,8,2,{gm},{sl}"
        os.environ["MX_GEMM_CONFIG"] = cfg
        try:
            plan = mx.mx_a4w4_gemm_plan(M, N, K, 1 << 31)
            assert (f"tail=128x{sl}" in plan) == (sl > 1), plan
            out = torch.full((M + 3, N), -7.0, dtype=torch.bfloat16, device="cuda")
            ws = torch.empty(48 << 20, dtype=torch.uint8, device="cuda")  # activations + 128 x 4 partial tiles
            mx.mx_a4w4_gemm(ad, wp, N, out=out[:M], workspace=ws)
        finally:
            del os.environ["MX_GEMM_CONFIG"]
        torch.cuda.synchronize()
        assert bool((out[M:] == -7.0).all()), f"{cfg}: rows past M were written"
        outs[sl] = host_bits(out[:M])
        check_gemm(outs[sl], exact, what=f"register-direct {cfg} M={M} N={N} K={K}")
    tiles_m, tiles_n = M // 128, N // 128
    tail = tiles_m * tiles_n - 1024
    same = np.ones((M, N), dtype=bool)
    for v in range(tail):
        bm, bn = _logical_tile(1024 + v, tiles_m, tiles_n, gm)
        same[bm * 128:(bm + 1) * 128, bn * 128:(bn + 1) * 128] = False
    assert np.array_equal(outs[1][same], outs[slices][same]), "whole tiles changed with the tail split"


def test_quantize_once_needs_workspace():
    """A forced quantize-once configuration without room for the quantized activations fails
    instead of running."""
    torch = torch_or_skip()
    mx = lib_or_fail()
    a, wp, _ = _case(4224)
    os.environ["MX_GEMM_CONFIG"] = "q,2,2,4,4,4,2,8"
    try:
        with pytest.raises(mx.MxError):
            mx.mx_a4w4_gemm(dev_bf16(a[:64]), wp, N_TEST, workspace=False)
        small = torch.empty(64 * 4224 * 17 // 32 - 16, dtype=torch.uint8, device="cuda")
        with pytest.raises(mx.MxError):
            mx.mx_a4w4_gemm(dev_bf16(a[:64]), wp, N_TEST, workspace=small)
    finally:
        del os.environ["MX_GEMM_CONFIG"]


@pytest.mark.parametrize("K", SWEEP_K)
@pytest.mark.parametrize("J", (2, 4))
def test_sweep_config(J, K):
    """The short-K sweep kernel (each 128-row tile quantized once, J column tiles of 128 per
    CTA): a ragged last row tile (300 = 2 x 128 + 44; 37 rows alone), a CTA with only some
    of its column tiles (N = 768 = 6 x 128 with J = 4), several tile orders, and canary
    rows past M that must stay untouched."""
    torch = torch_or_skip()
    a, wp, exact = _case(K)
    for M, gm in ((300, 8), (37, 1), (256, 3)):
        full = torch.full((M + 5, N_TEST), -7.0, dtype=torch.bfloat16, device="cuda")
        os.environ["MX_GEMM_CONFIG"] = f"k,{J},{gm}"
        try:
            mx = lib_or_fail()
            mx.mx_a4w4_gemm(dev_bf16(a[:M]), wp, N_TEST, out=full[:M], workspace=False)
        finally:
            del os.environ["MX_GEMM_CONFIG"]
        torch.cuda.synchronize()
        check_gemm(host_bits(full[:M]), exact[:M], what=f"sweep J={J} GM={gm} M={M} K={K}")
        assert bool((full[M:] == -7.0).all()), f"sweep J={J} M={M} K={K}: rows past M were written"


def test_sweep_rejects_long_k():
    """The sweep kernel holds a row tile's whole K in LDS: an override at K = 4224 (33
    steps, not compiled) fails instead of running."""
    torch_or_skip()
    mx = lib_or_fail()
    a, wp, _ = _case(4224)
    os.environ["MX_GEMM_CONFIG"] = "k,2,8"
    try:
        with pytest.raises(mx.MxError):
            mx.mx_a4w4_gemm(dev_bf16(a[:64]), wp, N_TEST, workspace=False)
    finally:
        del os.environ["MX_GEMM_CONFIG"]


def test_invalid_override_fails_loudly():
    torch_or_skip()
    mx = lib_or_fail()
    a, wp, _ = _case(768)
    # not compiled, malformed, and a streaming choice that cannot cover M = 40
    for bad, M in (("s,3,1,4,1", 5), ("t,9,9,9,9,9,9", 5), ("garbage", 5), ("s,1,1,4,1", 40)):
        os.environ["MX_GEMM_CONFIG"] = bad
        try:
            with pytest.raises(mx.MxError):
                mx.mx_a4w4_gemm(dev_bf16(a[:M]), wp, N_TEST, workspace=False)
        finally:
            del os.environ["MX_GEMM_CONFIG"]
