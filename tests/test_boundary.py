"""The C ABI boundary on the host: the library loads, exports every function that the
headers under include/ declare, sizes its buffers as documented, and rejects bad arguments
synchronously (before any HIP call, so these run without a GPU)."""
import ctypes
import glob
import os
import re

import pytest

import mxfp4_quantized_gemm_inline_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

pytestmark = pytest.mark.skipif(not os.path.exists(mx.LIB_PATH), reason="libmxgemm.so not built")

A = 0x10000   # fake, 16-byte aligned addresses: every call below returns before using them
B = 0x20000
Cp = 0x30000
MIS = 0x10008  # 8-byte aligned only


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    assert [os.path.basename(h) for h in HEADERS] == ["mx.h", "mx_calib.h"]
    names = declared_functions()
    assert len(names) >= 12 and "mx_calib_mfma" in names
    lib = mx.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(mx.SIGNATURES), "binding and header disagree"


def test_status_strings():
    for s in range(7):
        assert mx.status_string(s).startswith("MX_")
    assert "UNKNOWN" in mx.status_string(99)


def test_prepared_bytes():
    assert mx.mx_prepared_weight_bytes(8448, 7168) == 32_169_984      # the page's figure
    assert mx.mx_prepared_weight_bytes(7168, 768) == 7168 * 768 * 17 // 32
    assert mx.mx_prepared_weight_bytes(7168, 4224) == 7168 * 4224 * 17 // 32
    assert mx.mx_prepared_weight_bytes(1536, 3584) == 2_924_544
    for n, k in [(0, 256), (256, 0), (100, 256), (256, 100), (-256, 256), (256, 64)]:
        assert mx.mx_prepared_weight_bytes(n, k) == 0
    assert mx.mx_prepared_layout_version() == 2
    assert mx.mx_a4w4_gemm_workspace_bytes(1, 7168, 768) >= 0


def test_gemm_argument_errors():
    f = mx.lib().mx_a4w4_gemm
    assert f(A, B, Cp, 16, 100, 256, None, 0, None) == mx.MX_ERR_SHAPE
    assert f(A, B, Cp, 16, 256, 100, None, 0, None) == mx.MX_ERR_SHAPE
    assert f(A, B, Cp, -1, 256, 256, None, 0, None) == mx.MX_ERR_SHAPE
    assert f(A, B, Cp, 0, 256, 256, None, 0, None) == mx.MX_OK          # M = 0 is a no-op
    assert f(None, B, Cp, 16, 256, 256, None, 0, None) == mx.MX_ERR_NULL
    assert f(A, None, Cp, 16, 256, 256, None, 0, None) == mx.MX_ERR_NULL
    assert f(A, B, None, 16, 256, 256, None, 0, None) == mx.MX_ERR_NULL
    assert f(MIS, B, Cp, 16, 256, 256, None, 0, None) == mx.MX_ERR_ALIGN
    assert f(A, MIS, Cp, 16, 256, 256, None, 0, None) == mx.MX_ERR_ALIGN
    assert f(A, B, MIS, 16, 256, 256, None, 0, None) == mx.MX_ERR_ALIGN


def test_quant_and_prepare_argument_errors():
    q = mx.lib().mx_quant_act
    assert q(A, 4, 33, B, Cp, None) == mx.MX_ERR_SHAPE
    assert q(A, -1, 64, B, Cp, None) == mx.MX_ERR_SHAPE
    assert q(A, 0, 64, B, Cp, None) == mx.MX_OK
    assert q(None, 4, 64, B, Cp, None) == mx.MX_ERR_NULL
    assert q(A, 4, 64, MIS, Cp, None) == mx.MX_ERR_ALIGN
    p = mx.lib().mx_prepare_weight
    assert p(None, 256, 256, B, None) == mx.MX_ERR_NULL
    assert p(A, 255, 256, B, None) == mx.MX_ERR_SHAPE
    assert p(A, 256, 256, MIS, None) == mx.MX_ERR_ALIGN
    u = mx.lib().mx_unprepare_weight
    assert u(A, 256, 128 + 64, B, Cp, None) == mx.MX_ERR_SHAPE
    assert u(A, 256, 256, None, Cp, None) == mx.MX_ERR_NULL
    pk = mx.lib().mx_prepare_weight_packed
    #         fp4 scale N    K    prep stream
    assert pk(None, B, 256, 256, Cp, None) == mx.MX_ERR_NULL
    assert pk(A, None, 256, 256, Cp, None) == mx.MX_ERR_NULL
    assert pk(A, B, 256, 256, None, None) == mx.MX_ERR_NULL
    assert pk(A, B, 512 + 64, 256, Cp, None) == mx.MX_ERR_SHAPE
    assert pk(A, B, 256, 128 + 32, Cp, None) == mx.MX_ERR_SHAPE
    assert pk(A, B, 256, 0, Cp, None) == mx.MX_ERR_SHAPE
    assert pk(MIS, B, 256, 256, Cp, None) == mx.MX_ERR_ALIGN
    assert pk(A, MIS, 256, 256, Cp, None) == mx.MX_ERR_ALIGN
    assert pk(A, B, 256, 256, MIS, None) == mx.MX_ERR_ALIGN


def test_grouped_argument_errors():
    g = mx.lib().mx_a4w4_gemm_grouped
    #       a  rt  offs E   Rmax w   c   T   N    K    hint stream
    assert g(A, B, Cp, 0, 16, A, B, 1, 256, 256, 1, None) == mx.MX_ERR_SHAPE
    assert g(A, B, Cp, 4, 16, A, B, 1, 100, 256, 1, None) == mx.MX_ERR_SHAPE
    assert g(A, B, Cp, 4, -1, A, B, 1, 256, 256, 1, None) == mx.MX_ERR_SHAPE
    assert g(A, B, None, 4, 16, A, B, 1, 256, 256, 1, None) == mx.MX_ERR_NULL
    assert g(A, None, Cp, 4, 16, A, B, 1, 256, 256, 1, None) == mx.MX_ERR_NULL
    assert g(None, B, Cp, 4, 16, A, B, 1, 256, 256, 1, None) == mx.MX_ERR_NULL
    assert g(A, B, Cp, 4, 16, MIS, B, 1, 256, 256, 1, None) == mx.MX_ERR_ALIGN
    assert g(A, B, Cp, 4, 0, A, B, 1, 256, 256, 1, None) == mx.MX_OK     # no rows: no-op


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(mx, "_lib", None)
    monkeypatch.setattr(mx, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        mx.lib()


def test_gemm_plan_names_the_selected_kernel(monkeypatch):
    monkeypatch.delenv("MX_GEMM_CONFIG", raising=False)
    assert mx.mx_a4w4_gemm_plan(0, 7168, 768) == "none"
    assert mx.mx_a4w4_gemm_plan(1, 7168, 768).startswith("k_gemm_stream<1, ")
    assert mx.mx_a4w4_gemm_plan(2048, 7168, 768) == "k_gemm_sweep<2, 4, 4, 2, 6, 9, 4> GM=8"
    assert mx.mx_a4w4_gemm_plan(1024, 7168, 768) == "k_gemm_tile<1, 4, 4, 4, 1, 2> GM=8"
    # many rows at long K: the activations are quantized once into the workspace (k_prepare),
    # then both prepared operands are multiplied (k_gemm_qo); without that workspace the
    # inline kernels run
    assert mx.mx_a4w4_gemm_plan(2048, 7168, 4224) == "k_prepare + k_gemm_qo<2, 4, 8, 4, 4, 2> GM=8"
    # 1056 tiles of 128 x 128, a little over one wave per SIMD: the register-direct kernel on
    # 944 tiles of 128 x 144; 144 x 128 tiles when only those fit one round (M = 2304 at N =
    # 8192: 1026 of 128 x 144, 1024 of 144 x 128); at 1188 tiles (M = 2304 at N = 8448) both
    # still exceed it (1062, 1056), so 128 x 128 tiles run with the 164 past the first round in
    # four K slices
    assert mx.mx_a4w4_gemm_plan(2048, 8448, 7168) == "k_prepare + k_gemm_qr<8, 9, 1> GM=8"
    assert mx.mx_a4w4_gemm_plan(2304, 8192, 7168) == "k_prepare + k_gemm_qr<9, 8, 1> GM=8"
    assert mx.mx_a4w4_gemm_plan(2304, 8448, 7168) == \
        "k_prepare + k_gemm_qr<8, 8, 2> GM=8 tail=164x4 + k_qr_tail_reduce"
    # one CTA of four register-direct waves per tile, the narrowest tile that fits one round
    # of 256 CTAs: 236 of 128 x 144, 256 of 128 x 96
    assert mx.mx_a4w4_gemm_plan(512, 8448, 7168) == "k_prepare + k_gemm_qk<8, 9, 1> GM=4"
    assert mx.mx_a4w4_gemm_plan(2048, 1536, 7168) == "k_prepare + k_gemm_qk<8, 6, 2> GM=4"
    assert mx.mx_a4w4_gemm_plan(2048, 7168, 4224, workspace_bytes=0) == "k_gemm_tile<1, 8, 8, 4, 1, 2> GM=8"
    assert mx.mx_a4w4_gemm_plan(2048, 8448, 7168, workspace_bytes=0) == "k_gemm_tile<1, 4, 4, 4, 1, 2> GM=8"
    # the quantize-once workspace: the activations of M rows padded to 64, in the prepared layout
    # (then, for the register-direct kernel, 256-byte aligned FP32 partials of its tail slices)
    act = 2048 * 7168 * 17 // 32
    assert mx.mx_a4w4_gemm_workspace_bytes(2048, 8448, 7168) == (act + 255) // 256 * 256
    act_t = (2304 * 7168 * 17 // 32 + 255) // 256 * 256
    assert mx.mx_a4w4_gemm_workspace_bytes(2304, 8448, 7168) == act_t + 164 * 4 * 128 * 128 * 4
    assert mx.mx_a4w4_gemm_workspace_bytes(520, 8448, 7168) == 576 * 7168 * 17 // 32
    assert mx.mx_a4w4_gemm_plan(2048, 8448, 7168, workspace_bytes=act) == "k_prepare + k_gemm_qr<8, 9, 1> GM=8"
    assert mx.mx_a4w4_gemm_plan(2048, 8448, 7168, workspace_bytes=act - 1).startswith("k_gemm_tile<")
    # no room for the tail partials: the LDS quantize-once kernel
    assert mx.mx_a4w4_gemm_plan(2304, 8448, 7168, workspace_bytes=act_t) == \
        "k_prepare + k_gemm_qo<2, 2, 4, 4, 4, 2> GM=8"
    # N = 1536 at M = 512 gives 48 tiles of 128 x 128, too few for the LDS kernel; 128 tiles of
    # 128 x 48 run four waves each over K quarters
    assert mx.mx_a4w4_gemm_plan(512, 1536, 7168) == "k_prepare + k_gemm_qk<8, 3, 4> GM=4"
    assert mx.mx_a4w4_gemm_plan(384, 1536, 7168).startswith("k_gemm_tile<")   # 96 such tiles
    # mid M: 64 x 64 tiles while the activation re-reads stay modest, K slices beyond
    assert mx.mx_a4w4_gemm_plan(128, 7168, 768) == "k_gemm_tile<1, 4, 4, 1, 2, 2> GM=8"
    assert mx.mx_a4w4_gemm_plan(100, 7168, 4224) == "k_prepare + k_gemm_qk<8, 3, 4> GM=1"
    assert mx.mx_a4w4_gemm_plan(100, 7168, 4224, workspace_bytes=0) == "k_gemm_tile<1, 4, 4, 1, 2, 2> GM=8"
    assert mx.mx_a4w4_gemm_plan(96, 7168, 4224).startswith("k_gemm_")   # not the four-wave kernel
    assert "k_gemm_qk" not in mx.mx_a4w4_gemm_plan(96, 7168, 4224)
    assert "k_splitk_reduce" in mx.mx_a4w4_gemm_plan(64, 8448, 7168)
    # 17..32 rows at 8448 x 7168: 64 x 256 tiles in as many K slices as fit one CTA per CU (33 x 7)
    assert mx.mx_a4w4_gemm_plan(32, 8448, 7168) == "k_gemm_tile<1, 4, 4, 4, 2, 2> GM=8 S=7 + k_splitk_reduce"
    assert mx.mx_a4w4_gemm_plan(17, 8448, 7168) == "k_gemm_tile<1, 4, 4, 4, 2, 2> GM=8 S=7 + k_splitk_reduce"
    assert mx.mx_a4w4_gemm_plan(32, 8448, 7168, workspace_bytes=4 * 32 * 8448 * 4) == \
        "k_gemm_tile<1, 4, 4, 4, 2, 2> GM=8 S=4 + k_splitk_reduce"
    assert mx.mx_a4w4_gemm_plan(32, 16384, 7168) == "k_gemm_tile<1, 4, 4, 4, 2, 2> GM=8 S=4 + k_splitk_reduce"
    assert mx.mx_a4w4_gemm_plan(32, 8448, 7168, workspace_bytes=0).startswith("k_gemm_stream<")
    # one 128-row tile at long K: 176 CTAs of 128 x 48, four waves over K quarters
    assert mx.mx_a4w4_gemm_plan(128, 8448, 7168) == "k_prepare + k_gemm_qk<8, 3, 4> GM=1"
    assert mx.mx_a4w4_gemm_plan(128, 8448, 7168, workspace_bytes=0).startswith("k_gemm_tile<")
    # split K only with a workspace; the streaming kernels never need one otherwise
    with_ws = mx.mx_a4w4_gemm_plan(32, 1536, 7168)
    no_ws = mx.mx_a4w4_gemm_plan(32, 1536, 7168, workspace_bytes=0)
    assert "k_splitk_reduce" in with_ws and "S=1" in no_ws and "k_splitk_reduce" not in no_ws
    monkeypatch.setenv("MX_GEMM_CONFIG", "t,1,4,4,4,2,16,2")
    assert mx.mx_a4w4_gemm_plan(64, 7168, 768) == "k_gemm_tile<1, 4, 4, 4, 2, 2> GM=16"
    monkeypatch.setenv("MX_GEMM_CONFIG", "t,9,9,9,9,9,9")
    with pytest.raises(mx.MxError):
        mx.mx_a4w4_gemm_plan(64, 7168, 768)
    # the short-K sweep kernel exists for 2, 4, 6 and 8 steps of K and one or two column tiles
    monkeypatch.setenv("MX_GEMM_CONFIG", "k,2,8")
    assert mx.mx_a4w4_gemm_plan(2048, 7168, 768) == "k_gemm_sweep<2, 4, 4, 2, 6, 9, 2> GM=8"
    assert mx.mx_a4w4_gemm_plan(300, 768, 256) == "k_gemm_sweep<2, 4, 4, 2, 2, 3, 2> GM=8"
    for K in (384, 4224):
        with pytest.raises(mx.MxError):
            mx.mx_a4w4_gemm_plan(2048, 7168, K)
    monkeypatch.setenv("MX_GEMM_CONFIG", "k,3,8")
    with pytest.raises(mx.MxError):
        mx.mx_a4w4_gemm_plan(2048, 7168, 768)
    # the quantize-once kernel can be forced (it needs its workspace) at any shape
    monkeypatch.setenv("MX_GEMM_CONFIG", "q,2,2,4,4,5,2,3")
    ws = 64 * 768 * 17 // 32
    assert mx.mx_a4w4_gemm_plan(37, 768, 768, ws) == "k_prepare + k_gemm_qo<2, 2, 4, 4, 5, 2> GM=3"
    with pytest.raises(mx.MxError):
        mx.mx_a4w4_gemm_plan(37, 768, 768, ws - 1)
    monkeypatch.setenv("MX_GEMM_CONFIG", "q,2,2,4,4,9,2,3")  # not compiled
    with pytest.raises(mx.MxError):
        mx.mx_a4w4_gemm_plan(37, 768, 768, ws)


def test_a16w4_plan_names_the_selected_kernel():
    assert mx.mx_a16w4_gemm_plan(0, 7168, 768) == "none"
    assert mx.mx_a16w4_gemm_plan(1, 7168, 768) == "k_gemm_a16w4_stream<1, 2, 4, 2>"
    assert mx.mx_a16w4_gemm_plan(16, 8448, 7168) == "k_gemm_a16w4_stream<1, 1, 8, 8>"
    assert mx.mx_a16w4_gemm_plan(17, 7168, 768) == "k_gemm_a16w4_stream<2, 2, 4, 2>"
    assert mx.mx_a16w4_gemm_plan(32, 8448, 7168) == "k_gemm_a16w4_stream<2, 1, 8, 4>"
    # tiled form: the widest tile that still gives about 200 CTAs
    assert mx.mx_a16w4_gemm_plan(33, 7168, 768) == "k_gemm_a16w4<1, 2> (64 x 64 tiles)"
    assert mx.mx_a16w4_gemm_plan(128, 7168, 768) == "k_gemm_a16w4<1, 2> (64 x 64 tiles)"
    assert mx.mx_a16w4_gemm_plan(256, 7168, 768) == "k_gemm_a16w4<2, 2> (64 x 128 tiles)"
    assert mx.mx_a16w4_gemm_plan(2048, 7168, 768) == "k_gemm_a16w4<4, 2> (64 x 256 tiles)"
    for bad in ((1, 100, 768), (1, 7168, 100), (-1, 7168, 768)):
        with pytest.raises(mx.MxError):
            mx.mx_a16w4_gemm_plan(*bad)


def test_grouped_plan_names_the_selected_kernel(monkeypatch):
    monkeypatch.delenv("MX_GROUPED_CONFIG", raising=False)
    N, K, E = 1536, 3584, 896
    assert mx.mx_a4w4_gemm_grouped_plan(E, 0, 0, N, K) == "none"
    assert mx.mx_a4w4_gemm_grouped_plan(E, 16, 1, N, K).startswith("k_gemm_grouped<1, 1, 4, ")
    # segments of about 5 rows (256 tokens): 64 x 256 tiles; about 73 rows (4096 tokens): 128 x 512
    assert mx.mx_a4w4_gemm_grouped_plan(E, 4096, 256, N, K, 5) == "k_gemm_grouped_tile<1, 4, 4, 4, 2, 2>"
    assert mx.mx_a4w4_gemm_grouped_plan(E, 65536, 4096, N, K, 73) == "k_gemm_grouped_tile<1, 8, 8, 4, 1, 2>"
    # N = 768 is no multiple of 512: long segments stay on 64 x 256 tiles
    assert mx.mx_a4w4_gemm_grouped_plan(E, 65536, 4096, 768, K, 73) == "k_gemm_grouped_tile<1, 4, 4, 4, 2, 2>"
    monkeypatch.setenv("MX_GROUPED_CONFIG", "gs,2,4")
    assert mx.mx_a4w4_gemm_grouped_plan(E, 65536, 4096, N, K).startswith("k_gemm_grouped<2, 4, 4, ")
    monkeypatch.setenv("MX_GROUPED_CONFIG", "gt,1,4,4,4,3,2")
    with pytest.raises(mx.MxError):
        mx.mx_a4w4_gemm_grouped_plan(E, 65536, 4096, N, K)


def test_plan_argument_errors():
    f, g = mx.lib().mx_a4w4_gemm_plan, mx.lib().mx_a4w4_gemm_grouped_plan
    buf = ctypes.create_string_buffer(64)
    assert f(16, 100, 256, 0, buf, 64) == mx.MX_ERR_SHAPE
    assert f(16, 256, 256, 0, None, 64) == mx.MX_ERR_NULL
    assert f(16, 256, 256, 0, buf, 0) == mx.MX_ERR_NULL
    assert g(0, 16, 1, 256, 256, 1, buf, 64) == mx.MX_ERR_SHAPE
    assert g(4, 16, -1, 256, 256, 1, buf, 64) == mx.MX_ERR_SHAPE
    assert g(4, 16, 1, 256, 256, 1, None, 64) == mx.MX_ERR_NULL
    tiny = ctypes.create_string_buffer(8)  # truncated, still NUL-terminated
    assert f(2048, 7168, 768, 0, tiny, 8) == mx.MX_OK and tiny.value == b"k_gemm_"


def test_calibration_argument_errors():
    L = mx.lib()
    sink = 0x40000
    assert L.mx_calib_read(None, 1024, 8, sink, None) == mx.MX_ERR_NULL
    assert L.mx_calib_read(A, 1024, 8, None, None) == mx.MX_ERR_NULL
    assert L.mx_calib_read(A, 0, 8, sink, None) == mx.MX_ERR_SHAPE
    assert L.mx_calib_read(A, 1000, 8, sink, None) == mx.MX_ERR_SHAPE      # not a multiple of 16
    assert L.mx_calib_read(A, 1024, 0, sink, None) == mx.MX_ERR_SHAPE
    assert L.mx_calib_read(A, 1024, (1 << 20) + 1, sink, None) == mx.MX_ERR_SHAPE
    assert L.mx_calib_read(MIS, 1024, 8, sink, None) == mx.MX_ERR_ALIGN
    assert L.mx_calib_mfma(8, 16, None, None) == mx.MX_ERR_NULL
    assert L.mx_calib_mfma(0, 16, sink, None) == mx.MX_ERR_SHAPE
    assert L.mx_calib_mfma(8, 0, sink, None) == mx.MX_ERR_SHAPE
    assert L.mx_calib_mfma(8, (1 << 24) + 1, sink, None) == mx.MX_ERR_SHAPE
    # 256 CTAs x 4 waves x 100 rounds x 8 MFMAs x 65,536 flop
    assert mx.mx_calib_mfma_flops(256, 100) == 256 * 4 * 100 * 8 * 65536
    assert L.mx_calib_mfma_operands(None, 16384, 8, 16, sink, None) == mx.MX_ERR_NULL
    assert L.mx_calib_mfma_operands(A, 16384, 8, 16, None, None) == mx.MX_ERR_NULL
    assert L.mx_calib_mfma_operands(A, 16383, 8, 16, sink, None) == mx.MX_ERR_SHAPE  # less than one window
    assert L.mx_calib_mfma_operands(A, 16384, 0, 16, sink, None) == mx.MX_ERR_SHAPE
    assert L.mx_calib_mfma_operands(A, 16384, 8, 0, sink, None) == mx.MX_ERR_SHAPE
    assert L.mx_calib_mfma_operands(A, 16384, 8, (1 << 24) + 1, sink, None) == mx.MX_ERR_SHAPE
    assert L.mx_calib_mfma_operands(MIS, 16384, 8, 16, sink, None) == mx.MX_ERR_ALIGN
    # 256 CTAs x 4 waves x 100 rounds x 64 MFMAs x 65,536 flop
    assert mx.mx_calib_mfma_operands_flops(256, 100) == 256 * 4 * 100 * 64 * 65536
    clk = 0x80000
    f = L.mx_calib_mfma_operands_clock
    assert f(None, 16384, 8, 16, sink, clk, None) == mx.MX_ERR_NULL
    assert f(A, 16384, 8, 16, None, clk, None) == mx.MX_ERR_NULL
    assert f(A, 16384, 8, 16, sink, None, None) == mx.MX_ERR_NULL
    assert f(A, 16383, 8, 16, sink, clk, None) == mx.MX_ERR_SHAPE
    assert f(A, 16384, 0, 16, sink, clk, None) == mx.MX_ERR_SHAPE
    assert f(A, 16384, 8, 0, sink, clk, None) == mx.MX_ERR_SHAPE
    assert f(MIS, 16384, 8, 16, sink, clk, None) == mx.MX_ERR_ALIGN
    assert f(A, 16384, 8, 16, sink, clk + 4, None) == mx.MX_ERR_ALIGN  # clocks hold uint64


def test_gemm2_plan_picks_the_sweep_for_long_segments_at_short_k(monkeypatch):
    monkeypatch.delenv("MX_GROUPED_CONFIG", raising=False)
    plan = mx.mx_a4w4_gemm_grouped_mx_plan
    assert plan(3584, 768, 73) == "k_gemm_grouped_sweep_mx<6, 9, 14>"
    assert plan(1024, 512, 73) == "k_gemm_grouped_sweep_mx<4, 6, 4>"
    assert plan(3584, 768, 5).startswith("k_gemm_grouped_tile_mx<")
    assert plan(3584, 4224, 73).startswith("k_gemm_grouped_tile_mx<")  # 33 steps: not compiled
    monkeypatch.setenv("MX_GROUPED_CONFIG", "gk,4")
    assert plan(3584, 768, 5) == "k_gemm_grouped_sweep_mx<6, 9, 4>"
    monkeypatch.setenv("MX_GROUPED_CONFIG", "gk,5")
    with pytest.raises(mx.MxError):
        plan(3584, 768, 73)


def test_fused_act_quant_argument_errors_and_plan(monkeypatch):
    monkeypatch.delenv("MX_GROUPED_CONFIG", raising=False)
    f = mx.lib().mx_a4w4_gemm_grouped_act_quant
    #        a  rt  offs E  Rmax w  T  N     K    act hint hq  hs  stream
    assert f(A, B, Cp, 4, 16, A, 1, 1536, 3584, 2, 1, A, B, None) == mx.MX_ERR_SHAPE     # unknown act
    assert f(A, B, Cp, 4, 16, A, 1, 1000, 3584, 1, 1, A, B, None) == mx.MX_ERR_SHAPE
    assert f(A, B, Cp, 0, 16, A, 1, 1536, 3584, 1, 1, A, B, None) == mx.MX_ERR_SHAPE
    assert f(A, B, Cp, 4, 16, A, 1, 1536, 3584, 1, 1, None, B, None) == mx.MX_ERR_NULL
    assert f(A, B, Cp, 4, 16, A, 1, 1536, 3584, 1, 1, A, None, None) == mx.MX_ERR_NULL
    assert f(None, B, Cp, 4, 16, A, 1, 1536, 3584, 1, 1, A, B, None) == mx.MX_ERR_NULL
    assert f(A, B, Cp, 4, 16, A, 1, 1536, 3584, 1, 1, MIS, B, None) == mx.MX_ERR_ALIGN
    assert f(A, B, Cp, 4, 16, A, 1, 1536, 3584, 1, 1, A, MIS, None) == mx.MX_ERR_ALIGN
    assert f(A, B, Cp, 4, 0, A, 1, 1536, 3584, 1, 1, None, None, None) == mx.MX_OK       # no rows: no-op
    plan = mx.mx_a4w4_gemm_grouped_act_quant_plan
    assert plan(896, 65536, 1536, 3584, mx.MX_ACT_SWIGLU, 73) == "k_gemm_grouped_tile<1, 8, 8, 4, 1, 2, swiglu>"
    assert plan(896, 4096, 1536, 3584, mx.MX_ACT_SWIGLU, 5) == "k_gemm_grouped_tile<1, 4, 4, 4, 2, 2, swiglu>"
    assert plan(896, 65536, 768, 3584, mx.MX_ACT_SILU, 73) == "k_gemm_grouped_tile<1, 4, 4, 4, 2, 2, silu>"   # 768 % 512
    # a handful of rows (T = 1: 16 rows, 96 CTAs of 64 x 256): 64 x 128 tiles
    assert plan(896, 16, 1536, 3584, mx.MX_ACT_SWIGLU, 1) == "k_gemm_grouped_tile<1, 4, 4, 2, 2, 2, swiglu>"
    assert plan(896, 256, 1536, 3584, mx.MX_ACT_SWIGLU, 1) == "k_gemm_grouped_tile<1, 4, 4, 4, 2, 2, swiglu>"
    for bad in ((896, 16, 1536, 3584, 2, 1), (0, 16, 1536, 3584, 1, 1), (896, -1, 1536, 3584, 1, 1)):
        with pytest.raises(mx.MxError):
            plan(*bad)
    monkeypatch.setenv("MX_GROUPED_CONFIG", "gt,1,4,4,4,1,2")   # compiled, but not with the fused epilogue
    with pytest.raises(mx.MxError):
        plan(896, 16, 1536, 3584, mx.MX_ACT_SWIGLU, 1)


def test_gemm2_and_combine_argument_errors_and_plan(monkeypatch):
    monkeypatch.delenv("MX_GROUPED_CONFIG", raising=False)
    g = mx.lib().mx_a4w4_gemm_grouped_mx
    #        aq as  offs E  Rmax w  c   N     K    hint stream
    assert g(A, B, Cp, 0, 16, A, B, 3584, 768, 1, None) == mx.MX_ERR_SHAPE
    assert g(A, B, Cp, 4, 16, A, B, 3584, 700, 1, None) == mx.MX_ERR_SHAPE
    assert g(None, B, Cp, 4, 16, A, B, 3584, 768, 1, None) == mx.MX_ERR_NULL
    assert g(A, None, Cp, 4, 16, A, B, 3584, 768, 1, None) == mx.MX_ERR_NULL
    assert g(A, B, None, 4, 16, A, B, 3584, 768, 1, None) == mx.MX_ERR_NULL
    assert g(A, B, Cp, 4, 16, A, None, 3584, 768, 1, None) == mx.MX_ERR_NULL
    assert g(MIS, B, Cp, 4, 16, A, B, 3584, 768, 1, None) == mx.MX_ERR_ALIGN
    assert g(A, B, Cp, 4, 0, A, B, 3584, 768, 1, None) == mx.MX_OK          # no rows: no-op
    c = mx.lib().mx_moe_combine
    #        y  R   rows wts T  topk N   out stream
    assert c(A, 8, B, Cp, 0, 2, 64, A, None) == mx.MX_OK                     # no tokens: no-op
    assert c(A, 8, B, Cp, 4, 0, 64, A, None) == mx.MX_ERR_SHAPE
    assert c(A, 8, B, Cp, 4, 2, 60, A, None) == mx.MX_ERR_SHAPE
    assert c(A, -1, B, Cp, 4, 2, 64, A, None) == mx.MX_ERR_SHAPE
    assert c(A, 8, None, Cp, 4, 2, 64, A, None) == mx.MX_ERR_NULL
    assert c(None, 8, B, Cp, 4, 2, 64, A, None) == mx.MX_ERR_NULL
    assert c(A, 8, B, Cp, 4, 2, 64, MIS, None) == mx.MX_ERR_ALIGN
    assert c(A, 8, B + 2, Cp, 4, 2, 64, A, None) == mx.MX_ERR_ALIGN
    assert mx.mx_a4w4_gemm_grouped_mx_plan(3584, 768, 73) == "k_gemm_grouped_sweep_mx<6, 9, 14>"
    assert mx.mx_a4w4_gemm_grouped_mx_plan(3584, 768, 5) == "k_gemm_grouped_tile_mx<1, 4, 4, 4, 2, 2>"
    assert mx.mx_a4w4_gemm_grouped_mx_plan(768, 768, 73) == "k_gemm_grouped_sweep_mx<6, 9, 14>"


def test_a16w4_argument_errors():
    f = mx.lib().mx_a16w4_gemm
    assert f(A, B, Cp, 0, 256, 256, None) == mx.MX_OK              # M = 0: no-op
    assert f(A, B, Cp, -1, 256, 256, None) == mx.MX_ERR_SHAPE
    assert f(A, B, Cp, 4, 300, 256, None) == mx.MX_ERR_SHAPE
    assert f(A, B, Cp, 4, 256, 200, None) == mx.MX_ERR_SHAPE
    assert f(None, B, Cp, 4, 256, 256, None) == mx.MX_ERR_NULL
    assert f(A, None, Cp, 4, 256, 256, None) == mx.MX_ERR_NULL
    assert f(A, B, None, 4, 256, 256, None) == mx.MX_ERR_NULL
    assert f(MIS, B, Cp, 4, 256, 256, None) == mx.MX_ERR_ALIGN


def _meta(shape, dtype):
    import torch
    return torch.empty(shape, dtype=dtype, device="meta")


def test_binding_checks_sizes_before_any_pointer_is_taken():
    """Every wrapper validates shapes and sizes from tensor metadata before it takes a device
    pointer: a short weight blob, output or table would be read or written out of bounds by
    kernels that receive only pointers and sizes. Shape-only ("meta") tensors reach these
    checks without any device; a well-sized one then fails only for not being on a device."""
    torch = pytest.importorskip("torch")
    bf, u8, i32, f32 = torch.bfloat16, torch.uint8, torch.int32, torch.float32
    N, K, M = 512, 768, 40
    wbytes = mx.mx_prepared_weight_bytes(N, K)
    a, c = _meta((M, K), bf), _meta((M, N), bf)
    size_err = "needs at least|must have shape|must be 2-D|need at least"
    # dense GEMM and A16WFP4: the weight blob and the output
    for fn in (mx.mx_a4w4_gemm, mx.mx_a16w4_gemm):
        with pytest.raises(ValueError, match=size_err):
            fn(a, _meta((wbytes - 16,), u8), N, out=c)
        with pytest.raises(ValueError, match=size_err):
            fn(a, _meta((wbytes,), u8), N, out=_meta((M, N - 8), bf))
        with pytest.raises(ValueError, match=size_err):
            fn(_meta((M * K,), bf), _meta((wbytes,), u8), N, out=c)
        with pytest.raises(TypeError):
            fn(a, _meta((wbytes,), torch.int8), N, out=c)
        with pytest.raises(ValueError, match="device tensor"):   # sizes fine: only the device is missing
            fn(a, _meta((wbytes,), u8), N, out=c)
    # prepare / unprepare / standalone quantizer
    with pytest.raises(ValueError, match=size_err):
        mx.mx_prepare_weight(_meta((N, K), bf), out=_meta((wbytes - 1,), u8))
    with pytest.raises(ValueError, match=size_err):
        mx.mx_prepare_weight_packed(_meta((N, K // 2), u8), _meta((N, K // 32 - 1), u8))
    with pytest.raises(ValueError, match=size_err):
        mx.mx_prepare_weight_packed(_meta((N, K // 2), u8), _meta((N, K // 32), u8), out=_meta((wbytes - 1,), u8))
    with pytest.raises(ValueError, match=size_err):
        mx.mx_unprepare_weight(_meta((wbytes - 1,), u8), N, K)
    with pytest.raises(ValueError, match=size_err):
        mx.mx_quant_act(a, q_out=_meta((M, K // 2 - 1), u8), s_out=_meta((M, K // 32), u8))
    with pytest.raises(ValueError, match=size_err):
        mx.mx_quant_act(a, q_out=_meta((M, K // 2), u8), s_out=_meta((M - 1, K // 32), u8))
    # grouped calls: segment table, row map, stacked weights, outputs
    E, R, T, Nh = 6, 100, 20, N // 2
    at, rt, of = _meta((T, K), bf), _meta((R,), i32), _meta((E + 1,), i32)
    wst = _meta((E * wbytes,), u8)
    for bad in (dict(row_token=_meta((R - 1,), i32)), dict(expert_offsets=_meta((E,), i32)),
                dict(w_prep_stacked=_meta((E * wbytes - 1,), u8)), dict(out=_meta((R, N - 8), bf))):
        args = dict(row_token=rt, expert_offsets=of, w_prep_stacked=wst, out=_meta((R, N), bf))
        args.update(bad)
        with pytest.raises(ValueError, match=size_err):
            mx.mx_a4w4_gemm_grouped(at, args["row_token"], args["expert_offsets"], E, R, args["w_prep_stacked"], N,
                                    out=args["out"])
    with pytest.raises(ValueError, match=size_err):
        mx.mx_a4w4_gemm_grouped_act_quant(at, rt, of, E, R, wst, N, h_fp4=_meta((R, Nh // 2 - 1), u8),
                                          h_scale=_meta((R, Nh // 32), u8))
    with pytest.raises(ValueError, match=size_err):
        mx.mx_a4w4_gemm_grouped_act_quant(at, rt, _meta((E,), i32), E, R, wst, N)
    K2, N2 = 256, 512
    w2 = _meta((E * mx.mx_prepared_weight_bytes(N2, K2),), u8)
    with pytest.raises(ValueError, match=size_err):
        mx.mx_a4w4_gemm_grouped_mx(_meta((R - 1, K2 // 2), u8), _meta((R - 1, K2 // 32), u8), of, E, R, w2, N2)
    with pytest.raises(ValueError, match=size_err):
        mx.mx_a4w4_gemm_grouped_mx(_meta((R, K2 // 2), u8), _meta((R, K2 // 32), u8), of, E, R, w2[:-1], N2)
    with pytest.raises(ValueError, match=size_err):
        mx.mx_a4w4_gemm_grouped_mx(_meta((R, K2 // 2), u8), _meta((R, K2 // 32), u8), of, E, R, w2, N2,
                                   out=_meta((R - 1, N2), bf))
    # combine
    with pytest.raises(ValueError, match=size_err):
        mx.mx_moe_combine(_meta((R, N2), bf), _meta((T, 16), i32), _meta((T, 15), f32))
    with pytest.raises(ValueError, match=size_err):
        mx.mx_moe_combine(_meta((R, N2), bf), _meta((T, 16), i32), _meta((T, 16), f32), out=_meta((T, N2 - 8), bf))
    with pytest.raises(TypeError):
        mx.mx_moe_combine(_meta((R, N2), bf), _meta((T, 16), torch.int64), _meta((T, 16), f32))


def test_register_direct_override_plans(monkeypatch):
    """The tuning override for the register-direct quantize-once kernel: tail slices only
    when the tiles pass one wave per SIMD, a workspace that holds their partials, and no
    configuration that is not compiled."""
    monkeypatch.setenv("MX_GEMM_CONFIG", "r,8,8,2,8")
    assert mx.mx_a4w4_gemm_plan(2048, 7168, 4224) == "k_prepare + k_gemm_qr<8, 8, 2> GM=8"
    monkeypatch.setenv("MX_GEMM_CONFIG", "r,8,8,2,16,4")
    assert mx.mx_a4w4_gemm_plan(2048, 7168, 4224) == "k_prepare + k_gemm_qr<8, 8, 2> GM=16"  # 896 tiles
    big = 1 << 30
    assert mx.mx_a4w4_gemm_plan(2048, 8448, 7168, workspace_bytes=big) == \
        "k_prepare + k_gemm_qr<8, 8, 2> GM=16 tail=32x4 + k_qr_tail_reduce"
    act = (2048 * 7168 * 17 // 32 + 255) // 256 * 256
    with pytest.raises(mx.MxError):  # no room for the partials
        mx.mx_a4w4_gemm_plan(2048, 8448, 7168, workspace_bytes=act + 32 * 4 * 65536 - 1)
    # 128 x 144 tiles, one step ahead: 7168 / 144 leaves a last column tile of 112 columns
    monkeypatch.setenv("MX_GEMM_CONFIG", "r,8,9,1,4")
    assert mx.mx_a4w4_gemm_plan(2048, 7168, 4224) == "k_prepare + k_gemm_qr<8, 9, 1> GM=4"
    monkeypatch.setenv("MX_GEMM_CONFIG", "r,9,8,1,2")
    assert mx.mx_a4w4_gemm_plan(2048, 7168, 4224) == "k_prepare + k_gemm_qr<9, 8, 1> GM=2"
    for bad in ("r,8,8,3,8", "r,4,8,2,8", "r,8,8,2,8,17", "r,8,9,2,8", "r,8,10,1,8", "r,9,9,1,8"):
        monkeypatch.setenv("MX_GEMM_CONFIG", bad)
        with pytest.raises(mx.MxError):
            mx.mx_a4w4_gemm_plan(2048, 8448, 7168, workspace_bytes=big)


def test_four_wave_override_plans(monkeypatch):
    """The tuning override for the four-wave register-direct kernel: K slices need a
    workspace for their partials and at least one K step per wave."""
    monkeypatch.setenv("MX_GEMM_CONFIG", "x,8,8,2,8")
    assert mx.mx_a4w4_gemm_plan(512, 7168, 4224) == "k_prepare + k_gemm_qk<8, 8, 2> GM=8"
    monkeypatch.setenv("MX_GEMM_CONFIG", "x,8,8,2,8,3")
    act = (128 * 7168 * 17 // 32 + 255) // 256 * 256
    need = act + 3 * 128 * 8448 * 4
    assert mx.mx_a4w4_gemm_plan(128, 8448, 7168, workspace_bytes=need) == \
        "k_prepare + k_gemm_qk<8, 8, 2> GM=8 S=3 + k_splitk_reduce"
    with pytest.raises(mx.MxError):
        mx.mx_a4w4_gemm_plan(128, 8448, 7168, workspace_bytes=need - 1)
    monkeypatch.setenv("MX_GEMM_CONFIG", "x,8,8,2,8,2")
    with pytest.raises(mx.MxError):  # 6 steps cannot give 2 x 4 waves a step each
        mx.mx_a4w4_gemm_plan(512, 7168, 768, workspace_bytes=1 << 30)
    for cfg, plan in (("x,8,9,1,8", "k_gemm_qk<8, 9, 1> GM=8"), ("x,8,7,2,2", "k_gemm_qk<8, 7, 2> GM=2"),
                      ("x,8,6,2,4", "k_gemm_qk<8, 6, 2> GM=4")):
        monkeypatch.setenv("MX_GEMM_CONFIG", cfg)
        assert mx.mx_a4w4_gemm_plan(512, 7168, 4224) == "k_prepare + " + plan
    for bad in ("x,8,8,3,8", "x,4,4,2,8", "x,8,8,2,8,17", "x,8,9,2,8", "x,8,10,1,8"):
        monkeypatch.setenv("MX_GEMM_CONFIG", bad)
        with pytest.raises(mx.MxError):
            mx.mx_a4w4_gemm_plan(512, 7168, 4224, workspace_bytes=1 << 30)
