"""Inline-quantized A4W4 MXFP4 GEMM for MI355X (gfx950).

A thin Python binding over the C ABI in ``include/mx.h`` (``libmxgemm.so``, built
in-tree by ``python -m mxfp4_quantized_gemm_inline_amd.build``). Every function here
only marshals arguments: torch supplies device memory and the current HIP stream, and
all computation runs in the library's HIP kernels. There is no fallback: if the library
is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmxgemm.so")

# Symbols declared in include/mx.h, with ctypes signatures.
_c_i64, _c_sz, _vp, _c_int = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
SIGNATURES = {
    "mx_status_string": (ctypes.c_char_p, [_c_int]),
    "mx_prepared_layout_version": (_c_int, []),
    "mx_prepared_weight_bytes": (_c_sz, [_c_i64, _c_i64]),
    "mx_prepare_weight": (_c_int, [_vp, _c_i64, _c_i64, _vp, _vp]),
    "mx_prepare_weight_packed": (_c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _vp]),
    "mx_unprepare_weight": (_c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _vp]),
    "mx_quant_act": (_c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _vp]),
    "mx_a4w4_gemm_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64]),
    "mx_a4w4_gemm": (_c_int, [_vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _vp, _c_sz, _vp]),
    "mx_a4w4_gemm_grouped": (_c_int, [_vp, _vp, _vp, _c_i64, _c_i64, _vp, _vp, _c_i64, _c_i64,
                                      _c_i64, _c_i64, _vp]),
    "mx_a4w4_gemm_plan": (_c_int, [_c_i64, _c_i64, _c_i64, _c_sz, ctypes.c_char_p, _c_sz]),
    "mx_a16w4_gemm_plan": (_c_int, [_c_i64, _c_i64, _c_i64, ctypes.c_char_p, _c_sz]),
    "mx_a4w4_gemm_grouped_plan": (_c_int, [_c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_char_p,
                                           _c_sz]),
    "mx_a4w4_gemm_grouped_act_quant": (_c_int, [_vp, _vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _c_i64, _c_i64,
                                                ctypes.c_int32, _c_i64, _vp, _vp, _vp]),
    "mx_a4w4_gemm_grouped_act_quant_plan": (_c_int, [_c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_int32, _c_i64, ctypes.c_char_p,
                                                     _c_sz]),
    "mx_a4w4_gemm_grouped_mx": (_c_int, [_vp, _vp, _vp, _c_i64, _c_i64, _vp, _vp, _c_i64, _c_i64, _c_i64, _vp]),
    "mx_a4w4_gemm_grouped_mx_plan": (_c_int, [_c_i64, _c_i64, _c_i64, ctypes.c_char_p, _c_sz]),
    "mx_moe_combine": (_c_int, [_vp, _c_i64, _vp, _vp, _c_i64, _c_i64, _c_i64, _vp, _vp]),
    "mx_a16w4_gemm": (_c_int, [_vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _vp]),
    "mx_a4w4_gemm_noalloc": (_c_int, [_vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _vp]),
    "mx_noalloc_scratch_bytes": (_c_sz, []),
    "mx_calib_read": (_c_int, [_vp, _c_sz, _c_i64, _vp, _vp]),
    "mx_calib_mfma": (_c_int, [_c_i64, _c_i64, _vp, _vp]),
    "mx_calib_mfma_flops": (ctypes.c_double, [_c_i64, _c_i64]),
    "mx_calib_mfma_operands": (_c_int, [_vp, _c_sz, _c_i64, _c_i64, _vp, _vp]),
    "mx_calib_mfma_operands_flops": (ctypes.c_double, [_c_i64, _c_i64]),
    "mx_calib_mfma_operands_clock": (_c_int, [_vp, _c_sz, _c_i64, _c_i64, _vp, _vp, _vp]),
}

MX_OK, MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_ALIGN, MX_ERR_DEVICE, MX_ERR_WORKSPACE, MX_ERR_HIP = range(7)
MX_ACT_SILU, MX_ACT_SWIGLU = 0, 1

_lib = None


class MxError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with "
                              "`python -m mxfp4_quantized_gemm_inline_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().mx_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != MX_OK:
        raise MxError(status, what)


# ----------------------------------------------------------------------------- torch marshalling

def _torch():
    import torch
    return torch


def _stream_ptr(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _need(t, name, dtype=None, shape=None, min_bytes=None, min_numel=None):
    """Validate a tensor argument from its metadata alone (type, dtype, shape, size), before
    any device pointer is taken: a short or mis-shaped buffer would otherwise be read or
    written out of bounds by the kernels, which receive only pointers and sizes."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(int(d) for d in shape):
        raise ValueError(f"{name} must have shape {tuple(int(d) for d in shape)}, got {tuple(t.shape)}")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs at least {min_bytes}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {min_numel}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dev(t, dtype, name):
    """Device pointer of a validated tensor (raises if it is not on the current device)."""
    torch = _torch()
    _need(t, name, dtype)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.device.index is not None and t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, not on the current device cuda:{torch.cuda.current_device()}")
    return t.data_ptr()


def _dims2(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    return int(t.shape[0]), int(t.shape[1])


def mx_prepared_layout_version() -> int:
    return int(lib().mx_prepared_layout_version())


def mx_prepared_weight_bytes(N: int, K: int) -> int:
    return int(lib().mx_prepared_weight_bytes(int(N), int(K)))


def mx_a4w4_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().mx_a4w4_gemm_workspace_bytes(int(M), int(N), int(K)))


def mx_prepare_weight(w_bf16, out=None, stream=None):
    """W [N, K] bf16 -> opaque prepared MXFP4 blob (uint8, mx_prepared_weight_bytes(N, K))."""
    torch = _torch()
    _need(w_bf16, "w_bf16", torch.bfloat16)
    N, K = _dims2(w_bf16, "w_bf16")
    nbytes = mx_prepared_weight_bytes(N, K)
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=w_bf16.device)
    _need(out, "out", torch.uint8, min_bytes=nbytes)
    _check(lib().mx_prepare_weight(_dev(w_bf16, torch.bfloat16, "w_bf16"), N, K,
                                   _dev(out, torch.uint8, "w_prep"), _stream_ptr(stream)),
           "mx_prepare_weight")
    return out


def mx_prepare_weight_packed(w_fp4, w_scale, out=None, stream=None):
    """Caller-quantized weight -> prepared blob: w_fp4 uint8 [N, K/2] (low nibble = even k),
    w_scale uint8 [N, K/32] (E8M0)."""
    torch = _torch()
    _need(w_fp4, "w_fp4", torch.uint8)
    N, K2 = _dims2(w_fp4, "w_fp4")
    K = 2 * K2
    _need(w_scale, "w_scale", torch.uint8, shape=(N, K // 32))
    nbytes = mx_prepared_weight_bytes(N, K)
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=w_fp4.device)
    _need(out, "out", torch.uint8, min_bytes=nbytes)
    _check(lib().mx_prepare_weight_packed(_dev(w_fp4, torch.uint8, "w_fp4"), _dev(w_scale, torch.uint8, "w_scale"),
                                          N, K, _dev(out, torch.uint8, "w_prep"), _stream_ptr(stream)),
           "mx_prepare_weight_packed")
    return out


def mx_unprepare_weight(w_prep, N: int, K: int, stream=None):
    """Prepared blob -> canonical (payload uint8 [N, K/2], scales uint8 [N, K/32])."""
    torch = _torch()
    _need(w_prep, "w_prep", torch.uint8, min_bytes=mx_prepared_weight_bytes(N, K))
    q = torch.empty((N, K // 2), dtype=torch.uint8, device=w_prep.device)
    s = torch.empty((N, K // 32), dtype=torch.uint8, device=w_prep.device)
    _check(lib().mx_unprepare_weight(_dev(w_prep, torch.uint8, "w_prep"), N, K,
                                     _dev(q, None, "w_fp4"), _dev(s, None, "w_scale"),
                                     _stream_ptr(stream)), "mx_unprepare_weight")
    return q, s


def mx_quant_act(a_bf16, q_out=None, s_out=None, stream=None):
    """A [M, K] bf16 -> (payload uint8 [M, K/2], scales uint8 [M, K/32]), canonical layout."""
    torch = _torch()
    _need(a_bf16, "a_bf16", torch.bfloat16)
    M, K = _dims2(a_bf16, "a_bf16")
    q = q_out if q_out is not None else torch.empty((M, K // 2), dtype=torch.uint8, device=a_bf16.device)
    s = s_out if s_out is not None else torch.empty((M, K // 32), dtype=torch.uint8, device=a_bf16.device)
    _need(q, "a_fp4", torch.uint8, min_bytes=M * (K // 2))
    _need(s, "a_scale", torch.uint8, min_bytes=M * (K // 32))
    if M == 0:
        return q, s
    _check(lib().mx_quant_act(_dev(a_bf16, torch.bfloat16, "a_bf16"), M, K, _dev(q, torch.uint8, "a_fp4"),
                              _dev(s, torch.uint8, "a_scale"), _stream_ptr(stream)), "mx_quant_act")
    return q, s


def mx_a4w4_gemm(a_bf16, w_prep, N: int, out=None, workspace=None, stream=None):
    """C [M, N] bf16 = Q(A) Q(W)^T with A [M, K] bf16 and a prepared weight of shape [N, K].

    workspace: a device tensor for split-K partials, None to allocate
    mx_a4w4_gemm_workspace_bytes(M, N, K) bytes through torch, or False to pass none
    (the library then picks a configuration that needs no workspace).
    """
    torch = _torch()
    _need(a_bf16, "a_bf16", torch.bfloat16)
    M, K = _dims2(a_bf16, "a_bf16")
    _need(w_prep, "w_prep", torch.uint8, min_bytes=max(1, mx_prepared_weight_bytes(N, K)))
    c = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=a_bf16.device)
    _need(c, "out", torch.bfloat16, shape=(M, N))
    if M == 0:
        return c
    if workspace is None:
        nbytes = mx_a4w4_gemm_workspace_bytes(M, N, K)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=a_bf16.device) if nbytes else False
    ws_ptr, ws_bytes = (None, 0)
    if workspace is not False:
        ws_ptr, ws_bytes = _dev(workspace, None, "workspace"), workspace.numel() * workspace.element_size()
    _check(lib().mx_a4w4_gemm(_dev(a_bf16, torch.bfloat16, "a_bf16"), _dev(w_prep, torch.uint8, "w_prep"),
                              _dev(c, torch.bfloat16, "c_bf16"), M, int(N), K, ws_ptr, ws_bytes,
                              _stream_ptr(stream)), "mx_a4w4_gemm")
    return c


def mx_noalloc_scratch_bytes() -> int:
    """Size of the device scratch array mx_a4w4_gemm_noalloc uses in place of a workspace."""
    return int(lib().mx_noalloc_scratch_bytes())


def mx_a4w4_gemm_noalloc(a_bf16, w_prep, N: int, out, stream=None):
    """mx_a4w4_gemm without a caller workspace and without any allocation: the library's own
    device scratch array serves as the workspace (calls that overlap on one device share it).
    `out` [M, N] bf16 is required (allocating it here would defeat the purpose)."""
    torch = _torch()
    _need(a_bf16, "a_bf16", torch.bfloat16)
    M, K = _dims2(a_bf16, "a_bf16")
    _need(w_prep, "w_prep", torch.uint8, min_bytes=max(1, mx_prepared_weight_bytes(N, K)))
    _need(out, "out", torch.bfloat16, shape=(M, N))
    if M == 0:
        return out
    _check(lib().mx_a4w4_gemm_noalloc(_dev(a_bf16, torch.bfloat16, "a_bf16"), _dev(w_prep, torch.uint8, "w_prep"),
                                      _dev(out, torch.bfloat16, "c_bf16"), M, int(N), K, _stream_ptr(stream)),
           "mx_a4w4_gemm_noalloc")
    return out


def _grouped_tables(row_token, expert_offsets, w_prep_stacked, E, R_max, N, K):
    """The segment table, the row-to-token map and the stacked weights of a grouped call:
    expert_offsets [E+1] int32, row_token at least R_max int32 (when rows exist), E prepared
    weights of shape [N, K]."""
    torch = _torch()
    _need(expert_offsets, "expert_offsets", torch.int32, min_numel=int(E) + 1)
    if row_token is not None and R_max > 0:
        _need(row_token, "row_token", torch.int32, min_numel=int(R_max))
    _need(w_prep_stacked, "w_prep_stacked", torch.uint8,
          min_bytes=max(1, int(E) * mx_prepared_weight_bytes(N, K)))


def mx_a4w4_gemm_grouped(a_bf16, row_token, expert_offsets, E: int, R_max: int, w_prep_stacked,
                         N: int, rows_hint: int = 1, out=None, stream=None):
    """Grouped GEMM1: C [R_max, N] bf16, rows in expert-sorted order (rows >= R untouched)."""
    torch = _torch()
    _need(a_bf16, "a_bf16", torch.bfloat16)
    T, K = _dims2(a_bf16, "a_bf16")
    _grouped_tables(row_token, expert_offsets, w_prep_stacked, E, R_max, N, K)
    c = out if out is not None else torch.empty((R_max, N), dtype=torch.bfloat16, device=a_bf16.device)
    _need(c, "out", torch.bfloat16, shape=(R_max, N))
    _check(lib().mx_a4w4_gemm_grouped(
        _dev(a_bf16, torch.bfloat16, "a_bf16") if T > 0 else None,
        _dev(row_token, torch.int32, "row_token") if R_max > 0 else None,
        _dev(expert_offsets, torch.int32, "expert_offsets"), int(E), int(R_max),
        _dev(w_prep_stacked, torch.uint8, "w_prep_stacked"), _dev(c, torch.bfloat16, "c_bf16") if R_max > 0 else None,
        T, int(N), K, int(rows_hint), _stream_ptr(stream)), "mx_a4w4_gemm_grouped")
    return c


def mx_a4w4_gemm_grouped_act_quant(a_bf16, row_token, expert_offsets, E: int, R_max: int, w_prep_stacked,
                                   N: int, act: int = MX_ACT_SWIGLU, rows_hint: int = 1, h_fp4=None, h_scale=None,
                                   stream=None):
    """Grouped GEMM1 with fused SiLU / SwiGLU + MXFP4 quantization: returns (h_fp4 uint8
    [R_max, Nh/2], h_scale uint8 [R_max, Nh/32]) with Nh = N/2 (SwiGLU) or N (SiLU)."""
    torch = _torch()
    _need(a_bf16, "a_bf16", torch.bfloat16)
    T, K = _dims2(a_bf16, "a_bf16")
    _grouped_tables(row_token, expert_offsets, w_prep_stacked, E, R_max, N, K)
    Nh = N // 2 if act == MX_ACT_SWIGLU else N
    if h_fp4 is None:
        h_fp4 = torch.empty((R_max, Nh // 2), dtype=torch.uint8, device=a_bf16.device)
    if h_scale is None:
        h_scale = torch.empty((R_max, Nh // 32), dtype=torch.uint8, device=a_bf16.device)
    _need(h_fp4, "h_fp4", torch.uint8, min_bytes=R_max * (Nh // 2))
    _need(h_scale, "h_scale", torch.uint8, min_bytes=R_max * (Nh // 32))
    _check(lib().mx_a4w4_gemm_grouped_act_quant(
        _dev(a_bf16, torch.bfloat16, "a_bf16") if T > 0 else None,
        _dev(row_token, torch.int32, "row_token") if R_max > 0 else None,
        _dev(expert_offsets, torch.int32, "expert_offsets"), int(E), int(R_max),
        _dev(w_prep_stacked, torch.uint8, "w_prep_stacked"), T, int(N), K, int(act), int(rows_hint),
        _dev(h_fp4, torch.uint8, "h_fp4") if R_max > 0 else None,
        _dev(h_scale, torch.uint8, "h_scale") if R_max > 0 else None, _stream_ptr(stream)),
        "mx_a4w4_gemm_grouped_act_quant")
    return h_fp4, h_scale


def mx_a4w4_gemm_grouped_act_quant_plan(E: int, R_max: int, N: int, K: int, act: int = MX_ACT_SWIGLU,
                                        rows_hint: int = 1) -> str:
    """Kernel mx_a4w4_gemm_grouped_act_quant launches for this table size, shape and hint."""
    buf = ctypes.create_string_buffer(256)
    _check(lib().mx_a4w4_gemm_grouped_act_quant_plan(int(E), int(R_max), int(N), int(K), int(act), int(rows_hint),
                                                     buf, len(buf)),
           "mx_a4w4_gemm_grouped_act_quant_plan")
    return buf.value.decode()


def mx_a4w4_gemm_grouped_mx(a_fp4, a_scale, expert_offsets, E: int, R_max: int, w_prep_stacked, N: int,
                            rows_hint: int = 1, out=None, stream=None):
    """Second MoE GEMM on MXFP4 rows: a_fp4 uint8 [R_max, K/2], a_scale uint8 [R_max, K/32]
    -> C [R_max, N] bf16 (rows >= R untouched)."""
    torch = _torch()
    _need(a_fp4, "a_fp4", torch.uint8)
    rows, K2 = _dims2(a_fp4, "a_fp4")
    K = 2 * K2
    _need(a_scale, "a_scale", torch.uint8, shape=(rows, K // 32))
    if rows < R_max:
        raise ValueError(f"a_fp4 / a_scale hold {rows} rows, need at least R_max = {R_max}")
    _grouped_tables(None, expert_offsets, w_prep_stacked, E, R_max, N, K)
    c = out if out is not None else torch.empty((R_max, N), dtype=torch.bfloat16, device=a_fp4.device)
    _need(c, "out", torch.bfloat16, shape=(R_max, N))
    _check(lib().mx_a4w4_gemm_grouped_mx(
        _dev(a_fp4, torch.uint8, "a_fp4") if R_max > 0 else None,
        _dev(a_scale, torch.uint8, "a_scale") if R_max > 0 else None,
        _dev(expert_offsets, torch.int32, "expert_offsets"), int(E), int(R_max),
        _dev(w_prep_stacked, torch.uint8, "w_prep_stacked"), _dev(c, torch.bfloat16, "c_bf16") if R_max > 0 else None,
        int(N), K, int(rows_hint), _stream_ptr(stream)), "mx_a4w4_gemm_grouped_mx")
    return c


def mx_a4w4_gemm_grouped_mx_plan(N: int, K: int, rows_hint: int = 1) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().mx_a4w4_gemm_grouped_mx_plan(int(N), int(K), int(rows_hint), buf, len(buf)),
           "mx_a4w4_gemm_grouped_mx_plan")
    return buf.value.decode()


def mx_moe_combine(y_bf16, token_rows, token_weights, out=None, stream=None):
    """out [T, N] bf16 = sum_k token_weights[t, k] * y[token_rows[t, k]] (FP32, k order)."""
    torch = _torch()
    _need(y_bf16, "y_bf16", torch.bfloat16)
    R, N = _dims2(y_bf16, "y_bf16")
    _need(token_rows, "token_rows", torch.int32)
    T, topk = _dims2(token_rows, "token_rows")
    _need(token_weights, "token_weights", torch.float32, shape=(T, topk))
    o = out if out is not None else torch.empty((T, N), dtype=torch.bfloat16, device=token_rows.device)
    _need(o, "out", torch.bfloat16, shape=(T, N))
    _check(lib().mx_moe_combine(
        _dev(y_bf16, torch.bfloat16, "y_bf16") if R > 0 else None, R,
        _dev(token_rows, torch.int32, "token_rows") if T > 0 else None,
        _dev(token_weights, torch.float32, "token_weights") if T > 0 else None, T, topk, N,
        _dev(o, torch.bfloat16, "out_bf16") if T > 0 else None, _stream_ptr(stream)), "mx_moe_combine")
    return o


def mx_a16w4_gemm(a_bf16, w_prep, N: int, out=None, stream=None):
    """A16WFP4: A [M, K] bf16 (not quantized) x decoded prepared weight -> C [M, N] bf16."""
    torch = _torch()
    _need(a_bf16, "a_bf16", torch.bfloat16)
    M, K = _dims2(a_bf16, "a_bf16")
    _need(w_prep, "w_prep", torch.uint8, min_bytes=max(1, mx_prepared_weight_bytes(N, K)))
    c = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=a_bf16.device)
    _need(c, "out", torch.bfloat16, shape=(M, N))
    if M == 0:
        return c
    _check(lib().mx_a16w4_gemm(_dev(a_bf16, torch.bfloat16, "a_bf16"), _dev(w_prep, torch.uint8, "w_prep"),
                               _dev(c, torch.bfloat16, "c_bf16"), M, int(N), K, _stream_ptr(stream)),
           "mx_a16w4_gemm")
    return c


def mx_a4w4_gemm_plan(M: int, N: int, K: int, workspace_bytes=None) -> str:
    """Kernel(s) mx_a4w4_gemm launches for this shape; workspace_bytes defaults to what
    mx_a4w4_gemm allocates when given no workspace."""
    if workspace_bytes is None:
        workspace_bytes = mx_a4w4_gemm_workspace_bytes(M, N, K)
    buf = ctypes.create_string_buffer(256)
    _check(lib().mx_a4w4_gemm_plan(int(M), int(N), int(K), int(workspace_bytes), buf, len(buf)),
           "mx_a4w4_gemm_plan")
    return buf.value.decode()


def mx_a16w4_gemm_plan(M: int, N: int, K: int) -> str:
    """Kernel mx_a16w4_gemm launches for this shape."""
    buf = ctypes.create_string_buffer(256)
    _check(lib().mx_a16w4_gemm_plan(int(M), int(N), int(K), buf, len(buf)), "mx_a16w4_gemm_plan")
    return buf.value.decode()


def mx_a4w4_gemm_grouped_plan(E: int, R_max: int, T: int, N: int, K: int, rows_hint: int = 1) -> str:
    """Kernel mx_a4w4_gemm_grouped launches for this table size, token count and hint."""
    buf = ctypes.create_string_buffer(256)
    _check(lib().mx_a4w4_gemm_grouped_plan(int(E), int(R_max), int(T), int(N), int(K), int(rows_hint), buf,
                                           len(buf)), "mx_a4w4_gemm_grouped_plan")
    return buf.value.decode()


def mx_calib_read(buf, ctas: int, sink, stream=None) -> None:
    """One streaming-read launch over the whole of `buf` (a contiguous device tensor whose
    byte size is a multiple of 16); `sink` is a device tensor of at least 4 bytes."""
    _dev(buf, None, "buf")
    _dev(sink, None, "sink")
    nbytes = buf.numel() * buf.element_size()
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must hold at least 4 bytes")
    _check(lib().mx_calib_read(buf.data_ptr(), nbytes, int(ctas), sink.data_ptr(), _stream_ptr(stream)),
           "mx_calib_read")


def mx_calib_mfma(ctas: int, iters: int, sink, stream=None) -> None:
    """One MFMA-only launch (ctas x 4 waves x iters x 8 FP4 MFMAs)."""
    _dev(sink, None, "sink")
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must hold at least 4 bytes")
    _check(lib().mx_calib_mfma(int(ctas), int(iters), sink.data_ptr(), _stream_ptr(stream)), "mx_calib_mfma")


def mx_calib_mfma_flops(ctas: int, iters: int) -> float:
    return float(lib().mx_calib_mfma_flops(int(ctas), int(iters)))


def mx_calib_mfma_operands(ops, ctas: int, iters: int, sink, stream=None) -> None:
    """The MFMA loop on the operand bytes of `ops` (a contiguous device tensor of at least
    16 KiB, e.g. a prepared weight); `sink` is a device tensor of at least 4 bytes."""
    _dev(ops, None, "ops")
    _dev(sink, None, "sink")
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must hold at least 4 bytes")
    _check(lib().mx_calib_mfma_operands(ops.data_ptr(), ops.numel() * ops.element_size(), int(ctas), int(iters),
                                        sink.data_ptr(), _stream_ptr(stream)), "mx_calib_mfma_operands")


def mx_calib_mfma_operands_flops(ctas: int, iters: int) -> float:
    return float(lib().mx_calib_mfma_operands_flops(int(ctas), int(iters)))


def mx_calib_mfma_operands_clock(ops, ctas: int, iters: int, sink, clocks, stream=None) -> None:
    """mx_calib_mfma_operands that writes each wave's core-clock and 100 MHz counter ticks over
    its MFMA loop to `clocks` (an int64 device tensor of at least 8 * ctas elements)."""
    _dev(ops, None, "ops")
    _dev(sink, None, "sink")
    _dev(clocks, None, "clocks")
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must hold at least 4 bytes")
    if clocks.numel() * clocks.element_size() < 64 * int(ctas):
        raise ValueError("clocks must hold 8 * ctas uint64 values")
    _check(lib().mx_calib_mfma_operands_clock(ops.data_ptr(), ops.numel() * ops.element_size(), int(ctas),
                                              int(iters), sink.data_ptr(), clocks.data_ptr(), _stream_ptr(stream)),
           "mx_calib_mfma_operands_clock")


__all__ = [
    "LIB_PATH", "MxError", "lib", "status_string", "mx_prepared_layout_version",
    "mx_prepared_weight_bytes", "mx_a4w4_gemm_workspace_bytes", "mx_prepare_weight",
    "mx_prepare_weight_packed", "mx_unprepare_weight", "mx_quant_act", "mx_a4w4_gemm", "mx_a4w4_gemm_grouped",
    "mx_a4w4_gemm_plan", "mx_a16w4_gemm_plan", "mx_a4w4_gemm_grouped_plan", "mx_a4w4_gemm_grouped_act_quant",
    "mx_a4w4_gemm_grouped_act_quant_plan", "mx_a4w4_gemm_grouped_mx", "mx_a4w4_gemm_grouped_mx_plan",
    "mx_moe_combine", "mx_a16w4_gemm", "MX_ACT_SILU", "MX_ACT_SWIGLU", "mx_calib_read", "mx_calib_mfma",
    "mx_calib_mfma_flops", "mx_calib_mfma_operands", "mx_calib_mfma_operands_flops",
    "mx_calib_mfma_operands_clock",
]
