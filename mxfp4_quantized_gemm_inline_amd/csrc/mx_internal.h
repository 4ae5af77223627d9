// mx_internal.h - launchers shared between the C ABI (mx_api.cpp) and the kernels
// (mx_kernels.hip). Shapes are validated by the caller before any of these runs.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "mx.h"

namespace mx {

// MX_OK when the current device is gfx950, else MX_ERR_DEVICE (MX_ERR_HIP if it cannot be
// queried); cached per device.
mx_status check_device();

hipError_t launch_quant_act(const void* a, int64_t M, int64_t K, void* q, void* s, hipStream_t st);
hipError_t launch_prepare(const void* w, int64_t N, int64_t K, void* wp, hipStream_t st);
// The prepared layout for N rows (N % 64 == 0) of which the first `valid` are read from w; the
// rest encode as zero blocks.
hipError_t launch_prepare_rows(const void* w, int64_t valid, int64_t N, int64_t K, void* wp, hipStream_t st);
hipError_t launch_prepare_packed(const void* q, const void* s, int64_t N, int64_t K, void* wp, hipStream_t st);
hipError_t launch_unprepare(const void* wp, int64_t N, int64_t K, void* q, void* s, hipStream_t st);
hipError_t launch_gemm(const void* a, const void* wp, void* c, int64_t M, int64_t N, int64_t K,
                       void* workspace, size_t workspace_bytes, hipStream_t st);
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_grouped(const void* a, const int32_t* row_token, const int32_t* offsets,
                               int64_t E, int64_t R_max, const void* wp, void* c, int64_t T,
                               int64_t N, int64_t K, int64_t rows_hint, hipStream_t st);
// act: 0 = SiLU, 1 = SwiGLU (gate columns first). Outputs hq [R_max, Nh/2], hs [R_max, Nh/32].
hipError_t launch_gemm_grouped_act(const void* a, const int32_t* row_token, const int32_t* offsets, int64_t E,
                                   int64_t R_max, const void* wp, void* hq, void* hs, int64_t T, int64_t N,
                                   int64_t K, int act, int64_t rows_hint, hipStream_t st);
bool grouped_act_plan(int64_t E, int64_t R_max, int64_t N, int act, int64_t rows_hint, char* buf, size_t len);
// Second MoE GEMM on MXFP4 rows (aq [R_max, K/2], as [R_max, K/32]) and the top-k combine.
hipError_t launch_gemm_grouped_mx(const void* aq, const void* as, const int32_t* offsets, int64_t E, int64_t R_max,
                                  const void* wp, void* c, int64_t N, int64_t K, int64_t rows_hint, hipStream_t st);
bool grouped_mx_plan(int64_t N, int64_t K, int64_t rows_hint, char* buf, size_t len);
// A16WFP4: bf16 A [M, K] times the prepared weight decoded to bf16, bf16 C [M, N].
hipError_t launch_a16w4(const void* a, const void* wp, void* c, int64_t M, int64_t N, int64_t K, hipStream_t st);
bool a16w4_plan(int64_t M, int64_t N, int64_t K, char* buf, size_t len);
hipError_t launch_moe_combine(const void* y, int64_t R, const int32_t* rows, const float* w, int64_t T, int64_t topk,
                              int64_t N, void* out, hipStream_t st);
// Quantize-once GEMM (mx_gemm_qo.hip): the activations are laid out in the prepared layout in
// ws (qo_act_bytes(M, K) bytes) by k_prepare, then k_gemm_qo<WM, WN, MT, NG, NBUF, OCC>
// multiplies the two prepared operands.
size_t qo_act_bytes(int64_t M, int64_t K);
bool qo_supported(int WM, int WN, int MT, int NG, int NBUF, int OCC);
hipError_t launch_gemm_qo(int WM, int WN, int MT, int NG, int NBUF, int OCC, const void* a, const void* wp, void* c,
                          int64_t M, int64_t N, int64_t K, int GM, void* ws, hipStream_t st);
// The register-direct form: k_prepare as above, then k_gemm_qr<MT, NG, D> (one wave per
// 16 MT x 16 NG tile, operands D steps ahead in registers; N % (16 NG) == 0). With slices > 1
// the tiles beyond one round of the chip (qr_tail_tiles) run as `slices` K slices each into
// FP32 partials after the activations in ws, added in slice order by k_qr_tail_reduce.
bool qr_supported(int MT, int NG, int D);
int qr_tail_tiles(int64_t M, int64_t N, int MT, int NG);
size_t qr_workspace_bytes(int64_t M, int64_t N, int64_t K, int MT, int NG, int slices);
hipError_t launch_gemm_qr(int MT, int NG, int D, int slices, const void* a, const void* wp, void* c, int64_t M,
                          int64_t N, int64_t K, int GM, void* ws, hipStream_t st);
// Four register-direct waves per CTA on one tile, each over a quarter of the CTA's K range,
// added through LDS: k_prepare as above, then k_gemm_qk<MT, NG, D>; with slices > 1 the CTAs
// of a tile split K `slices` ways into FP32 partials after the activations in ws, added by
// k_splitk_reduce. Needs 4 * slices <= K / 128.
bool qk_supported(int MT, int NG, int D);
size_t qk_workspace_bytes(int64_t M, int64_t N, int64_t K, int slices);
hipError_t launch_gemm_qk(int MT, int NG, int D, int slices, const void* a, const void* wp, void* c, int64_t M,
                          int64_t N, int64_t K, int GM, void* ws, hipStream_t st);
// C [M, N] bf16 = the sum over s = 0..S-1, in order, of the FP32 partials P[s] [M, N].
hipError_t launch_splitk_reduce(const float* P, void* c, int64_t M, int64_t N, int S, hipStream_t st);
// Name the kernel(s) the launchers above would run (false: the tuning override is invalid).
bool gemm_plan(int64_t M, int64_t N, int64_t K, size_t ws_bytes, char* buf, size_t len);
bool grouped_plan(int64_t E, int64_t R_max, int64_t N, int64_t K, int64_t T, int64_t rows_hint, char* buf,
                  size_t len);

}  // namespace mx
