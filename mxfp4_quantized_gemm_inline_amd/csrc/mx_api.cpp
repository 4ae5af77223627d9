// mx_api.cpp - the C ABI declared in include/mx.h: argument validation (pure host code,
// run before any HIP call), the gfx950 device check, and dispatch to the launchers.
#include "mx.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdio>
#include <cstring>

#include "mx_internal.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other
std::atomic<int> g_arch_ok[kMaxDevices];

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Rows of one GEMM call: at most 2^30, so row and tile counts (M + 255, M padded to 64) stay
// within 32-bit integers in the kernels and launchers.
constexpr int64_t kMaxRows = 1ll << 30;

// K <= 2^24 keeps a tile row's byte offset (at most 127 rows of 2K bytes) in 32 bits.
bool gemm_shape_ok(int64_t N, int64_t K) {
  return N > 0 && K > 0 && N % 256 == 0 && K % 128 == 0 && N <= (1ll << 30) && K <= (1ll << 24);
}

}  // namespace

namespace mx {
// The gfx950 check every entry point makes (also used by the measurement entry points).
mx_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MX_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MX_ERR_DEVICE;
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MX_ERR_HIP;
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? MX_OK : MX_ERR_DEVICE;
}
}  // namespace mx

namespace {
using mx::check_device;

mx_status from_hip(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_HIP; }

}  // namespace

extern "C" {

const char* mx_status_string(mx_status s) {
  switch (s) {
    case MX_OK: return "MX_OK";
    case MX_ERR_NULL: return "MX_ERR_NULL: a required pointer is NULL";
    case MX_ERR_SHAPE: return "MX_ERR_SHAPE: invalid shape (need M >= 0, N % 256 == 0, K % 128 == 0)";
    case MX_ERR_ALIGN: return "MX_ERR_ALIGN: a pointer is not 16-byte aligned";
    case MX_ERR_DEVICE: return "MX_ERR_DEVICE: the current device is not gfx950";
    case MX_ERR_WORKSPACE: return "MX_ERR_WORKSPACE: workspace missing or too small";
    case MX_ERR_HIP: return "MX_ERR_HIP: a HIP runtime call or kernel launch failed";
  }
  return "MX_ERR_UNKNOWN";
}

int mx_prepared_layout_version(void) { return 2; }

size_t mx_prepared_weight_bytes(int64_t N, int64_t K) {
  if (!gemm_shape_ok(N, K)) return 0;
  return (size_t)N * (size_t)K / 2 + (size_t)N * (size_t)K / 32;
}

mx_status mx_prepare_weight(const void* w_bf16, int64_t N, int64_t K, void* w_prep, hipStream_t stream) {
  if (!w_bf16 || !w_prep) return MX_ERR_NULL;
  if (!gemm_shape_ok(N, K)) return MX_ERR_SHAPE;
  if (!aligned16(w_bf16) || !aligned16(w_prep)) return MX_ERR_ALIGN;
  mx_status d = check_device();
  if (d != MX_OK) return d;
  return from_hip(mx::launch_prepare(w_bf16, N, K, w_prep, stream));
}

mx_status mx_prepare_weight_packed(const void* w_fp4, const void* w_scale, int64_t N, int64_t K, void* w_prep,
                                   hipStream_t stream) {
  if (!w_fp4 || !w_scale || !w_prep) return MX_ERR_NULL;
  if (!gemm_shape_ok(N, K)) return MX_ERR_SHAPE;
  if (!aligned16(w_fp4) || !aligned16(w_scale) || !aligned16(w_prep)) return MX_ERR_ALIGN;
  mx_status d = check_device();
  if (d != MX_OK) return d;
  return from_hip(mx::launch_prepare_packed(w_fp4, w_scale, N, K, w_prep, stream));
}

mx_status mx_unprepare_weight(const void* w_prep, int64_t N, int64_t K, void* w_fp4, void* w_scale,
                              hipStream_t stream) {
  if (!w_prep || !w_fp4 || !w_scale) return MX_ERR_NULL;
  if (!gemm_shape_ok(N, K)) return MX_ERR_SHAPE;
  if (!aligned16(w_prep) || !aligned16(w_fp4) || !aligned16(w_scale)) return MX_ERR_ALIGN;
  mx_status d = check_device();
  if (d != MX_OK) return d;
  return from_hip(mx::launch_unprepare(w_prep, N, K, w_fp4, w_scale, stream));
}

mx_status mx_quant_act(const void* a_bf16, int64_t M, int64_t K, void* a_fp4, void* a_scale,
                       hipStream_t stream) {
  if (M < 0 || K <= 0 || K % 32 != 0 || K > (1ll << 30) || M > (1ll << 40) / K) return MX_ERR_SHAPE;
  if (M == 0) return MX_OK;
  if (!a_bf16 || !a_fp4 || !a_scale) return MX_ERR_NULL;
  if (!aligned16(a_bf16) || !aligned16(a_fp4) || !aligned16(a_scale)) return MX_ERR_ALIGN;
  mx_status d = check_device();
  if (d != MX_OK) return d;
  return from_hip(mx::launch_quant_act(a_bf16, M, K, a_fp4, a_scale, stream));
}

size_t mx_a4w4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || !gemm_shape_ok(N, K) || M > kMaxRows) return 0;
  return mx::gemm_workspace_bytes(M, N, K);
}

mx_status mx_a4w4_gemm(const void* a_bf16, const void* w_prep, void* c_bf16, int64_t M, int64_t N,
                       int64_t K, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (M < 0 || !gemm_shape_ok(N, K) || M > kMaxRows) return MX_ERR_SHAPE;
  if (M == 0) return MX_OK;
  if (!a_bf16 || !w_prep || !c_bf16) return MX_ERR_NULL;
  if (!aligned16(a_bf16) || !aligned16(w_prep) || !aligned16(c_bf16)) return MX_ERR_ALIGN;
  if (workspace && !aligned16(workspace)) return MX_ERR_ALIGN;
  mx_status d = check_device();
  if (d != MX_OK) return d;
  return from_hip(mx::launch_gemm(a_bf16, w_prep, c_bf16, M, N, K, workspace, workspace_bytes, stream));
}

mx_status mx_a16w4_gemm(const void* a_bf16, const void* w_prep, void* c_bf16, int64_t M, int64_t N, int64_t K,
                        hipStream_t stream) {
  if (M < 0 || !gemm_shape_ok(N, K) || M > kMaxRows) return MX_ERR_SHAPE;
  if (M == 0) return MX_OK;
  if (!a_bf16 || !w_prep || !c_bf16) return MX_ERR_NULL;
  if (!aligned16(a_bf16) || !aligned16(w_prep) || !aligned16(c_bf16)) return MX_ERR_ALIGN;
  mx_status d = check_device();
  if (d != MX_OK) return d;
  return from_hip(mx::launch_a16w4(a_bf16, w_prep, c_bf16, M, N, K, stream));
}

mx_status mx_a4w4_gemm_grouped(const void* a_bf16, const int32_t* row_token, const int32_t* expert_offsets,
                               int64_t E, int64_t R_max, const void* w_prep_stacked, void* c_bf16,
                               int64_t T, int64_t N, int64_t K, int64_t rows_hint, hipStream_t stream) {
  if (E < 1 || T < 0 || R_max < 0 || !gemm_shape_ok(N, K) || E > (1 << 20) || R_max > kMaxRows ||
      T > kMaxRows)
    return MX_ERR_SHAPE;
  if (!expert_offsets || !w_prep_stacked) return MX_ERR_NULL;
  if (R_max > 0 && (!row_token || !c_bf16)) return MX_ERR_NULL;
  if (T > 0 && !a_bf16) return MX_ERR_NULL;
  if ((a_bf16 && !aligned16(a_bf16)) || !aligned16(w_prep_stacked) || (c_bf16 && !aligned16(c_bf16)) ||
      (reinterpret_cast<uintptr_t>(expert_offsets) & 3u) || (reinterpret_cast<uintptr_t>(row_token) & 3u))
    return MX_ERR_ALIGN;
  if (R_max == 0) return MX_OK;
  mx_status d = check_device();
  if (d != MX_OK) return d;
  return from_hip(mx::launch_gemm_grouped(a_bf16, row_token, expert_offsets, E, R_max, w_prep_stacked,
                                          c_bf16, T, N, K, rows_hint < 1 ? 1 : rows_hint, stream));
}

mx_status mx_a4w4_gemm_grouped_act_quant(const void* a_bf16, const int32_t* row_token,
                                         const int32_t* expert_offsets, int64_t E, int64_t R_max,
                                         const void* w_prep_stacked, int64_t T, int64_t N, int64_t K, int32_t act,
                                         int64_t rows_hint, void* h_fp4, void* h_scale, hipStream_t stream) {
  if (E < 1 || T < 0 || R_max < 0 || !gemm_shape_ok(N, K) || E > (1 << 20) || R_max > kMaxRows ||
      T > kMaxRows || (act != MX_ACT_SILU && act != MX_ACT_SWIGLU))
    return MX_ERR_SHAPE;
  if (!expert_offsets || !w_prep_stacked) return MX_ERR_NULL;
  if (R_max > 0 && (!row_token || !h_fp4 || !h_scale)) return MX_ERR_NULL;
  if (T > 0 && !a_bf16) return MX_ERR_NULL;
  if ((a_bf16 && !aligned16(a_bf16)) || !aligned16(w_prep_stacked) || (h_fp4 && !aligned16(h_fp4)) ||
      (h_scale && !aligned16(h_scale)) || (reinterpret_cast<uintptr_t>(expert_offsets) & 3u) ||
      (reinterpret_cast<uintptr_t>(row_token) & 3u))
    return MX_ERR_ALIGN;
  if (R_max == 0) return MX_OK;
  mx_status d = check_device();
  if (d != MX_OK) return d;
  return from_hip(mx::launch_gemm_grouped_act(a_bf16, row_token, expert_offsets, E, R_max, w_prep_stacked, h_fp4,
                                              h_scale, T, N, K, act, rows_hint < 1 ? 1 : rows_hint, stream));
}

mx_status mx_a4w4_gemm_grouped_mx(const void* a_fp4, const void* a_scale, const int32_t* expert_offsets, int64_t E,
                                  int64_t R_max, const void* w_prep_stacked, void* c_bf16, int64_t N, int64_t K,
                                  int64_t rows_hint, hipStream_t stream) {
  if (E < 1 || R_max < 0 || !gemm_shape_ok(N, K) || E > (1 << 20) || R_max > kMaxRows) return MX_ERR_SHAPE;
  if (!expert_offsets || !w_prep_stacked) return MX_ERR_NULL;
  if (R_max > 0 && (!a_fp4 || !a_scale || !c_bf16)) return MX_ERR_NULL;
  if ((a_fp4 && !aligned16(a_fp4)) || (a_scale && !aligned16(a_scale)) || !aligned16(w_prep_stacked) ||
      (c_bf16 && !aligned16(c_bf16)) || (reinterpret_cast<uintptr_t>(expert_offsets) & 3u))
    return MX_ERR_ALIGN;
  if (R_max == 0) return MX_OK;
  mx_status d = check_device();
  if (d != MX_OK) return d;
  return from_hip(mx::launch_gemm_grouped_mx(a_fp4, a_scale, expert_offsets, E, R_max, w_prep_stacked, c_bf16, N,
                                             K, rows_hint < 1 ? 1 : rows_hint, stream));
}

mx_status mx_a4w4_gemm_grouped_mx_plan(int64_t N, int64_t K, int64_t rows_hint, char* buf, size_t buf_len) {
  if (!gemm_shape_ok(N, K)) return MX_ERR_SHAPE;
  if (!buf || buf_len == 0) return MX_ERR_NULL;
  if (!mx::grouped_mx_plan(N, K, rows_hint < 1 ? 1 : rows_hint, buf, buf_len)) {
    buf[0] = '\0';
    return MX_ERR_HIP;
  }
  return MX_OK;
}

mx_status mx_moe_combine(const void* y_bf16, int64_t R, const int32_t* token_rows, const float* token_weights,
                         int64_t T, int64_t topk, int64_t N, void* out_bf16, hipStream_t stream) {
  if (R < 0 || T < 0 || topk < 1 || topk > 1024 || N <= 0 || N % 8 != 0 || R > kMaxRows ||
      T > kMaxRows || N > (1ll << 30) || T * (N / 8) > (1ll << 39))
    return MX_ERR_SHAPE;
  if (T == 0) return MX_OK;
  if (!token_rows || !token_weights || !out_bf16 || (R > 0 && !y_bf16)) return MX_ERR_NULL;
  if ((y_bf16 && !aligned16(y_bf16)) || !aligned16(out_bf16) ||
      (reinterpret_cast<uintptr_t>(token_rows) & 3u) || (reinterpret_cast<uintptr_t>(token_weights) & 3u))
    return MX_ERR_ALIGN;
  mx_status d = check_device();
  if (d != MX_OK) return d;
  return from_hip(mx::launch_moe_combine(y_bf16, R, token_rows, token_weights, T, topk, N, out_bf16, stream));
}

mx_status mx_a4w4_gemm_grouped_act_quant_plan(int64_t E, int64_t R_max, int64_t N, int64_t K, int32_t act,
                                              int64_t rows_hint, char* buf, size_t buf_len) {
  if (E < 1 || R_max < 0 || E > (1 << 20) || R_max > kMaxRows || !gemm_shape_ok(N, K) ||
      (act != MX_ACT_SILU && act != MX_ACT_SWIGLU))
    return MX_ERR_SHAPE;
  if (!buf || buf_len == 0) return MX_ERR_NULL;
  if (!mx::grouped_act_plan(E, R_max, N, act, rows_hint < 1 ? 1 : rows_hint, buf, buf_len)) {
    buf[0] = '\0';
    return MX_ERR_HIP;
  }
  return MX_OK;
}

mx_status mx_a16w4_gemm_plan(int64_t M, int64_t N, int64_t K, char* buf, size_t buf_len) {
  if (M < 0 || !gemm_shape_ok(N, K) || M > kMaxRows) return MX_ERR_SHAPE;
  if (!buf || buf_len == 0) return MX_ERR_NULL;
  if (!mx::a16w4_plan(M, N, K, buf, buf_len)) {  // the tuning override names nothing compiled
    buf[0] = '\0';
    return MX_ERR_HIP;
  }
  return MX_OK;
}

mx_status mx_a4w4_gemm_plan(int64_t M, int64_t N, int64_t K, size_t workspace_bytes, char* buf, size_t buf_len) {
  if (M < 0 || !gemm_shape_ok(N, K) || M > kMaxRows) return MX_ERR_SHAPE;
  if (!buf || buf_len == 0) return MX_ERR_NULL;
  if (M == 0) {
    std::snprintf(buf, buf_len, "none");
    return MX_OK;
  }
  if (!mx::gemm_plan(M, N, K, workspace_bytes, buf, buf_len)) {
    buf[0] = '\0';
    return MX_ERR_HIP;
  }
  return MX_OK;
}

mx_status mx_a4w4_gemm_grouped_plan(int64_t E, int64_t R_max, int64_t T, int64_t N, int64_t K,
                                    int64_t rows_hint, char* buf, size_t buf_len) {
  if (E < 1 || T < 0 || R_max < 0 || !gemm_shape_ok(N, K) || E > (1 << 20) || R_max > kMaxRows ||
      T > kMaxRows)
    return MX_ERR_SHAPE;
  if (!buf || buf_len == 0) return MX_ERR_NULL;
  if (R_max == 0) {
    std::snprintf(buf, buf_len, "none");
    return MX_OK;
  }
  if (!mx::grouped_plan(E, R_max, N, K, T, rows_hint < 1 ? 1 : rows_hint, buf, buf_len)) {
    buf[0] = '\0';
    return MX_ERR_HIP;
  }
  return MX_OK;
}

}  // extern "C"
