// mx_noalloc.hip - the dense A4W4 GEMM for callers that cannot allocate device memory (code
// under stream capture, tight serving loops, harnesses that forbid allocation).
//
// mx_a4w4_gemm takes an optional caller workspace: FP32 partial sums of K slices, or the
// quantized activations of the quantize-once plan. Here that workspace is the library's own
// file-scope device array `scratch` of kScratchBytes, one copy per GPU, alive until the
// process ends. Its device address is obtained once per device (first call with that device
// current) through hipGetSymbolAddress and kept per device: in host code the array's name is
// a host-side stand-in, not a device address, so only the resolved pointer is ever handed to
// a kernel.
//
// Every plan writes the part of the workspace it reads before reading it (each K slice writes
// its whole partial tile; k_prepare writes every padded activation row), so nothing has to be
// cleared between calls. Calls that overlap on one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mx.h"
#include "mx_internal.h"

namespace {
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_mu;
void* g_scratch[kMaxDevices];  // resolved device address per device (null until resolved)

// The scratch address on the current device, resolved on first use; nullptr on failure.
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" size_t mx_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" mx_status mx_a4w4_gemm_noalloc(const void* a_bf16, const void* w_prep, void* c_bf16, int64_t M,
                                          int64_t N, int64_t K, hipStream_t stream) {
  if (M < 0 || M > (int64_t(1) << 30) || mx_prepared_weight_bytes(N, K) == 0) return MX_ERR_SHAPE;
  if (M == 0) return MX_OK;
  // the plan mx_a4w4_gemm runs when handed the workspace it asks for
  const size_t need = mx_a4w4_gemm_workspace_bytes(M, N, K);
  if (need > kScratchBytes) return MX_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need) {
    const mx_status d = mx::check_device();
    if (d != MX_OK) return d;
    ws = scratch_ptr();
    if (!ws) return MX_ERR_HIP;
  }
  return mx_a4w4_gemm(a_bf16, w_prep, c_bf16, M, N, K, ws, need, stream);
}
