// mx_prepare_packed.hip - weight preparation from an already-quantized weight: the
// caller's packed E2M1 codes and E8M0 scales are preshuffled into the prepared layout
// ("[gfx950][FlyDSL] Add direct dense A4W4 MXFP4 GEMM", Scope: packed E2M1 weights and
// E8M0 scales, preshuffled once).
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

// The preshuffle alone, for a weight the caller has already quantized: canonical payload
// [N, K/2] (16 bytes per 32-block) and E8M0 scales [N, K/32] into the prepared layout. One
// thread per (column-group quad, K step, lane), as in k_prepare; the bytes are copied as
// they are.
__global__ __launch_bounds__(256) void k_prepare_packed(const uint8_t* __restrict__ q,
                                                         const uint8_t* __restrict__ s,
                                                         uint8_t* __restrict__ Wp, int N, int K) {
  const int T = steps_of(K), Q = N / 64, KB = K / kBlock;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)Q * T * 64) return;
  const int lane = (int)(idx % 64);
  const int64_t r = idx / 64;
  const int t = (int)(r % T), qd = (int)(r / T);
  const int kb = 4 * t + (lane >> 4);
  uint32_t sword = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int g = 4 * qd + j;
    const int n = 16 * g + (lane & 15);
    *reinterpret_cast<uint4*>(Wp + wp_payload_off(g, t, lane, T)) =
        *reinterpret_cast<const uint4*>(q + (size_t)n * (K / 2) + (size_t)kb * 16);
    sword |= (uint32_t)s[(size_t)n * KB + kb] << (8 * j);
  }
  *reinterpret_cast<uint32_t*>(Wp + payload_bytes(N, K) + wp_scale_off(qd, t, lane, T)) = sword;
}

hipError_t launch_prepare_packed(const void* q, const void* s, int64_t N, int64_t K, void* wp, hipStream_t st) {
  const int64_t n = (N / 64) * steps_of((int)K) * 64;
  hipLaunchKernelGGL(k_prepare_packed, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(s), static_cast<uint8_t*>(wp),
                     (int)N, (int)K);
  return hipGetLastError();
}

}  // namespace mx
