/*
 * mx_calib.h - roofline calibration kernels (measurement support, not part of the GEMM path).
 *
 * The GEMM is priced against two ceilings: HBM read bandwidth for small M and dense
 * block-scaled FP4 MFMA throughput for large M ("[gfx950][FlyDSL] Add direct dense A4W4
 * MXFP4 GEMM", Kernel microbenchmark, reports both regimes). The published MI355X figures
 * (8 TB/s, 10.1 PFLOP/s dense MXFP4) are what a run is graded against; these two kernels
 * measure what the device at hand actually sustains, so a result can also be read against
 * a measured ceiling. Conventions are those of mx.h: device pointers, caller-owned memory,
 * argument errors returned before any HIP call, work enqueued on `stream` with no host sync.
 */
#ifndef MX_CALIB_H_
#define MX_CALIB_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "mx.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * One launch that reads `bytes` bytes of `buf` once, front to back, with coalesced 16-byte
 * loads (each wave load covers 1 KiB of contiguous memory, eight loads in flight per
 * thread), spread over `ctas` workgroups of 256 threads. The data is folded into a value
 * that is stored to the 4-byte device word `sink` only when it equals a fixed improbable
 * constant (the store keeps the loads from being optimized away; `sink` is normally left
 * untouched). bytes must be a positive multiple of 16; buf 16-byte aligned; ctas in
 * [1, 2^20]. Errors: MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_ALIGN, MX_ERR_DEVICE (not gfx950), MX_ERR_HIP.
 */
mx_status mx_calib_read(const void* buf, size_t bytes, int64_t ctas, void* sink, hipStream_t stream);

/*
 * One launch of `ctas` workgroups of 256 threads (four waves), each wave issuing `iters`
 * rounds of eight independent 16x16x128 block-scaled FP4 MFMAs on register operands (no
 * memory traffic but one conditional 4-byte store to `sink`, as above). ctas in [1, 2^20],
 * iters in [1, 2^24]. Errors: MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_ALIGN, MX_ERR_DEVICE (not gfx950), MX_ERR_HIP.
 */
mx_status mx_calib_mfma(int64_t ctas, int64_t iters, void* sink, hipStream_t stream);

/* Floating-point operations of one mx_calib_mfma launch (2 * 16 * 16 * 128 per MFMA). */
double mx_calib_mfma_flops(int64_t ctas, int64_t iters);

/*
 * The MFMA ceiling on given operand data. The rate of the block-scaled FP4 MFMA depends on
 * the operand bits (the device lowers its clock under the multipliers' power draw), so a
 * GEMM is best compared with the rate on its own operands. One launch of `ctas` workgroups
 * of 256 threads (four waves, one per SIMD); each wave reads one 16 KiB window of `ops`
 * (wave w takes window w modulo floor(bytes / 16384)): sixteen 1 KiB operand blocks in the
 * prepared layout (lane l's 16 bytes at 16 l of each block), then issues `iters` rounds of
 * the 64 block products of an 8 x 8 block tile with unit scales, accumulating in place. No
 * memory traffic after the first reads but one conditional 4-byte store to `sink`, as
 * above. bytes >= 16384; ops 16-byte aligned; ctas in [1, 2^20], iters in [1, 2^24].
 * Errors: MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_ALIGN, MX_ERR_DEVICE (not gfx950), MX_ERR_HIP.
 */
mx_status mx_calib_mfma_operands(const void* ops, size_t bytes, int64_t ctas, int64_t iters, void* sink,
                                 hipStream_t stream);

/* Floating-point operations of one mx_calib_mfma_operands launch (64 MFMAs per wave and round). */
double mx_calib_mfma_operands_flops(int64_t ctas, int64_t iters);

/*
 * mx_calib_mfma_operands that also reports the shader clock it ran at: lane 0 of wave w
 * (w = 4 * CTA + wave in CTA) writes two uint64 values to `clocks` (device memory of
 * 8 * ctas uint64, 8-byte aligned): clocks[2 w] = ticks of the core-clock counter
 * (s_memtime) over its MFMA loop, clocks[2 w + 1] = ticks of the constant 100 MHz counter
 * (s_memrealtime) over the same loop. Their ratio times 100 MHz is the wave's mean clock;
 * the MFMA count over core-clock ticks gives the cycles each MFMA held the pipe. Arguments
 * and errors otherwise as mx_calib_mfma_operands.
 */
mx_status mx_calib_mfma_operands_clock(const void* ops, size_t bytes, int64_t ctas, int64_t iters, void* sink,
                                       void* clocks, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MX_CALIB_H_ */
