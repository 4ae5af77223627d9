/*
 * mx.h - C ABI of the inline-quantized A4W4 MXFP4 GEMM library for MI355X (gfx950).
 *
 * The operation ("[gfx950][FlyDSL] Add direct dense A4W4 MXFP4 GEMM", Summary and
 * Implementation): BF16 activations A[M,K] are quantized inside the GEMM to MXFP4
 * (E2M1 elements, one E8M0 scale per 32 consecutive K) and multiplied against a
 * weight W[N,K] that was quantized to MXFP4 and preshuffled once; the product is
 * accumulated in FP32 and written as BF16 C[M,N]. Scope (same page, Scope): gfx950
 * only, N divisible by 256, K divisible by 128 (this library also caps N at 2^30 and K
 * at 2^24); rows of C at or beyond M are never read or written (same page,
 * Implementation: M-tail masking).
 *
 * Quantization rule (all entry points): for each 32-element block along K, the scale
 * byte is s = max(E - 2, 0) where E is the exponent field of the block's largest
 * magnitude (equivalently e = floor(log2 amax) - 2 clamped to [-127, 127], s = e + 127;
 * an all-zero block gets 0); each element x becomes the E2M1 code nearest to
 * x * 2^-e, ties to the even code, magnitudes >= 6 saturating to 6, with the sign bit
 * of x kept (so -0.0 encodes as 0x8).
 *
 * Conventions shared by every entry point:
 *  - All buffer pointers are device pointers, caller-allocated and caller-owned, and
 *    16-byte aligned. The library allocates no device memory and keeps no per-call state.
 *  - Matrices are dense row-major. bf16 values are raw 16-bit patterns.
 *  - Argument errors are returned synchronously before any HIP call is made.
 *  - Work is enqueued on `stream` (NULL = the default stream); no entry point
 *    synchronizes the host. Faults inside a kernel surface at the caller's next sync.
 *  - Inputs must be finite; NaN/Inf inputs give unspecified (but in-bounds) results.
 *  - Output is bitwise reproducible for a given (M, N, K), device and library build.
 *  - Entry points are thread-safe.
 */
#ifndef MX_H_
#define MX_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mx_status {
  MX_OK = 0,
  MX_ERR_NULL = 1,      /* a required pointer is NULL */
  MX_ERR_SHAPE = 2,     /* a size is negative or breaks a divisibility rule */
  MX_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned */
  MX_ERR_DEVICE = 4,    /* the current device is not gfx950 */
  MX_ERR_WORKSPACE = 5, /* a required workspace is missing or too small */
  MX_ERR_HIP = 6        /* a HIP runtime call or kernel launch failed */
} mx_status;

/* Static, human-readable name of a status code. Never NULL. */
const char* mx_status_string(mx_status s);

/* Version of the prepared-weight layout; a blob is only valid for the version that wrote it. */
int mx_prepared_layout_version(void);

/*
 * Size in bytes of a prepared MXFP4 weight of shape [N, K]: N*K/2 bytes of packed E2M1
 * payload followed by N*K/32 bytes of E8M0 scales, N*K*17/32 in all, e.g. 32,169,984
 * bytes for 8448 x 7168 ("[gfx950][FlyDSL] Add direct dense A4W4 MXFP4 GEMM", Model
 * validation). Returns 0 when N <= 0, K <= 0, N % 256, K % 128, N > 2^30 or K > 2^24.
 */
size_t mx_prepared_weight_bytes(int64_t N, int64_t K);

/*
 * One-time weight preparation ("prepare_gemm_a4w4_weight" of the page above,
 * Implementation: one-time packed E2M1 weight and E8M0 scale preshuffle).
 * w_bf16: [N, K] bf16 row-major (read only).
 * w_prep: mx_prepared_weight_bytes(N, K) bytes, written completely (opaque layout).
 * Requires N % 256 == 0, K % 128 == 0. Errors: MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_ALIGN,
 * MX_ERR_DEVICE, MX_ERR_HIP.
 */
mx_status mx_prepare_weight(const void* w_bf16, int64_t N, int64_t K, void* w_prep,
                            hipStream_t stream);

/*
 * Weight preparation from an already-quantized weight: the caller's packed E2M1 codes and
 * E8M0 scales are preshuffled once, as they are ("[gfx950][FlyDSL] Add direct dense A4W4
 * MXFP4 GEMM", Scope: packed E2M1 weights and E8M0 scales, preshuffled once).
 * w_fp4: [N, K/2] bytes, row n holding W[n, 2i] in the low nibble and W[n, 2i+1] in the
 * high nibble of byte i. w_scale: [N, K/32] bytes, the E8M0 scale of each 32-block along
 * K (value 2^(byte - 127)). Both read only. w_prep: mx_prepared_weight_bytes(N, K) bytes,
 * written completely. Every byte is copied as given; a scale byte of 255 (NaN in the OCP
 * MX encoding) is outside the contract. For a weight quantized by the rule above, the
 * result is identical to mx_prepare_weight's, and mx_unprepare_weight returns the inputs
 * unchanged. Same shape rules and errors as mx_prepare_weight.
 */
mx_status mx_prepare_weight_packed(const void* w_fp4, const void* w_scale, int64_t N, int64_t K,
                                   void* w_prep, hipStream_t stream);

/*
 * Test support: the inverse of the preshuffle. Writes the canonical MXFP4 form of a
 * prepared weight: w_fp4 [N, K/2] (element at even k in the low nibble) and
 * w_scale [N, K/32] (one E8M0 byte per 32-block). Same shape rules and errors as
 * mx_prepare_weight.
 */
mx_status mx_unprepare_weight(const void* w_prep, int64_t N, int64_t K, void* w_fp4,
                              void* w_scale, hipStream_t stream);

/*
 * Standalone activation quantizer: the same rule as the GEMM's inline quantization,
 * written out in canonical layout ("[gfx1250] Fuse A4W4 stage1 FP4 quantization",
 * Summary: the standalone quant path).
 * a_bf16: [M, K] bf16. a_fp4: [M, K/2] bytes (low nibble = even k). a_scale: [M, K/32]
 * bytes. Requires M >= 0, K > 0, K % 32 == 0. M == 0 is a no-op returning MX_OK.
 */
mx_status mx_quant_act(const void* a_bf16, int64_t M, int64_t K, void* a_fp4, void* a_scale,
                       hipStream_t stream);

/*
 * Workspace the dense GEMM can use at this shape: FP32 partial sums of a split-K
 * reduction (few rows), or, at large M, the activations quantized once into the
 * prepared layout (M rounded up to 64, times K * 17 / 32 bytes), followed, when the
 * 128 x 128 output tiles slightly exceed one round of the chip, by the FP32 partial tiles
 * of the tail tiles' K slices (from the next 256-byte boundary). It is always optional:
 * with a NULL or smaller workspace the library picks a configuration that needs less or
 * none; results stay within the same bound, and are bitwise equal where no K slices are
 * involved (K slices add their partial sums in slice order). 0 for an invalid shape.
 */
size_t mx_a4w4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * The dense A4W4 GEMM ("flydsl_gemm_a4w4" of "[gfx950][FlyDSL] Add direct dense A4W4
 * MXFP4 GEMM", Summary and Implementation): C = Q(A) * Q(W)^T with Q the MXFP4
 * quantization above; A is quantized inside the kernel, never written to memory, except
 * that at large M with a big enough workspace its MXFP4 codes are written once into the
 * workspace and read back by the product kernel (bit-identical results).
 * a_bf16: [M, K] bf16. w_prep: prepared weight of shape [N, K]. c_bf16: [M, N] bf16,
 * rows < M written with the FP32 sum rounded to nearest even. Requires 0 <= M <= 2^30,
 * N % 256 == 0, K % 128 == 0, N <= 2^30, K <= 2^24. M == 0 is a no-op. workspace may be
 * NULL (then workspace_bytes is ignored); a non-NULL workspace must be 16-byte aligned.
 * The call is asynchronous on stream; workspace must stay alive until it completes.
 */
mx_status mx_a4w4_gemm(const void* a_bf16, const void* w_prep, void* c_bf16, int64_t M,
                       int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under stream capture, tight serving
 * loops, harnesses that forbid allocation): mx_a4w4_gemm with the plan it runs when handed
 * mx_a4w4_gemm_workspace_bytes(M, N, K) of workspace, that workspace being the library's own
 * device array of mx_noalloc_scratch_bytes() bytes (32 MiB), one per GPU, held until the
 * process ends; the call allocates and frees nothing. Same arguments, shape rules and results
 * as mx_a4w4_gemm without the workspace pair. MX_ERR_WORKSPACE when the plan needs more than
 * the array holds (e.g. the quantize-once plan at M * K * 17 / 32 > 32 MiB); nothing is
 * launched then. Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (concurrent streams, threads) race and must be serialized by the caller. Nothing in the
 * array needs clearing between calls (each plan writes what it reads).
 */
mx_status mx_a4w4_gemm_noalloc(const void* a_bf16, const void* w_prep, void* c_bf16, int64_t M,
                               int64_t N, int64_t K, hipStream_t stream);

/* Size in bytes of the scratch array mx_a4w4_gemm_noalloc uses. Host only. */
size_t mx_noalloc_scratch_bytes(void);

/*
 * A16WFP4 variant (named in "[gfx950][FlyDSL] Add direct dense A4W4 MXFP4 GEMM", CI Guide, as
 * outside that change): C[M, N] = A[M, K] x W^T with the bf16 activations NOT quantized and
 * W the prepared MXFP4 weight decoded to real values (E2M1 value x 2^(scale - 127), exact
 * in bf16; weight blocks with scale byte 0, block amax below 2^-125, may decode to zero);
 * FP32 accumulation on the bf16 MFMA, bf16 output (round to nearest even); rows >= M are
 * untouched. Same arguments, shape rules and errors as mx_a4w4_gemm, without a workspace.
 */
mx_status mx_a16w4_gemm(const void* a_bf16, const void* w_prep, void* c_bf16, int64_t M,
                        int64_t N, int64_t K, hipStream_t stream);

/*
 * Grouped MoE GEMM1 (expert-segmented dense GEMM, "[HIP] [CK] [FlyDSL] [Kernel] Extend
 * MXFP4 GEMM1 replacement to A4W4", Summary; shape of "[gfx1250] Fuse A4W4 stage1 FP4
 * quantization", Performance). Output row r (expert-sorted order) is
 * Q(A[row_token[r]]) * Q(W_e)^T for the expert e with
 * expert_offsets[e] <= r < expert_offsets[e+1].
 * a_bf16: [T, K] bf16. row_token: [R_max] int32 device array; entries below R are token
 * indices in [0, T) (an index outside that range reads as an all-zero row).
 * expert_offsets: [E+1] int32 device array, non-decreasing, expert_offsets[0] == 0,
 * expert_offsets[E] == R <= R_max (segments are clamped to [0, R_max]).
 * w_prep_stacked: E prepared weights of shape [N, K],
 * expert e at byte offset e * mx_prepared_weight_bytes(N, K) (64-bit addressing).
 * c_bf16: [R_max, N] bf16; rows >= R are untouched. rows_hint: the expected rows per
 * active expert (only a tiling hint; any value >= 1 is correct).
 * Requires E >= 1, T >= 0, R_max >= 0, N % 256 == 0, K % 128 == 0.
 */
mx_status mx_a4w4_gemm_grouped(const void* a_bf16, const int32_t* row_token,
                               const int32_t* expert_offsets, int64_t E, int64_t R_max,
                               const void* w_prep_stacked, void* c_bf16, int64_t T, int64_t N,
                               int64_t K, int64_t rows_hint, hipStream_t stream);

/*
 * Second MoE GEMM (the stage after GEMM1 in "[HIP] [CK] [FlyDSL] [Kernel] Extend MXFP4 GEMM1
 * replacement to A4W4", Summary) on activation rows that are already MXFP4: output row r
 * (expert-sorted order) is Q_r * Q(W_e)^T for the expert e with
 * expert_offsets[e] <= r < expert_offsets[e+1], where Q_r is MXFP4 row r given in
 * canonical form (a_fp4 [R_max, K/2] bytes, element at even k in the low nibble; a_scale
 * [R_max, K/32] E8M0 bytes, 255 outside the contract), e.g. the output of
 * mx_a4w4_gemm_grouped_act_quant or mx_quant_act. No quantization takes place; the sums
 * accumulate in FP32 and are written as bf16 to c_bf16 [R_max, N] (rows >= R untouched).
 * expert_offsets, w_prep_stacked and rows_hint as for mx_a4w4_gemm_grouped.
 * Requires E >= 1, R_max >= 0, N % 256 == 0, K % 128 == 0. Errors: MX_ERR_NULL,
 * MX_ERR_SHAPE, MX_ERR_ALIGN, MX_ERR_DEVICE, MX_ERR_HIP.
 */
mx_status mx_a4w4_gemm_grouped_mx(const void* a_fp4, const void* a_scale, const int32_t* expert_offsets,
                                  int64_t E, int64_t R_max, const void* w_prep_stacked, void* c_bf16,
                                  int64_t N, int64_t K, int64_t rows_hint, hipStream_t stream);

/*
 * Top-k weighted combine of per-row outputs into per-token outputs:
 * out[t, n] = sum over k < topk of token_weights[t, k] * y[token_rows[t, k], n], summed in
 * FP32 in k order and rounded once to bf16 (round to nearest even); a row index outside
 * [0, R) contributes nothing. y_bf16: [R, N] bf16 (e.g. the output of
 * mx_a4w4_gemm_grouped_mx). token_rows: [T, topk] int32; token_weights: [T, topk] float32;
 * out_bf16: [T, N] bf16. Requires R >= 0, T >= 0, 1 <= topk <= 1024, N > 0, N % 8 == 0.
 * T == 0 is a no-op. Errors: MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_ALIGN (y, out: 16 bytes;
 * token_rows, token_weights: 4 bytes), MX_ERR_DEVICE, MX_ERR_HIP.
 */
mx_status mx_moe_combine(const void* y_bf16, int64_t R, const int32_t* token_rows,
                         const float* token_weights, int64_t T, int64_t topk, int64_t N,
                         void* out_bf16, hipStream_t stream);

/* Activation of the fused GEMM1 epilogue. */
enum { MX_ACT_SILU = 0, MX_ACT_SWIGLU = 1 };

/*
 * Grouped MoE GEMM1 with the activation and the MXFP4 quantization for the second GEMM
 * fused into its epilogue ("[gfx1250] Fuse A4W4 stage1 FP4 quantization", Summary: the
 * GEMM1 epilogue emits packed MXFP4 payloads and E8M0 scales directly after SiLU or
 * SwiGLU, the scale computed from the FP32 activation value). Routing, segments and
 * weights are those of mx_a4w4_gemm_grouped; for output row r with GEMM1 row c (FP32):
 *   act == MX_ACT_SWIGLU: h[j] = SiLU(c[j]) * c[N/2 + j], j < Nh = N/2 (gate columns first);
 *   act == MX_ACT_SILU:   h[j] = SiLU(c[j]), j < Nh = N;  SiLU(x) = x / (1 + exp(-x)),
 * evaluated in FP32 with the hardware exponential and reciprocal (relative error at most
 * (|x| + 8) * 2^-23).
 * h is quantized along its columns with the rule at the top of this file applied to the
 * FP32 value of h (E8M0 scale from the FP32 block amax, one conversion to E2M1) and written
 * in canonical form: h_fp4 [R_max, Nh/2] bytes (element at even j in the low nibble),
 * h_scale [R_max, Nh/32] bytes; rows >= R are untouched. Because h is formed in FP32 from
 * FP32 accumulators, a code or scale whose exact value lies at a rounding boundary may
 * differ from the exact product's by one step. Requirements and errors as for
 * mx_a4w4_gemm_grouped, plus act in {MX_ACT_SILU, MX_ACT_SWIGLU} (else MX_ERR_SHAPE).
 */
mx_status mx_a4w4_gemm_grouped_act_quant(const void* a_bf16, const int32_t* row_token,
                                         const int32_t* expert_offsets, int64_t E, int64_t R_max,
                                         const void* w_prep_stacked, int64_t T, int64_t N, int64_t K,
                                         int32_t act, int64_t rows_hint, void* h_fp4, void* h_scale,
                                         hipStream_t stream);

/*
 * Introspection (host only, no GPU needed): the kernel instantiation(s) mx_a4w4_gemm
 * would launch for (M, N, K) with a workspace of workspace_bytes, e.g.
 * "k_gemm_tile<1, 4, 4, 4, 1, 2> GM=8" or "k_gemm_stream<1, 1, 2, 16, 1> S=1", written
 * NUL-terminated (truncated to buf_len) into the caller's host buffer; "none" for M == 0.
 * The names match the kernel names a profiler reports. Honours the library's tuning
 * override (environment variable MX_GEMM_CONFIG) like the GEMM itself. Errors:
 * MX_ERR_SHAPE (as mx_a4w4_gemm), MX_ERR_NULL (buf NULL or buf_len 0), MX_ERR_HIP (the
 * override names no configuration that can run this call; the GEMM would fail the same way).
 */
mx_status mx_a4w4_gemm_plan(int64_t M, int64_t N, int64_t K, size_t workspace_bytes, char* buf,
                            size_t buf_len);

/*
 * Introspection (host only, no GPU needed): the kernel instantiation mx_a16w4_gemm would
 * launch for (M, N, K): "k_gemm_a16w4_stream<MT, NG, WK, PD>" (decode M, at most 32 rows) or
 * "k_gemm_a16w4 (64 x 256 tiles)", written NUL-terminated (truncated to buf_len) into the
 * caller's host buffer; "none" for M == 0. Errors: MX_ERR_SHAPE (as mx_a16w4_gemm),
 * MX_ERR_NULL (buf NULL or buf_len 0).
 */
mx_status mx_a16w4_gemm_plan(int64_t M, int64_t N, int64_t K, char* buf, size_t buf_len);

/*
 * The same for mx_a4w4_gemm_grouped with E experts, R_max rows and T tokens (the choice
 * may depend on any of them; tuning override MX_GROUPED_CONFIG); "none" for R_max == 0. Same shape rules and errors as the grouped
 * GEMM, plus MX_ERR_NULL for buf.
 */
mx_status mx_a4w4_gemm_grouped_plan(int64_t E, int64_t R_max, int64_t T, int64_t N, int64_t K,
                                    int64_t rows_hint, char* buf, size_t buf_len);

/*
 * The same for mx_a4w4_gemm_grouped_act_quant (its kernel depends on E, R_max, N, act and
 * the hint, as for the call; tuning override MX_GROUPED_CONFIG="gt,..."). Errors:
 * MX_ERR_SHAPE (E, R_max, shape or act as for the call), MX_ERR_NULL (buf), MX_ERR_HIP (the
 * override names no fused configuration for N).
 */
mx_status mx_a4w4_gemm_grouped_act_quant_plan(int64_t E, int64_t R_max, int64_t N, int64_t K,
                                              int32_t act, int64_t rows_hint, char* buf,
                                              size_t buf_len);

/* The same for mx_a4w4_gemm_grouped_mx (its kernel depends on N, K and the hint). Errors as
 * for mx_a4w4_gemm_grouped_act_quant_plan. */
mx_status mx_a4w4_gemm_grouped_mx_plan(int64_t N, int64_t K, int64_t rows_hint, char* buf,
                                       size_t buf_len);

#ifdef __cplusplus
}
#endif

#endif /* MX_H_ */
