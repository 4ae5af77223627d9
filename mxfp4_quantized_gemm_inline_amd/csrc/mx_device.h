// mx_device.h - device-side building blocks for gfx950: the MXFP4 block quantizer,
// the prepared-weight layout, and the block-scaled FP4 MFMA wrapper.
//
// MXFP4 (E2M1 elements, one E8M0 scale per 32 elements along K) as used by
// "[gfx950][FlyDSL] Add direct dense A4W4 MXFP4 GEMM", Summary. The block exponent is
// floor(log2 amax) - 2 clamped to [-127, 127] (OCP MX v1.0 conversion with the E2M1
// maximum exponent 2); elements round to nearest even and saturate at 6.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 32;      // elements per E8M0 scale
constexpr int kStepK = 128;     // K covered by one 16x16x128 MFMA
constexpr int kFragBytes = 16;  // one lane's share of an MFMA operand: one 32-block
constexpr int kLayoutVersion = 2;

// ------------------------------------------------------------------ prepared weight layout
//
// Payload: for column group g (16 columns n = 16g..16g+15) and K step t (k = 128t..128t+127)
// one 1 KiB tile; lane l = (n % 16) + 16 * ((k % 128) / 32) owns bytes [16l, 16l+16), which
// are the 32-block (n, kb = 4t + l/16) in canonical order (element at even k in the low
// nibble). This is exactly the operand layout of the 16x16x128 FP4 MFMA, so one
// global_load_dwordx4 per lane fetches a whole operand and a wave's load is 1 KiB contiguous.
// Tiles are ordered [g][t]: a column group's whole K range is contiguous.
//
// Scales: after the payload, for column-group quad q (groups 4q..4q+3, columns 64q..64q+63)
// and K step t, one 32-bit word per lane l whose byte j is the E8M0 scale of
// (n = 16 (4q + j) + l % 16, kb = 4t + l / 16). Byte j is the MFMA scale op_sel for column
// group 4q + j, so a wave that owns four adjacent column groups fetches all their scales
// for a step with one dword load per lane. The scale region is exactly N * K / 32 bytes.
__host__ __device__ inline int steps_of(int K) { return K / kStepK; }
__host__ __device__ inline size_t payload_bytes(int64_t N, int64_t K) { return (size_t)N * (size_t)K / 2; }
__host__ __device__ inline size_t scale_region_bytes(int64_t N, int64_t K) { return (size_t)N * (size_t)K / 32; }
__host__ __device__ inline size_t prepared_bytes(int64_t N, int64_t K) {
  return payload_bytes(N, K) + scale_region_bytes(N, K);
}
__host__ __device__ inline size_t wp_payload_off(int g, int t, int lane, int T) {
  return (((size_t)g * T + t) * 64 + lane) * 16;
}
// byte offset of the scale word of (column-group quad q, step t, lane)
__host__ __device__ inline size_t wp_scale_off(int q, int t, int lane, int T) {
  return (((size_t)q * T + t) * 64 + lane) * 4;
}

// ------------------------------------------------------------------ bf16 helpers

// FP32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  uint2 r;
  r.x = f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16);
  r.y = f32_to_bf16_rne(c) | (f32_to_bf16_rne(d) << 16);
  return r;
}

// ------------------------------------------------------------------ the block quantizer

// E8M0 scale byte of a 32-element bf16 block held as 16 words of bf16 pairs.
// For a finite block, floor(log2 amax) is (E - 127) with E the largest exponent field, so
// s = e + 127 = max(E - 2, 0); subnormal and zero blocks (E = 0) give 0.
__device__ __forceinline__ uint32_t block_scale_byte(const uint32_t (&x)[16]) {
  u16x2 m[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    u16x2 a = __builtin_bit_cast(u16x2, x[2 * i] & 0x7F807F80u);
    u16x2 b = __builtin_bit_cast(u16x2, x[2 * i + 1] & 0x7F807F80u);
    m[i] = __builtin_elementwise_max(a, b);
  }
#pragma unroll
  for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) m[i] = __builtin_elementwise_max(m[i], m[i + w]);
  uint32_t hi = m[0].x > m[0].y ? m[0].x : m[0].y;
  uint32_t E = hi >> 7;
  return E > 2u ? E - 2u : 0u;
}

// Quantize one block: q[j] byte b holds elements (8j + 2b) (low nibble) and (8j + 2b + 1).
// The hardware conversion divides by the scale operand, rounds to nearest even, saturates
// and keeps the sign of zero; a scale byte of 0 is passed as the fp32 value 2^-127.
__device__ __forceinline__ uint32_t quant_block(const uint32_t (&x)[16], uint32_t (&q)[4]) {
  const uint32_t s = block_scale_byte(x);
  const float sc = __builtin_bit_cast(float, s ? (s << 23) : 0x00400000u);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, x[4 * j + 0]), sc, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, x[4 * j + 1]), sc, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, x[4 * j + 2]), sc, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, x[4 * j + 3]), sc, 3);
    q[j] = r;
  }
  return s;
}

// Load one 32-element bf16 block (64 bytes, 16-byte aligned) into 16 words.
__device__ __forceinline__ void load_block(const uint16_t* __restrict__ p, uint32_t (&x)[16]) {
  const uint4* v = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 u = v[i];
    x[4 * i + 0] = u.x; x[4 * i + 1] = u.y; x[4 * i + 2] = u.z; x[4 * i + 3] = u.w;
  }
}

// 16-byte streaming load (non-temporal: data read once, e.g. the prepared weight).
__device__ __forceinline__ uint4 load16_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Load one 32-element bf16 block at byte offset `off` from a wave-uniform base (the
// compiler can then use a scalar base with a 32-bit per-lane offset).
__device__ __forceinline__ void load_block_at(const uint8_t* __restrict__ base, uint32_t off, uint32_t (&x)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = *reinterpret_cast<const uint4*>(base + off + 16 * i);
    x[4 * i + 0] = u.x; x[4 * i + 1] = u.y; x[4 * i + 2] = u.z; x[4 * i + 3] = u.w;
  }
}

__device__ __forceinline__ void zero_block(uint32_t (&x)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = 0u;
}

// ------------------------------------------------------------------ launch helpers

// Tile order: CTAs are dealt round-robin to the 8 XCDs (blockIdx % 8), each with its own
// L2, so CTA i is given logical tile (its XCD's contiguous share) and logical tiles walk
// GM tile-rows at a time; the CTAs resident on one XCD then share activation rows and
// weight columns in that XCD's L2.
// Logical tile -> (tile row, tile column): GM tile-rows at a time, down the rows first.
__device__ __forceinline__ void logical_tile(int logical, int tiles_m, int tiles_n, int GM, int& bm, int& bn) {
  const int gsize = GM * tiles_n;
  const int grp = logical / gsize, first = grp * GM;
  const int gm = min(tiles_m - first, GM);
  const int rem = logical - grp * gsize;
  bm = first + rem % gm;
  bn = rem / gm;
}
__device__ __forceinline__ void tile_coords(int i, int total, int tiles_m, int tiles_n, int GM, int& bm,
                                            int& bn) {
  const int q = total / 8, r = total % 8;
  const int x = i % 8, j = i / 8;
  logical_tile(x * q + min(x, r) + j, tiles_m, tiles_n, GM, bm, bn);
}

template <int N_, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) { (f(std::integral_constant<int, I>{}), ...); }(
      std::make_integer_sequence<int, N_>{});
}

// ------------------------------------------------------------------ MFMA

// acc += (a * 2^(sa-127)) (16 x 128 FP4, rows) times (b * 2^(sb-127)) (128 x 16 FP4, cols).
// Lane l supplies row/col l % 16, K block l / 16 of each operand and the scale byte for it
// in byte 0 of sa / sb. acc lane l, element r is C[row 4*(l/16) + r][col l % 16].
__device__ __forceinline__ v4f mfma_fp4(const uint4& a, const uint4& b, v4f acc, uint32_t sa, uint32_t sb) {
  v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 4, 4, 0, (int)sa, 0, (int)sb);
}

// Same, with the scales taken from byte SA of sa and byte SB of sb (the op_sel fields).
template <int SA, int SB>
__device__ __forceinline__ v4f mfma_fp4_sel(const uint4& a, const uint4& b, v4f acc, uint32_t sa, uint32_t sb) {
  v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 4, 4, SA, (int)sa, SB, (int)sb);
}

// Same on native 4 x 32-bit vectors (what LDS and global loads of 16 bytes return).
template <int SA, int SB>
__device__ __forceinline__ v4f mfma_fp4_sel(const u32x4& a, const u32x4& b, v4f acc, uint32_t sa, uint32_t sb) {
  v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 4, 4, SA, (int)sa, SB, (int)sb);
}

// The block-scaled FP4 MFMA through inline assembly with the accumulator tied to the
// destination ("+a", an AGPR tuple), for waves whose 64 accumulators fill the AGPRs: through
// the builtin the compiler picked the untied form at that register pressure and rotated
// accumulators through copies every step. The compiler still places the s_waitcnt for the
// operands (it sees the assembly read them); what it cannot see is the MFMA's own result
// latency, so a VALU read of an accumulator after the last MFMA needs mfma_drain() first.
// VACC = true keeps the accumulator in VGPRs instead ("+v"), for tiles with more accumulators
// than the AGPRs hold.
template <int SA, int SB, bool VACC = false>
__device__ __forceinline__ void mfma_fp4_tied(v4f& acc, const u32x4& a, const u32x4& b, uint32_t sa, uint32_t sb) {
  // scale byte select: A byte = op_sel[0] | 2 op_sel_hi[0], B byte = op_sel[1] | 2 op_sel_hi[1]
#define MXQ(A0, A1, B0, B1)                                                                                    \
  do {                                                                                                        \
    if constexpr (VACC)                                                                                       \
      asm("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[" #A0 "," #B0 ",0] op_sel_hi:[" #A1 \
          "," #B1 ",0] cbsz:4 blgp:4"                                                                         \
          : "+v"(acc)                                                                                       \
          : "v"(a), "v"(b), "v"(sa), "v"(sb));                                                              \
    else                                                                                                      \
      asm("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[" #A0 "," #B0 ",0] op_sel_hi:[" #A1 \
          "," #B1 ",0] cbsz:4 blgp:4"                                                                         \
          : "+a"(acc)                                                                                       \
          : "v"(a), "v"(b), "v"(sa), "v"(sb));                                                              \
  } while (0)
  if constexpr (SA == 0 && SB == 0) MXQ(0, 0, 0, 0);
  else if constexpr (SA == 0 && SB == 1) MXQ(0, 0, 1, 0);
  else if constexpr (SA == 0 && SB == 2) MXQ(0, 0, 0, 1);
  else if constexpr (SA == 0 && SB == 3) MXQ(0, 0, 1, 1);
  else if constexpr (SA == 1 && SB == 0) MXQ(1, 0, 0, 0);
  else if constexpr (SA == 1 && SB == 1) MXQ(1, 0, 1, 0);
  else if constexpr (SA == 1 && SB == 2) MXQ(1, 0, 0, 1);
  else if constexpr (SA == 1 && SB == 3) MXQ(1, 0, 1, 1);
  else if constexpr (SA == 2 && SB == 0) MXQ(0, 1, 0, 0);
  else if constexpr (SA == 2 && SB == 1) MXQ(0, 1, 1, 0);
  else if constexpr (SA == 2 && SB == 2) MXQ(0, 1, 0, 1);
  else if constexpr (SA == 2 && SB == 3) MXQ(0, 1, 1, 1);
  else if constexpr (SA == 3 && SB == 0) MXQ(1, 1, 0, 0);
  else if constexpr (SA == 3 && SB == 1) MXQ(1, 1, 1, 0);
  else if constexpr (SA == 3 && SB == 2) MXQ(1, 1, 0, 1);
  else MXQ(1, 1, 1, 1);
#undef MXQ
}

// 32 wait states between the last MFMA's accumulator write and the moves that read them.
__device__ __forceinline__ void mfma_drain() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace mx
