// mx_gemm_qo.hip - the quantize-once A4W4 GEMM for large M on gfx950.
//
// Operation: the dense A4W4 MXFP4 GEMM of "[gfx950][FlyDSL] Add direct dense A4W4 MXFP4 GEMM",
// Summary and Implementation. At large M with long K every activation block would otherwise be
// re-read as bf16 and re-quantized once per output column tile (33 times at N = 8448 with
// 256-wide tiles), and that page's own microbenchmark table shows a split quantize-then-GEMM
// path overtaking the inline kernel at its largest shape (8448 x 7168, M = 2048). Here the bf16
// rows are quantized once, with the quantizer every kernel of this library uses, into the
// prepared operand layout (k_prepare on M rows padded to a multiple of 64, in the caller's
// workspace), and k_gemm_qo multiplies the two prepared operands.
//
// k_gemm_qo: a CTA owns a BM x BN output tile; WM x WN waves compute MT x NG 16x16x128
// block-scaled FP4 MFMA tiles each, accumulating in ordinary VGPRs (where the scaled MFMA
// accumulates in place; with accumulators in AGPRs the compiler rotated them through copies
// every step, so a wave computes at most 128 x 64). Per 128-wide K step both operands (BM/16
// + BN/16 blocks of 1 KiB and their 256-byte scale-word chunks) go from global memory straight
// into LDS with global_load_lds_dwordx4 / _dword: each lane's 16 (4) bytes land at the block's
// LDS base + 16 l (4 l), which is the MFMA operand layout itself, so no register holds data in
// flight and a ring of NBUF stage buffers keeps NBUF - 2 steps of copies outstanding beyond the
// one being published. The MFMA operand reads are plain 16-byte LDS reads of a lane's own
// operand (bank-conflict free), and the scale bytes come from the op_sel fields.
//
// Orientation as in the inline kernels: the weight is the MFMA "A" operand (16 output columns
// as rows) and the activations the "B" operand, so lane l's accumulator element r is
// C[m = l % 16][n = 4 (l / 16) + r]. The per-element sum runs over K steps in order 0..T-1,
// as in every inline kernel without K slices, so both paths give bitwise equal results.
#include <atomic>
#include <cstdio>

#include "mx_device.h"
#include "mx_internal.h"

namespace mx {
namespace {

// Epilogue: stage the bf16 tile in LDS (rows padded by 16 bytes), then store whole rows, 16
// bytes per lane; rows >= M and columns >= N are never written. The LDS must be free (every
// wave past its last operand read) and hold BM x (2 BN + 16) bytes.
template <int BM, int BN, int MT, int NG, int WN>
__device__ __forceinline__ void store_tile(const v4f (&acc)[NG][MT], uint8_t* smem, uint16_t* __restrict__ C,
                                           int M, int N, int bm, int bn) {
  constexpr int CROW = BN * 2 + 16, NTH = (BM / (16 * MT)) * WN * 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w / WN, wn = w % WN;
#pragma unroll
  for (int j = 0; j < NG; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int r = 16 * (wm * MT + i) + (lane & 15);
      const int cl = 16 * (wn * NG + j) + 4 * (lane >> 4);
      *reinterpret_cast<uint2*>(smem + r * CROW + cl * 2) =
          pack4_bf16(acc[j][i][0], acc[j][i][1], acc[j][i][2], acc[j][i][3]);
    }
  __syncthreads();
  constexpr int CPR = BN / 8;  // 16-byte chunks per tile row
  static_assert((BM * CPR) % NTH == 0, "every thread stores the same number of chunks");
  const int m0 = bm * BM, n0 = bn * BN;
#pragma unroll
  for (int k = 0; k < BM * CPR / NTH; ++k) {
    const int id = threadIdx.x + k * NTH;
    const int r = id / CPR, ch = id % CPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * CROW + ch * 16);
    if (m0 + r < M && n0 + 8 * ch < N)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(C + (size_t)(m0 + r) * N + n0 + 8 * ch));
  }
}

// The copies are issued through inline assembly: the compiler's builtin for them marks the
// instruction as touching both global memory and LDS, after which every later wait it places
// becomes a full drain (vmcnt(0) / lgkmcnt(0)), and __syncthreads() would drain every copy in
// flight too (its fence waits on all outstanding memory operations). The assembly writes no
// vector register (the data goes to LDS; the address operands are read at issue), saves and
// restores m0 around the copy and declares memory clobbered, so no memory access is moved
// across it; its completion is awaited by the explicit waits in the kernel.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* l) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)l);
}
__device__ __forceinline__ void copy16(const uint8_t* g, const uint8_t* l) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(g), "s"(lds_addr(l))
      : "memory");
}
__device__ __forceinline__ void copy4(const uint8_t* g, const uint8_t* l) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(g), "s"(lds_addr(l))
      : "memory");
}
// s_waitcnt immediate for vmcnt(vm) expcnt(7) lgkmcnt(lgkm) (vmcnt split over bits 3:0 and
// 15:14, expcnt bits 6:4, lgkmcnt bits 11:8).
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}
static_assert(waitcnt_imm(0, 0) == 0x70 && waitcnt_imm(5, 15) == 0xF75 && waitcnt_imm(17, 0) == 0x4071,
              "s_waitcnt encoding");

template <int WM, int WN, int MT, int NG, int NBUF>
struct QOShape {
  static constexpr int NW = WM * WN, NTH = 64 * NW;
  static constexpr int BM = 16 * MT * WM, BN = 16 * NG * WN;
  static constexpr int GA = BM / 16, GW = BN / 16;  // 1 KiB operand blocks per stage
  static constexpr int QA = BM / 64, QW = BN / 64;  // 256-byte scale-word chunks per stage
  static constexpr int NB = GA + GW, NS = QA + QW;
  static constexpr int SC_OFF = NB * 1024;          // the scale chunks follow the blocks
  static constexpr int STAGE = NB * 1024 + NS * 256;
  static constexpr int BPW = (NB + NW - 1) / NW, SPW = (NS + NW - 1) / NW;  // copies per wave
  static constexpr int CSTAGE = BM * (BN * 2 + 16);
  static constexpr int SMEM = NBUF * STAGE > CSTAGE ? NBUF * STAGE : CSTAGE;
  static_assert(MT % 4 == 0 && NG % 4 == 0, "a wave's tiles cover whole scale words");
  static_assert(NBUF >= 3, "stage t + 1 is read while stage t + NBUF - 1 is being copied");
  static_assert(SMEM <= 160 * 1024, "the stages and the output staging fit the LDS");
};

// Ap: activations in the prepared layout for Mp = round_up(M, 64) rows (rows >= M are zero
// blocks); Wp: the prepared weight [N, K]; C: bf16 [M, N]. Rows >= M and columns >= N of a
// tile are computed from clamped (valid) operand blocks and never stored.
template <int WM, int WN, int MT, int NG, int NBUF, int OCC>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void k_gemm_qo(const uint8_t* __restrict__ Ap, const uint8_t* __restrict__ Wp, uint16_t* __restrict__ C, int M,
               int N, int K, int GM) {
  using S = QOShape<WM, WN, MT, NG, NBUF>;
  constexpr int NW = S::NW, GA = S::GA, QA = S::QA, BPW = S::BPW, SPW = S::SPW, STAGE = S::STAGE;
  constexpr int MH = MT / 2, NQ = NG / 4, D = BPW + SPW;  // D: copies each wave issues per step
  extern __shared__ __align__(16) uint8_t smem[];
  const int T = steps_of(K);
  const int Mp = (M + 63) / 64 * 64;
  const int GAall = Mp / 16, GWall = N / 16;
  const int tiles_m = (M + S::BM - 1) / S::BM, tiles_n = (N + S::BN - 1) / S::BN;
  int bm, bn;
  tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, GM, bm, bn);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w / WN, wn = w % WN;
  const uint32_t l16 = lane * 16, l4 = lane * 4;

  // Copy slot i of this wave is CTA block min(w + NW i, NB - 1) (an idle slot repeats the last
  // block: the same bytes written twice) and scale chunk min(w + NW i, NS - 1); the global
  // source is clamped to a valid row or column group.
  const uint8_t* src[BPW];
  int dstb[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int b = min(w + NW * i, S::NB - 1);
    dstb[i] = b * 1024;
    src[i] = (b < GA ? Ap + (size_t)min(bm * GA + b, GAall - 1) * T * 1024
                     : Wp + (size_t)min(bn * S::GW + (b - GA), GWall - 1) * T * 1024) + l16;
  }
  const uint8_t* ssrc[SPW];
  int dsts[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int c = min(w + NW * i, S::NS - 1);
    dsts[i] = S::SC_OFF + c * 256;
    ssrc[i] = (c < QA ? Ap + payload_bytes(Mp, K) + (size_t)min(bm * QA + c, GAall / 4 - 1) * T * 256
                      : Wp + payload_bytes(N, K) + (size_t)min(bn * S::QW + (c - QA), GWall / 4 - 1) * T * 256) + l4;
  }
  auto copy_stage = [&](int t, int buf) {
    uint8_t* L = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < BPW; ++i) copy16(src[i] + (size_t)t * 1024, L + dstb[i]);
#pragma unroll
    for (int i = 0; i < SPW; ++i) copy4(ssrc[i] + (size_t)t * 256, L + dsts[i]);
  };

  v4f acc[NG][MT];
#pragma unroll
  for (int j = 0; j < NG; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[j][i] = v4f{0.f, 0.f, 0.f, 0.f};
  // a[P][i]: step t's first-half activation operands in set P = t % 2 (the next step's are read
  // into the other set at the start of the step), ah: the second half (read at the start of the
  // step from its own buffer), b: the weight operands (each re-read for the next step after its
  // last use); scale words double-buffered by parity.
  u32x4 a[2][MH], ah[MT - MH], b[NG];
  uint32_t sa[2][MT / 4], sb[2][NQ];
  auto rd_a = [&](int buf, int i) {
    return *reinterpret_cast<const u32x4*>(smem + buf * STAGE + (wm * MT + i) * 1024 + l16);
  };
  auto rd_b = [&](int buf, int j) {
    return *reinterpret_cast<const u32x4*>(smem + buf * STAGE + (GA + wn * NG + j) * 1024 + l16);
  };
  auto rd_scales = [&](int buf, auto r_c) {
    constexpr int R = decltype(r_c)::value;
    const uint8_t* L = smem + buf * STAGE + S::SC_OFF;
#pragma unroll
    for (int q = 0; q < MT / 4; ++q) sa[R][q] = *reinterpret_cast<const uint32_t*>(L + (wm * (MT / 4) + q) * 256 + l4);
#pragma unroll
    for (int q = 0; q < NQ; ++q) sb[R][q] = *reinterpret_cast<const uint32_t*>(L + (QA + wn * NQ + q) * 256 + l4);
  };
  auto mfma_at = [&](auto j_c, auto i_c, auto r_c) {
    constexpr int j = decltype(j_c)::value, i = decltype(i_c)::value, R = decltype(r_c)::value;
    const u32x4& av = i < MH ? a[R][i < MH ? i : 0] : ah[i < MH ? 0 : i - MH];
    acc[j][i] = mfma_fp4_sel<j & 3, i & 3>(b[j], av, acc[j][i], sb[R][j >> 2], sa[R][i >> 2]);
  };

  // Prologue: stages 0 .. NBUF - 2 copied, stages 0 and 1 complete and published, step 0's
  // first-half activation operands, weights and scales read.
  for (int s = 0; s < NBUF - 1; ++s) copy_stage(min(s, T - 1), s);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm((NBUF - 3) * D, 0));
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < MH; ++i) a[0][i] = rd_a(0, i);
#pragma unroll
  for (int j = 0; j < NG; ++j) b[j] = rd_b(0, j);
  rd_scales(0, std::integral_constant<int, 0>{});

  // Step t (its buffer t % NBUF; stage t + 1 in the next buffer, complete since the last
  // barrier): read the second-half activation operands of step t and step t + 1's first-half
  // operands and scale words; copy stage t + NBUF - 1 into the buffer of step t - 1 (read last
  // before the barrier that ended step t - 1); run the first-half MFMAs, then the second-half
  // ones, reading each next weight operand after its last use; then wait for the copies of
  // stage t + 2 (the only ones allowed to remain are those of the NBUF - 3 stages after it) and
  // for this wave's LDS reads (so the buffer they read may be refilled), and meet at the
  // barrier. Steps past the last copy the last step again: branch-free, never used. The fences
  // keep each phase in place (the MFMAs touch no memory, so the scheduler could move them).
  auto step = [&](int t, int b0, int b1, int bc, auto par_c) {
    constexpr int P = decltype(par_c)::value;  // t % 2
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = MH; i < MT; ++i) ah[i - MH] = rd_a(b0, i);
#pragma unroll
    for (int i = 0; i < MH; ++i) a[P ^ 1][i] = rd_a(b1, i);
    rd_scales(b1, std::integral_constant<int, P ^ 1>{});
    copy_stage(min(t + NBUF - 1, T - 1), bc);
    __builtin_amdgcn_sched_barrier(0);
    static_for<MH>([&](auto i_c) { static_for<NG>([&](auto j_c) { mfma_at(j_c, i_c, par_c); }); });
    __builtin_amdgcn_sched_barrier(0);
    static_for<NG>([&](auto j_c) {
      static_for<MT - MH>([&](auto i_c) {
        mfma_at(j_c, std::integral_constant<int, MH + decltype(i_c)::value>{}, par_c);
      });
      b[decltype(j_c)::value] = rd_b(b1, decltype(j_c)::value);
    });
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm((NBUF - 3) * D, 0));
    __builtin_amdgcn_s_barrier();
  };
  int t = 0, b0 = 0;
  auto nxt = [](int x) { return x + 1 == NBUF ? 0 : x + 1; };
  auto prv = [](int x) { return x == 0 ? NBUF - 1 : x - 1; };
  for (; t + 2 <= T; t += 2) {
    step(t, b0, nxt(b0), prv(b0), std::integral_constant<int, 0>{});
    b0 = nxt(b0);
    step(t + 1, b0, nxt(b0), prv(b0), std::integral_constant<int, 1>{});
    b0 = nxt(b0);
  }
  if (t < T) step(t, b0, nxt(b0), prv(b0), std::integral_constant<int, 0>{});
  // every copy has landed and every wave is done with the stage buffers before the staging
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  __syncthreads();
  store_tile<S::BM, S::BN, MT, NG, WN>(acc, smem, C, M, N, bm, bn);
}

// ---------------------------------------------------------------------- k_gemm_qr
//
// The register-direct form: one wave per SIMD owns a 16 MT x 16 NG output tile and streams
// both prepared operands straight from global memory into its registers, D steps ahead,
// with no LDS and no barrier in the K loop, so no wave ever waits for another. Its
// accumulators are tied in place (mfma_fp4_tied): the first 64 (a 128 x 128 tile) fill the
// 256 AGPRs, further accumulator rows (NG > 64 / MT) live in VGPRs. Every step's loads are
// fenced as a group ahead of its MFMAs so that D steps stay in flight.
//
// NG need not be a multiple of four: then a tile's first weight column group g0 = NG bn can
// sit at any byte of a scale word, and each step's weight scale words are realigned by
// g0 % 4 bytes (one v_alignbyte per word) so that group j's scale is byte j % 4 of word j / 4
// for the compile-time op_sel. The last column tile may reach past N: its loads are clamped
// to the last column group and its columns >= N never stored. Tile widths that are not a
// power of two let the tile count fit the chip (8448 x 2048 in 128 x 144 tiles: 944 waves,
// one round, where 128 x 128 tiles number 1056).
//
// When the tiles exceed one wave per SIMD (1024) by a little the last `tail` logical tiles
// would run as a second, nearly empty round; instead each is cut into `slices` K ranges run
// by CTAs of their own, which write FP32 partial tiles, and k_qr_tail_reduce adds them in
// slice order. The other tiles sum their K steps in order 0..T-1, as every inline kernel
// does.

template <int MT, int NG>
struct RDWave {
  static constexpr int BM = 16 * MT, BN = 16 * NG;
  static constexpr bool AAL = MT % 4 == 0;                         // first row group % 4 == 0
  static constexpr int MQL = AAL ? MT / 4 : (MT + 2) / 4 + 1;      // activation scale words loaded
  static constexpr int MQ = (MT + 3) / 4;                          // ... after realignment
  static constexpr bool WAL = NG % 4 == 0;                         // g0 % 4 == 0 for every tile
  static constexpr int NQL = WAL ? NG / 4 : (NG + 2) / 4 + 1;      // weight scale words loaded
  static constexpr int NQ = (NG + 3) / 4;                          // ... after realignment
  static constexpr int JA = 64 / MT;                               // accumulator rows in the AGPRs
  static_assert(MT >= 1 && MT <= 16 && NG >= 1, "tile of 1..16 row groups");
};

// One wave's K steps t0 .. t1 - 1 of output tile (bm, bn) into acc (zeroed here). Ap holds the
// activations prepared for Mp = round_up(M, 64) rows, Wp the prepared weight [N, K].
template <int MT, int NG, int D>
__device__ __forceinline__ void rd_steps(v4f (&acc)[NG][MT], const uint8_t* __restrict__ Ap,
                                         const uint8_t* __restrict__ Wp, int M, int N, int K, int bm, int bn,
                                         int t0, int t1, int lane) {
  using R = RDWave<MT, NG>;
  constexpr int S = D + 1;  // register sets in the ring
  const int T = steps_of(K);
  const int Mp = (M + 63) / 64 * 64;
  const int GAall = Mp / 16, GW = N / 16;
  const int g0 = bn * NG, a0 = bm * MT;
  const uint32_t vsh = (uint32_t)(g0 & 3), vsha = (uint32_t)(a0 & 3);
  const uint8_t* pa[MT];
  const uint8_t* pw[NG];
  const uint8_t* psa[R::MQL];
  const uint8_t* psw[R::NQL];
#pragma unroll
  for (int i = 0; i < MT; ++i) pa[i] = Ap + (size_t)min(a0 + i, GAall - 1) * T * 1024;
#pragma unroll
  for (int j = 0; j < NG; ++j) pw[j] = Wp + (size_t)min(g0 + j, GW - 1) * T * 1024;
#pragma unroll
  for (int q = 0; q < R::MQL; ++q)
    psa[q] = Ap + payload_bytes(Mp, K) + (size_t)min((a0 >> 2) + q, GAall / 4 - 1) * T * 256;
#pragma unroll
  for (int q = 0; q < R::NQL; ++q)
    psw[q] = Wp + payload_bytes(N, K) + (size_t)min((g0 >> 2) + q, GW / 4 - 1) * T * 256;

  // ring set s holds step t's operands for (t - t0) % S == s; steps past the last load the
  // last step again (never used)
  u32x4 a[S][MT], b[S][NG];
  uint32_t sa[S][R::MQL], sb[S][R::NQL];
  const int tlast = max(t1 - 1, 0);
  auto load = [&](int t, auto s_c) {
    constexpr int s = decltype(s_c)::value;
    const uint32_t tt = (uint32_t)min(t, tlast);
    const uint32_t o = tt * 1024 + lane * 16, os = tt * 256 + lane * 4;
#pragma unroll
    for (int i = 0; i < MT; ++i) a[s][i] = *reinterpret_cast<const u32x4*>(pa[i] + o);
#pragma unroll
    for (int j = 0; j < NG; ++j) b[s][j] = *reinterpret_cast<const u32x4*>(pw[j] + o);
#pragma unroll
    for (int q = 0; q < R::MQL; ++q) sa[s][q] = *reinterpret_cast<const uint32_t*>(psa[q] + os);
#pragma unroll
    for (int q = 0; q < R::NQL; ++q) sb[s][q] = *reinterpret_cast<const uint32_t*>(psw[q] + os);
  };
#pragma unroll
  for (int j = 0; j < NG; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[j][i] = v4f{0.f, 0.f, 0.f, 0.f};
  auto mfmas = [&](auto s_c) {
    constexpr int s = decltype(s_c)::value;
    uint32_t sw[R::NQ], sv[R::MQ];
    static_for<R::NQ>([&](auto q_c) {
      constexpr int q = decltype(q_c)::value;
      if constexpr (R::WAL)
        sw[q] = sb[s][q];
      else  // bytes g0 % 4 + 4 q .. + 3 of the loaded words
        sw[q] = __builtin_amdgcn_alignbyte(sb[s][q + 1 < R::NQL ? q + 1 : R::NQL - 1], sb[s][q], vsh);
    });
    static_for<R::MQ>([&](auto q_c) {
      constexpr int q = decltype(q_c)::value;
      if constexpr (R::AAL)
        sv[q] = sa[s][q];
      else  // the same for the activation row groups a0 ..
        sv[q] = __builtin_amdgcn_alignbyte(sa[s][q + 1 < R::MQL ? q + 1 : R::MQL - 1], sa[s][q], vsha);
    });
    static_for<NG>([&](auto j_c) {
      constexpr int j = decltype(j_c)::value;
      static_for<MT>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        mfma_fp4_tied<j & 3, i & 3, (j >= R::JA)>(acc[j][i], b[s][j], a[s][i], sw[j >> 2], sv[i >> 2]);
      });
    });
  };

  static_for<D>([&](auto s_c) { load(t0 + decltype(s_c)::value, s_c); });
  int t = t0;
  for (; t + S <= t1; t += S) {
    static_for<S>([&](auto s_c) {
      constexpr int s = decltype(s_c)::value;
      __builtin_amdgcn_sched_barrier(0);
      load(t + s + D, std::integral_constant<int, (s + D) % S>{});
      __builtin_amdgcn_sched_barrier(0);
      mfmas(s_c);
    });
  }
  // the last (t1 - t0) % S steps (their operands are in sets 0 .. (t1 - t0) % S - 1)
  static_for<S - 1>([&](auto s_c) {
    if (t + decltype(s_c)::value < t1) mfmas(s_c);
  });
  mfma_drain();
}

template <int MT, int NG>
struct QRShape {
  static constexpr int BM = 16 * MT, BN = 16 * NG;
  static constexpr bool kTail = MT == 8 && NG == 8;  // the shape that runs tail K slices
  static constexpr int CROW = BN * 2 + 16;  // bf16 staging row, padded by 16 bytes
  static constexpr int SMEM = BM * CROW;
};

// Ap: activations in the prepared layout for Mp = round_up(M, 64) rows; Wp: the prepared
// weight [N, K] (N % 64 == 0); C: bf16 [M, N]. Tiles: ceil(M / BM) x ceil(N / BN). CTAs
// 0 .. full - 1 (full = tiles - tail) own whole tiles, dealt in the XCD-aware order over the
// first `full` logical tiles; CTA full + u (u < tail * slices) computes K slice u % slices of
// logical tile full + u / slices into P[u] (BM x BN FP32, row-major). Rows >= M and columns
// >= N are computed from clamped operand blocks and never stored.
template <int MT, int NG, int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_qr(const uint8_t* __restrict__ Ap, const uint8_t* __restrict__ Wp, uint16_t* __restrict__ C,
               float* __restrict__ P, int M, int N, int K, int GM, int tail, int slices) {
  using S_ = QRShape<MT, NG>;
  extern __shared__ __align__(16) uint8_t smem[];
  const int T = steps_of(K);
  const int tiles_m = (M + S_::BM - 1) / S_::BM, tiles_n = (N + S_::BN - 1) / S_::BN;
  const int full = tiles_m * tiles_n - tail;
  int bm, bn, t0 = 0, t1 = T;
  // only the 128 x 128 form runs tail slices; without that branch the others keep their
  // accumulators in registers through the epilogue
  const bool part = QRShape<MT, NG>::kTail && (int)blockIdx.x >= full;
  if (!part) {
    tile_coords(blockIdx.x, full, tiles_m, tiles_n, GM, bm, bn);
  } else {
    const int u = blockIdx.x - full, TS = (T + slices - 1) / slices;
    logical_tile(full + u / slices, tiles_m, tiles_n, GM, bm, bn);
    t0 = min(T, (u % slices) * TS);
    t1 = min(T, t0 + TS);
  }
  const int lane = threadIdx.x;
  v4f acc[NG][MT];
  rd_steps<MT, NG, D>(acc, Ap, Wp, M, N, K, bm, bn, t0, t1, lane);

  if constexpr (S_::kTail) {
    if (part) {
      // FP32 partial tile, row-major: lane l holds rows 16 i + l % 16, columns 16 j + 4 (l / 16) + 0..3
      float* Pt = P + (size_t)(blockIdx.x - full) * S_::BM * S_::BN;
#pragma unroll
      for (int j = 0; j < NG; ++j)
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const int r = 16 * i + (lane & 15), cl = 16 * j + 4 * (lane >> 4);
          *reinterpret_cast<v4f*>(Pt + r * S_::BN + cl) = acc[j][i];
        }
      return;
    }
  }
  // epilogue: stage the bf16 tile in this wave's LDS, then store whole rows, 16 bytes a lane
#pragma unroll
  for (int j = 0; j < NG; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int r = 16 * i + (lane & 15), cl = 16 * j + 4 * (lane >> 4);
      *reinterpret_cast<uint2*>(smem + r * S_::CROW + cl * 2) =
          pack4_bf16(acc[j][i][0], acc[j][i][1], acc[j][i][2], acc[j][i][3]);
    }
  __syncthreads();
  constexpr int CPR = S_::BN / 8;  // 16-byte chunks per tile row
  const int m0 = bm * S_::BM, n0 = bn * S_::BN;
  static_assert(S_::BM * CPR % 64 == 0, "whole rounds of 64 chunks");
#pragma unroll
  for (int k = 0; k < S_::BM * CPR / 64; ++k) {
    const int id = lane + 64 * k;
    const int r = id / CPR, ch = id % CPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * S_::CROW + ch * 16);
    if (m0 + r < M && n0 + 8 * ch < N)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(C + (size_t)(m0 + r) * N + n0 + 8 * ch));
  }
}

// The tail tiles of k_gemm_qr: tile v (logical tile full + v) is the sum of P[v * slices + s]
// over s = 0 .. slices - 1 in that order, written as bf16 (rows < M, columns < N). CTA (v, c)
// of 2 BN threads takes rows 16 c .. 16 c + 15 of tile v, a thread 8 adjacent columns of one
// row; its slices are loaded eight at a time, all in flight before the first add.
template <int BM, int BN>
__global__ __launch_bounds__(2 * BN) void k_qr_tail_reduce(const float* __restrict__ P, uint16_t* __restrict__ C,
                                                           int M, int N, int GM, int full, int slices) {
  static_assert(BN % 8 == 0 && BM % 16 == 0, "16 rows of BN / 8 eight-column chunks per CTA");
  constexpr int CPR = BN / 8;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int v = blockIdx.x / (BM / 16), c = blockIdx.x % (BM / 16);
  int bm, bn;
  logical_tile(full + v, tiles_m, tiles_n, GM, bm, bn);
  const int r = 16 * c + threadIdx.x / CPR, ch = threadIdx.x % CPR;
  const int m = bm * BM + r, n = bn * BN + ch * 8;
  if (m >= M || n >= N) return;
  const float* q = P + (size_t)v * slices * BM * BN + r * BN + ch * 8;
  v4f lo = *reinterpret_cast<const v4f*>(q), hi = *reinterpret_cast<const v4f*>(q + 4);
  for (int s0 = 1; s0 < slices; s0 += 8) {
    v4f xl[8], xh[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float* qs = q + (size_t)min(s0 + u, slices - 1) * BM * BN;
      xl[u] = *reinterpret_cast<const v4f*>(qs);
      xh[u] = *reinterpret_cast<const v4f*>(qs + 4);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < slices) {
        lo += xl[u];
        hi += xh[u];
      }
  }
  const uint2 p0 = pack4_bf16(lo[0], lo[1], lo[2], lo[3]), p1 = pack4_bf16(hi[0], hi[1], hi[2], hi[3]);
  const u32x4 o = {p0.x, p0.y, p1.x, p1.y};
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(C + (size_t)m * N + n));
}

// ---------------------------------------------------------------------- k_gemm_qk
//
// The register-direct wave of k_gemm_qr, four to a CTA (one per SIMD) on the same
// 16 MT x 16 NG tile, each over its own quarter of the CTA's K range: for calls with too few
// tiles to give every SIMD one (1536 x 2048: 192 tiles of 128 x 128, one CTA per CU). The
// four partial tiles are added through LDS in wave order, 64 rows at a time (4 x 64 rows of
// FP32, rows padded by 4 floats so the 16 rows a wave's float4 store covers fall in distinct
// banks), and written once. With slices > 1 a CTA covers one of `slices` K ranges of
// its tile and writes FP32 partials P[slice][M][N], which k_splitk_reduce adds in slice order.

template <int MT, int NG>
struct QKShape {
  static constexpr int BM = 16 * MT, BN = 16 * NG;
  static constexpr int HR = 64;               // rows per reduction pass
  static constexpr int NP = BM / HR;          // passes
  static constexpr int PROW = BN + 4;         // padded FP32 row
  static constexpr int SMEM = 4 * HR * PROW * 4;
  static_assert(BM % HR == 0 && BN % 8 == 0, "a wave sums 16 rows of each pass, 8 columns a chunk");
  static_assert(SMEM <= 160 * 1024, "the four partial 64-row tiles fit the LDS");
};

template <int MT, int NG, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_qk(const uint8_t* __restrict__ Ap, const uint8_t* __restrict__ Wp, uint16_t* __restrict__ C,
               float* __restrict__ P, int M, int N, int K, int GM, int slices) {
  using S_ = QKShape<MT, NG>;
  extern __shared__ __align__(16) uint8_t smem[];
  const int T = steps_of(K);
  const int tiles_m = (M + S_::BM - 1) / S_::BM, tiles_n = (N + S_::BN - 1) / S_::BN;
  // units = (tile, slice), a tile's slices consecutive; units dealt to the XCDs as tiles are
  const int units = tiles_m * tiles_n * slices;
  const int q8 = units / 8, r8 = units % 8, x8 = blockIdx.x % 8;
  const int unit = x8 * q8 + min(x8, r8) + (int)blockIdx.x / 8;
  const int slice = unit % slices;
  int bm, bn;
  logical_tile(unit / slices, tiles_m, tiles_n, GM, bm, bn);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int TSl = (T + slices - 1) / slices;
  const int k0 = min(T, slice * TSl), k1 = min(T, k0 + TSl);
  const int TW = (k1 - k0 + 3) / 4;
  const int t0 = min(k1, k0 + w * TW), t1 = min(k1, t0 + TW);
  v4f acc[NG][MT];
  rd_steps<MT, NG, D>(acc, Ap, Wp, M, N, K, bm, bn, t0, t1, lane);

  float* red = reinterpret_cast<float*>(smem);  // [4 waves][64 rows][PROW]
  const int m0 = bm * S_::BM, n0 = bn * S_::BN;
  static_for<S_::NP>([&](auto h_c) {
    constexpr int h = decltype(h_c)::value;
    if constexpr (h > 0) __syncthreads();  // every wave has summed the previous pass
#pragma unroll
    for (int j = 0; j < NG; ++j)
#pragma unroll
      for (int i = 4 * h; i < 4 * h + 4; ++i) {
        const int r = 16 * (i - 4 * h) + (lane & 15), cl = 16 * j + 4 * (lane >> 4);
        *reinterpret_cast<v4f*>(red + (w * S_::HR + r) * S_::PROW + cl) = acc[j][i];
      }
    __syncthreads();
    // wave w adds rows 16 w .. 16 w + 15 of this pass over the four waves, 8 columns a chunk
    constexpr int CPR = S_::BN / 8;
#pragma unroll
    for (int c = 0; c < (16 * CPR + 63) / 64; ++c) {
      const int id = lane + 64 * c;
      if (16 * CPR % 64 != 0 && id >= 16 * CPR) break;
      const int r = 16 * w + id / CPR, ch = id % CPR;
      const float* q = red + r * S_::PROW + 8 * ch;
      v4f lo = *reinterpret_cast<const v4f*>(q), hi = *reinterpret_cast<const v4f*>(q + 4);
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) {
        lo += *reinterpret_cast<const v4f*>(q + ww * S_::HR * S_::PROW);
        hi += *reinterpret_cast<const v4f*>(q + ww * S_::HR * S_::PROW + 4);
      }
      const int m = m0 + h * S_::HR + r, n = n0 + 8 * ch;
      if (m < M && n < N) {
        if (slices > 1) {
          float* dst = P + ((size_t)slice * M + m) * N + n;
          *reinterpret_cast<v4f*>(dst) = lo;
          *reinterpret_cast<v4f*>(dst + 4) = hi;
        } else {
          const uint2 p0 = pack4_bf16(lo[0], lo[1], lo[2], lo[3]), p1 = pack4_bf16(hi[0], hi[1], hi[2], hi[3]);
          const u32x4 v = {p0.x, p0.y, p1.x, p1.y};
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(C + (size_t)m * N + n));
        }
      }
    }
  });
}

// ====================================================================== launchers

// Compiled configurations (WM, WN, MT, NG, NBUF, OCC): 256 x 256 as 2 x 4 waves of 128 x 64 (two
// waves per SIMD, four stages: 136 KiB of LDS); 128 x 128 as 2 x 2 waves of 64 x 64 with four
// or five stages (two CTAs per CU with four).
#define MX_QO_CONFIGS(X) X(2, 4, 8, 4, 4, 2) X(2, 2, 4, 4, 4, 2) X(2, 2, 4, 4, 5, 2) X(1, 4, 8, 4, 3, 2)

std::atomic<uint64_t> g_qo_lds[8];

// Allow `bytes` of dynamic LDS for a kernel (once per device; `done` holds a bit per device
// already configured).
hipError_t ensure_dynamic_lds(const void* kern, int bytes, std::atomic<uint64_t>& done) {
  if (bytes <= 65536) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

template <int WM, int WN, int MT, int NG, int NBUF, int OCC>
hipError_t run_qo(int id, const void* ap, const void* wp, void* c, int M, int N, int K, int GM, hipStream_t st) {
  using S = QOShape<WM, WN, MT, NG, NBUF>;
  auto kern = k_gemm_qo<WM, WN, MT, NG, NBUF, OCC>;
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), S::SMEM, g_qo_lds[id]);
  if (e != hipSuccess) return e;
  const int64_t grid = (int64_t)((M + S::BM - 1) / S::BM) * ((N + S::BN - 1) / S::BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(S::NTH), S::SMEM, st, static_cast<const uint8_t*>(ap),
                     static_cast<const uint8_t*>(wp), static_cast<uint16_t*>(c), M, N, K, GM);
  return hipGetLastError();
}

// Register-direct configurations (MT, NG, D): 128 x 128 tiles two steps ahead; 128 x 144
// (72 accumulators, the ninth row of 16 columns in VGPRs) one step ahead, since two steps of
// its operands leave too few registers for the rest. Measured at 8448 x 7168 M=2048: 128 x 144
// two steps ahead 77.6 against 75.3 us one step ahead; 128 x 160 (80 accumulators) 114.9 us.
#define MX_QR_CONFIGS(X) X(8, 8, 2) X(8, 9, 1) X(9, 8, 1)

template <int MT, int NG, int D>
hipError_t run_qr(const void* ap, const void* wp, void* c, float* P, int M, int N, int K, int GM, int tail,
                  int slices, hipStream_t st) {
  using S = QRShape<MT, NG>;
  const int64_t tiles = (int64_t)((M + S::BM - 1) / S::BM) * ((N + S::BN - 1) / S::BN);
  const int64_t grid = tiles - tail + (int64_t)tail * slices;
  hipLaunchKernelGGL((k_gemm_qr<MT, NG, D>), dim3((unsigned)grid), dim3(64), S::SMEM, st,
                     static_cast<const uint8_t*>(ap), static_cast<const uint8_t*>(wp), static_cast<uint16_t*>(c), P,
                     M, N, K, GM, tail, slices);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || tail == 0) return e;
  hipLaunchKernelGGL((k_qr_tail_reduce<S::BM, S::BN>), dim3((unsigned)(tail * (S::BM / 16))), dim3(2 * S::BN), 0, st,
                     static_cast<const float*>(P), static_cast<uint16_t*>(c), M, N, GM, (int)(tiles - tail), slices);
  return hipGetLastError();
}

// Four-wave configurations (MT, NG, D): tiles 128 x 96 .. 128 x 144 (the widest holds its four
// partial 64-row tiles in 148 KiB of LDS), and 128 x 48 four steps ahead for a single row tile.
#define MX_QK_CONFIGS(X) X(8, 8, 2) X(8, 9, 1) X(8, 7, 2) X(8, 6, 2) X(8, 3, 4)

std::atomic<uint64_t> g_qk_lds[8];

template <int MT, int NG, int D>
hipError_t run_qk(int id, const void* ap, const void* wp, void* c, float* P, int M, int N, int K, int GM, int slices,
                  hipStream_t st) {
  using S = QKShape<MT, NG>;
  auto kern = k_gemm_qk<MT, NG, D>;
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), S::SMEM, g_qk_lds[id]);
  if (e != hipSuccess) return e;
  const int64_t grid = (int64_t)((M + S::BM - 1) / S::BM) * ((N + S::BN - 1) / S::BN) * slices;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), S::SMEM, st, static_cast<const uint8_t*>(ap),
                     static_cast<const uint8_t*>(wp), static_cast<uint16_t*>(c), P, M, N, K, GM, slices);
  e = hipGetLastError();
  if (e != hipSuccess || slices == 1) return e;
  return launch_splitk_reduce(P, c, M, N, slices, st);
}

}  // namespace

bool qk_supported(int MT, int NG, int D) {
#define X(mt, ng, d) if (MT == mt && NG == ng && D == d) return true;
  MX_QK_CONFIGS(X)
#undef X
  return false;
}

// Workspace: the prepared activations, then (256-byte aligned) the FP32 partials of `slices`
// K slices when there are several.
size_t qk_workspace_bytes(int64_t M, int64_t N, int64_t K, int slices) {
  const size_t act = (qo_act_bytes(M, K) + 255) / 256 * 256;
  return slices > 1 ? act + (size_t)slices * M * N * 4 : act;
}

hipError_t launch_gemm_qk(int MT, int NG, int D, int slices, const void* a, const void* wp, void* c, int64_t M,
                          int64_t N, int64_t K, int GM, void* ws, hipStream_t st) {
  if (!qk_supported(MT, NG, D) || N % 64 != 0 || slices < 1 || 4 * slices > steps_of((int)K))
    return hipErrorInvalidValue;
  const int64_t Mp = (M + 63) / 64 * 64;
  float* P = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + (qo_act_bytes(M, K) + 255) / 256 * 256);
  hipError_t e = launch_prepare_rows(a, M, Mp, K, ws, st);
  if (e != hipSuccess) return e;
  int id = 0;
#define X(mt, ng, d)                                                                                   \
  if (MT == mt && NG == ng && D == d)                                                                  \
    return run_qk<mt, ng, d>(id, ws, wp, c, P, (int)M, (int)N, (int)K, GM, slices, st);               \
  ++id;
  MX_QK_CONFIGS(X)
#undef X
  return hipErrorInvalidValue;
}

bool qr_supported(int MT, int NG, int D) {
#define X(mt, ng, d) if (MT == mt && NG == ng && D == d) return true;
  MX_QR_CONFIGS(X)
#undef X
  return false;
}

// Tail tiles split into K slices: the tiles beyond one wave per SIMD of the chip (256 CUs x
// 4), when they are at most a quarter round; none otherwise.
int qr_tail_tiles(int64_t M, int64_t N, int MT, int NG) {
  const int64_t tiles = (M + 16 * MT - 1) / (16 * MT) * ((N + 16 * NG - 1) / (16 * NG));
  constexpr int64_t kSlots = 256 * 4;
  return tiles > kSlots && tiles <= kSlots + kSlots / 4 ? (int)(tiles - kSlots) : 0;
}

size_t qr_workspace_bytes(int64_t M, int64_t N, int64_t K, int MT, int NG, int slices) {
  const size_t act = (qo_act_bytes(M, K) + 255) / 256 * 256;
  return act + (size_t)qr_tail_tiles(M, N, MT, NG) * slices * (16 * MT) * (16 * NG) * 4;
}

hipError_t launch_gemm_qr(int MT, int NG, int D, int slices, const void* a, const void* wp, void* c, int64_t M,
                          int64_t N, int64_t K, int GM, void* ws, hipStream_t st) {
  if (!qr_supported(MT, NG, D) || N % 64 != 0 || slices < 1) return hipErrorInvalidValue;
  const int64_t Mp = (M + 63) / 64 * 64;
  const int tail = slices > 1 ? qr_tail_tiles(M, N, MT, NG) : 0;
  if (tail > 0 && !(MT == 8 && NG == 8)) return hipErrorInvalidValue;  // only 128 x 128 runs tail slices
  float* P = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + (qo_act_bytes(M, K) + 255) / 256 * 256);
  hipError_t e = launch_prepare_rows(a, M, Mp, K, ws, st);
  if (e != hipSuccess) return e;
#define X(mt, ng, d)                                                                                     \
  if (MT == mt && NG == ng && D == d)                                                                    \
    return run_qr<mt, ng, d>(ws, wp, c, P, (int)M, (int)N, (int)K, GM, tail, slices, st);
  MX_QR_CONFIGS(X)
#undef X
  return hipErrorInvalidValue;
}

size_t qo_act_bytes(int64_t M, int64_t K) {
  const int64_t Mp = (M + 63) / 64 * 64;
  return prepared_bytes(Mp, K);
}

bool qo_supported(int WM, int WN, int MT, int NG, int NBUF, int OCC) {
#define X(wm, wn, mt, ng, nb, occ) \
  if (WM == wm && WN == wn && MT == mt && NG == ng && NBUF == nb && OCC == occ) return true;
  MX_QO_CONFIGS(X)
#undef X
  return false;
}

hipError_t launch_gemm_qo(int WM, int WN, int MT, int NG, int NBUF, int OCC, const void* a, const void* wp, void* c,
                          int64_t M, int64_t N, int64_t K, int GM, void* ws, hipStream_t st) {
  if (!qo_supported(WM, WN, MT, NG, NBUF, OCC)) return hipErrorInvalidValue;
  const int64_t Mp = (M + 63) / 64 * 64;
  hipError_t e = launch_prepare_rows(a, M, Mp, K, ws, st);
  if (e != hipSuccess) return e;
  int id = 0;
#define X(wm, wn, mt, ng, nb, occ)                                                               \
  if (WM == wm && WN == wn && MT == mt && NG == ng && NBUF == nb && OCC == occ)                  \
    return run_qo<wm, wn, mt, ng, nb, occ>(id, ws, wp, c, (int)M, (int)N, (int)K, GM, st);       \
  ++id;
  MX_QO_CONFIGS(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace mx
