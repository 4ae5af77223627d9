// mx_a16w4.hip - the A16WFP4 variant: bf16 activations, unquantized, times the prepared
// MXFP4 weight decoded to bf16, on the gfx950 bf16 MFMA (16x16x32), FP32 accumulation,
// bf16 output ("[gfx950][FlyDSL] Add direct dense A4W4 MXFP4 GEMM", CI Guide, names the
// variant as outside that change; the weight is the same prepared blob).
//
// Two forms: a weight-streaming kernel for decode M (at most 32 rows, below) and a tiled
// kernel for larger M. Tile: BM = 64 rows x BN = 64, 128 or 256 columns, four waves side by
// side along N, each 64 rows x BN / 64 column groups of 16 (four 16-row tiles each). Per
// 128-wide K step the CTA's bf16 activation tile (64 x 128, 16 KiB) goes to LDS, double
// buffered, its 16-byte chunks XOR-swizzled by row so the operand reads are conflict-free;
// each wave loads its weight operands (1 KiB per column group, as for the A4W4 kernels) and
// scale word straight into registers and decodes them with v_cvt_scalef32_pk_bf16_fp4. Both
// operands are loaded two steps ahead.
//
// K order inside a step: MFMA j (0..3) takes, from lane quarter q, the step's elements
// 32q + 8j .. 32q + 8j + 7 for both operands (a common permutation of k leaves every sum
// unchanged), so the 32 codes a lane loads for its column and 32-block are already in
// operand position: sub-chunk j of the block is bytes 4j .. 4j+3.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <utility>

#include "mx_device.h"
#include "mx_internal.h"

namespace mx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr int kA16BM = 64, kA16Threads = 256;
constexpr int kA16Row = 256;                                   // bytes of one staged activation row (128 bf16)
constexpr int kA16Stage = 2 * kA16BM * kA16Row;                // double-buffered activation tile

__device__ __forceinline__ int a16_chunk(int row, int chunk) { return chunk ^ (row & 15); }

// Tile BM = 64 x BN = 64 NGW: four waves side by side along N, each 64 rows x NGW column
// groups. Both operands run D steps ahead in registers: step t's activation block of each
// thread and each wave's weight operands and scale word sit in slot t % D, refilled with step
// t + D once the step has used them (the activations once stored to LDS).
template <int NGW, int D>
__global__ __launch_bounds__(kA16Threads, 2) void k_gemm_a16w4(const uint16_t* __restrict__ A,
                                                               const uint8_t* __restrict__ Wp,
                                                               uint16_t* __restrict__ C, int M, int N, int K) {
  constexpr int BN = 64 * NGW, CROW = BN * 2 + 16;
  constexpr int SMEM = kA16Stage > kA16BM * CROW ? kA16Stage : kA16BM * CROW;
  __shared__ __align__(16) uint8_t smem[SMEM];
  const int T = K / kStepK, G = N / 16;
  const int tiles_m = (M + kA16BM - 1) / kA16BM, tiles_n = N / BN;
  int bm, bn;
  tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, 8, bm, bn);
  const int m0 = bm * kA16BM, Mrows = min(kA16BM, M - m0);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gw0 = bn * (BN / 16) + w * NGW;                    // first of this wave's column groups
  const uint8_t* __restrict__ Wsc = Wp + payload_bytes(N, K);

  // activation loads: thread -> row tid/4 (clamped into the valid rows), 32-block tid%4
  const int ar = tid >> 2, ab = tid & 3;
  const uint16_t* arow = A + (size_t)(m0 + min(ar, Mrows - 1)) * K + ab * kBlock;
  const uint8_t* wb[NGW];
#pragma unroll
  for (int g = 0; g < NGW; ++g) wb[g] = Wp + (size_t)min(gw0 + g, G - 1) * T * 1024 + lane * 16;
  // the scale word of this wave's groups' quad, and the byte of its first group in it
  const uint8_t* sb = Wsc + (size_t)min(gw0 >> 2, G / 4 - 1) * T * 256 + lane * 4;
  const int sh0 = 8 * (gw0 & 3);

  uint32_t xa[D][16];
  uint4 wq[D][NGW];
  uint32_t ws[D];
  auto load = [&](int t, auto slot_c) {  // t past the end: the last step again, never used
    constexpr int SL = decltype(slot_c)::value;
    const int tt = min(t, T - 1);
    load_block(arow + (size_t)tt * kStepK, xa[SL]);
#pragma unroll
    for (int g = 0; g < NGW; ++g) wq[SL][g] = *reinterpret_cast<const uint4*>(wb[g] + (size_t)tt * 1024);
    ws[SL] = *reinterpret_cast<const uint32_t*>(sb + (size_t)tt * 256);
  };
  auto sa = [&](int buf, int row, int chunk) { return smem + buf * kA16BM * kA16Row + row * kA16Row + 16 * a16_chunk(row, chunk); };

  v4f acc[NGW][4];
#pragma unroll
  for (int g = 0; g < NGW; ++g)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[g][mt] = v4f{0.f, 0.f, 0.f, 0.f};

  // step t, its operands in slot SL = t % D
  auto step = [&](int t, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
    const int buf = t & 1;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<uint4*>(sa(buf, ar, 4 * ab + c)) =
          make_uint4(xa[SL][4 * c], xa[SL][4 * c + 1], xa[SL][4 * c + 2], xa[SL][4 * c + 3]);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 bop[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        bop[mt] = *reinterpret_cast<const uint4*>(sa(buf, 16 * mt + (lane & 15), 4 * (lane >> 4) + j));
#pragma unroll
      for (int g = 0; g < NGW; ++g) {
        const uint32_t s = (ws[SL] >> (sh0 + 8 * g)) & 0xffu;
        const float sc = __builtin_bit_cast(float, s ? (s << 23) : 0x00400000u);
        const uint32_t codes = j == 0 ? wq[SL][g].x : j == 1 ? wq[SL][g].y : j == 2 ? wq[SL][g].z : wq[SL][g].w;
        uint32_t d[4];
        d[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0));
        d[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1));
        d[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2));
        d[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3));
        const bf16x8 aop = __builtin_bit_cast(bf16x8, make_uint4(d[0], d[1], d[2], d[3]));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[g][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, __builtin_bit_cast(bf16x8, bop[mt]), acc[g][mt],
                                                               0, 0, 0);
      }
    }
    load(t + D, std::integral_constant<int, SL>{});  // the slot is free: refill it with step t + D
    __syncthreads();  // the buffer written two steps on is free only once every wave has read it
  };

  static_for<D>([&](auto u_c) { load(decltype(u_c)::value, u_c); });
  int t = 0;
  for (; t + D <= T; t += D) static_for<D>([&](auto u_c) { step(t + decltype(u_c)::value, u_c); });
  static_for<D>([&](auto u_c) {
    if (t + decltype(u_c)::value < T) step(t + decltype(u_c)::value, u_c);
  });

  // Epilogue: lane l holds C[m = 16 mt + l % 16][n = 16 g + 4 (l / 16) .. + 3] of its wave's
  // columns; stage the tile as bf16 in LDS, then write whole rows 16 bytes per lane.
#pragma unroll
  for (int g = 0; g < NGW; ++g)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int r = 16 * mt + (lane & 15), cl = 16 * (w * NGW + g) + 4 * (lane >> 4);
      *reinterpret_cast<uint2*>(smem + r * CROW + cl * 2) =
          pack4_bf16(acc[g][mt][0], acc[g][mt][1], acc[g][mt][2], acc[g][mt][3]);
    }
  __syncthreads();
  const int n0 = bn * BN;
  static_assert(kA16BM * (BN / 8) % kA16Threads == 0, "every thread stores the same number of chunks");
#pragma unroll
  for (int i = 0; i < kA16BM * (BN / 8) / kA16Threads; ++i) {
    const int id = tid + i * kA16Threads;
    const int r = id / (BN / 8), ch = id % (BN / 8);
    if (r < Mrows) {
      const uint4 v = *reinterpret_cast<const uint4*>(smem + r * CROW + ch * 16);
      *reinterpret_cast<uint4*>(C + (size_t)(m0 + r) * N + n0 + 8 * ch) = v;
    }
  }
}

// Decode-M form (M <= 32): MT 16-row MFMA tiles. A CTA owns 16 NG columns over all of K;
// its WK waves split the K steps. Each wave issues the weight loads of up to PD steps at
// once (1 KiB per column group and step, the A4W4 layout, plus one scale byte per lane and
// group), then the matching activation loads, which go from global memory straight into
// MFMA operands: lane l reads, for row tile mt, the 64 bytes of row 16 mt + l % 16
// (clamped to the last row, never stored) and 32-block l / 16, which are its operands of
// the four 16x16x32 MFMAs of the step under the k order above; each decoded weight operand
// serves all MT row tiles. No LDS staging, no barrier in the K loop; the wave partial sums
// meet in LDS in a fixed wave order.
template <int MT, int NG, int WK, int PD>
__global__ __launch_bounds__(64 * WK) void k_gemm_a16w4_stream(const uint16_t* __restrict__ A,
                                                               const uint8_t* __restrict__ Wp,
                                                               uint16_t* __restrict__ C, int M, int N, int K) {
  __shared__ __align__(16) v4f red[WK > 1 ? WK * NG * MT * 64 : 1];
  const int T = K / kStepK;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g0 = blockIdx.x * NG;
  const int per = (T + WK - 1) / WK, t0 = min(T, w * per), t1 = min(T, t0 + per);
  const uint8_t* __restrict__ Wsc = Wp + payload_bytes(N, K);
  const uint8_t* arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    arow[mt] = reinterpret_cast<const uint8_t*>(A + (size_t)min(16 * mt + (lane & 15), M - 1) * K) +
               (lane >> 4) * (kBlock * 2);

  v4f acc[NG][MT];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[g][mt] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int tb = t0; tb < t1; tb += PD) {
    uint4 wq[PD][NG];
    uint32_t wsb[PD][NG];
    uint32_t xa[PD][MT][16];
    // branch-free: steps past the wave's range re-load its last step and are never used
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      const int t = min(tb + i, t1 - 1);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        wq[i][g] = load16_nt(Wp + wp_payload_off(g0 + g, t, lane, T));
        wsb[i][g] = __builtin_nontemporal_load(Wsc + wp_scale_off((g0 + g) >> 2, t, lane, T) + ((g0 + g) & 3));
      }
    }
#pragma unroll
    for (int i = 0; i < PD; ++i)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        load_block_at(arow[mt], (uint32_t)(min(tb + i, t1 - 1) * kStepK * 2), xa[i][mt]);
    __builtin_amdgcn_sched_barrier(0);  // every load of the chunk ahead of its first use
    const int nh = min(PD, t1 - tb);
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      if (i < nh) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const uint32_t s = wsb[i][g];
          const float sc = __builtin_bit_cast(float, s ? (s << 23) : 0x00400000u);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t codes = j == 0 ? wq[i][g].x : j == 1 ? wq[i][g].y : j == 2 ? wq[i][g].z : wq[i][g].w;
            uint32_t d[4];
            d[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0));
            d[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1));
            d[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2));
            d[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3));
            const bf16x8 aop = __builtin_bit_cast(bf16x8, make_uint4(d[0], d[1], d[2], d[3]));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const bf16x8 bop = __builtin_bit_cast(
                  bf16x8, make_uint4(xa[i][mt][4 * j], xa[i][mt][4 * j + 1], xa[i][mt][4 * j + 2], xa[i][mt][4 * j + 3]));
              acc[g][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop, acc[g][mt], 0, 0, 0);
            }
          }
        }
      }
    }
  }
  // lane l holds C[m = 16 mt + l % 16][n = 16 (g0 + g) + 4 (l / 16) .. + 3]
  auto store = [&](int g, int mt, const v4f& v) {
    const int m = 16 * mt + (lane & 15);
    if (m < M)
      *reinterpret_cast<uint2*>(C + (size_t)m * N + 16 * (g0 + g) + 4 * (lane >> 4)) = pack4_bf16(v[0], v[1], v[2], v[3]);
  };
  if constexpr (WK == 1) {
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) store(g, mt, acc[g][mt]);
  } else {
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) red[((w * NG + g) * MT + mt) * 64 + lane] = acc[g][mt];
    __syncthreads();
    for (int p = w; p < NG * MT; p += WK) {
      v4f sum = red[p * 64 + lane];
      for (int ww = 1; ww < WK; ++ww) sum += red[(ww * NG * MT + p) * 64 + lane];
      store(p / MT, p % MT, sum);
    }
  }
}

// Decode-M choice: one 16-row tile up to 16 rows, two up to 32; one column group per CTA
// when there are at least 512 of them, else two; eight waves per CTA for long K (16 steps
// or more), else four; a wave's whole K share in registers in chunks of PD = 2, 4 or 8 steps
// (at most 4 with two row tiles).
struct A16StreamCfg {
  int MT, NG, WK, PD;
};
A16StreamCfg a16_stream_cfg(int64_t M, int64_t N, int64_t K) {
  const int G = (int)(N / 16), T = (int)(K / kStepK);
  A16StreamCfg c{M > 16 ? 2 : 1, G >= 512 ? 1 : 2, T >= 16 ? 8 : 4, 2};
  const int per = (T + c.WK - 1) / c.WK, cap = c.MT == 2 ? 4 : 8;
  while (c.PD < per && c.PD < cap) c.PD *= 2;
  return c;
}

template <int MT, int NG, int WK>
hipError_t run_a16_stream(int PD, const void* a, const void* wp, void* c, int M, int N, int K, hipStream_t st) {
  const dim3 grid((unsigned)(N / (16 * NG))), block(64 * WK);
  const auto* A = static_cast<const uint16_t*>(a);
  const auto* W = static_cast<const uint8_t*>(wp);
  auto* C = static_cast<uint16_t*>(c);
  if (PD == 2) hipLaunchKernelGGL((k_gemm_a16w4_stream<MT, NG, WK, 2>), grid, block, 0, st, A, W, C, M, N, K);
  else if (PD == 4) hipLaunchKernelGGL((k_gemm_a16w4_stream<MT, NG, WK, 4>), grid, block, 0, st, A, W, C, M, N, K);
  else if constexpr (MT == 1) hipLaunchKernelGGL((k_gemm_a16w4_stream<MT, NG, WK, 8>), grid, block, 0, st, A, W, C, M, N, K);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int MT>
hipError_t run_a16_stream_mt(const A16StreamCfg& cfg, const void* a, const void* wp, void* c, int M, int N, int K,
                             hipStream_t st) {
  if (cfg.NG == 1)
    return cfg.WK == 8 ? run_a16_stream<MT, 1, 8>(cfg.PD, a, wp, c, M, N, K, st)
                       : run_a16_stream<MT, 1, 4>(cfg.PD, a, wp, c, M, N, K, st);
  return cfg.WK == 8 ? run_a16_stream<MT, 2, 8>(cfg.PD, a, wp, c, M, N, K, st)
                     : run_a16_stream<MT, 2, 4>(cfg.PD, a, wp, c, M, N, K, st);
}

constexpr int64_t kA16StreamMaxM = 32;

// Compiled tiled forms (NGW, D).
#define MX_A16_TILE_CONFIGS(X) X(4, 2) X(2, 2) X(1, 2)

struct A16TileCfg {
  int NGW, D;
};
// Tiled form: the widest tile (64 x 256, 64 x 128 or 64 x 64) that still gives about 200 CTAs
// or more (N = 7168, K = 768: 64 x 64 at M = 128, 6.7 us against 10.8 us for 64 x 256 tiles;
// 64 x 256 from M = 449 on), loads two steps ahead (three or more measured no faster).
// Tuning only: MX_A16W4_CONFIG="NGW,D" replaces the choice (a pair not compiled fails the call).
bool a16_tile_cfg(int64_t M, int64_t N, A16TileCfg& c) {
  const int64_t tm = (M + kA16BM - 1) / kA16BM;
  c.NGW = tm * (N / 256) >= 200 ? 4 : tm * (N / 128) >= 200 ? 2 : 1;
  c.D = 2;
  const char* e = std::getenv("MX_A16W4_CONFIG");
  if (e && *e) {
    if (std::sscanf(e, "%d,%d", &c.NGW, &c.D) != 2) return false;
    bool ok = false;
#define X(ngw, d) ok = ok || (c.NGW == ngw && c.D == d);
    MX_A16_TILE_CONFIGS(X)
#undef X
    return ok;
  }
  return true;
}

}  // namespace

bool a16w4_plan(int64_t M, int64_t N, int64_t K, char* buf, size_t len) {
  if (M <= 0) {
    std::snprintf(buf, len, "none");
  } else if (M <= kA16StreamMaxM) {
    const A16StreamCfg c = a16_stream_cfg(M, N, K);
    std::snprintf(buf, len, "k_gemm_a16w4_stream<%d, %d, %d, %d>", c.MT, c.NG, c.WK, c.PD);
  } else {
    A16TileCfg c;
    if (!a16_tile_cfg(M, N, c)) return false;
    std::snprintf(buf, len, "k_gemm_a16w4<%d, %d> (64 x %d tiles)", c.NGW, c.D, 64 * c.NGW);
  }
  return true;
}

hipError_t launch_a16w4(const void* a, const void* wp, void* c, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (M <= kA16StreamMaxM) {
    const A16StreamCfg cfg = a16_stream_cfg(M, N, K);
    return cfg.MT == 2 ? run_a16_stream_mt<2>(cfg, a, wp, c, (int)M, (int)N, (int)K, st)
                       : run_a16_stream_mt<1>(cfg, a, wp, c, (int)M, (int)N, (int)K, st);
  }
  A16TileCfg cfg;
  if (!a16_tile_cfg(M, N, cfg)) return hipErrorInvalidValue;
  const int64_t tiles = ((M + kA16BM - 1) / kA16BM) * (N / (64 * cfg.NGW));
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  const auto* A = static_cast<const uint16_t*>(a);
  const auto* W = static_cast<const uint8_t*>(wp);
  auto* C = static_cast<uint16_t*>(c);
  const dim3 grid((unsigned)tiles), block(kA16Threads);
#define X(ngw, d)                                                                                        \
  if (cfg.NGW == ngw && cfg.D == d) {                                                                    \
    hipLaunchKernelGGL((k_gemm_a16w4<ngw, d>), grid, block, 0, st, A, W, C, (int)M, (int)N, (int)K);     \
    return hipGetLastError();                                                                            \
  }
  MX_A16_TILE_CONFIGS(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace mx
