// mx_kernels.hip - gfx950 kernels of the inline-quantized A4W4 MXFP4 GEMM and their
// launchers.
//
// Operation: "[gfx950][FlyDSL] Add direct dense A4W4 MXFP4 GEMM", Summary (BF16 activation
// -> inline MXFP4 quant -> MXFP4 x MXFP4 scaled MFMA) and Implementation (one-time weight
// preshuffle, direct BF16 output, small-M and large-M tiles, BK=128 steps, M-tail masking).
//
// MFMA orientation: the weight is the MFMA "A" operand (16 output columns n as rows) and
// the quantized activations are the "B" operand (16 output rows m as columns), so lane l's
// accumulator element r is C[m = l % 16][n = 4 * (l / 16) + r]: four consecutive columns of
// one output row, stored as one 8-byte write.
#include <atomic>

#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

// ====================================================================== standalone quant

// One thread per 32-block. Row-major A with K % 32 == 0 makes block b start at element
// 32b, its payload at byte 16b and its scale at byte b of the canonical outputs.
__global__ __launch_bounds__(256) void k_quant_act(const uint16_t* __restrict__ A,
                                                    uint8_t* __restrict__ q,
                                                    uint8_t* __restrict__ s, int64_t nblocks) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  uint32_t x[16];
  load_block(A + b * kBlock, x);
  uint32_t qq[4];
  const uint32_t sc = quant_block(x, qq);
  reinterpret_cast<uint4*>(q)[b] = make_uint4(qq[0], qq[1], qq[2], qq[3]);
  s[b] = (uint8_t)sc;
}

// ====================================================================== weight prepare

// One thread per (column group g, step quad t4, lane): quantizes the up to four 32-blocks
// that lane owns in steps 4t4..4t4+3 and writes them and their scale word in place.
__global__ __launch_bounds__(256) void k_prepare(const uint16_t* __restrict__ W,
                                                  uint8_t* __restrict__ Wp, int N, int K) {
  const int T = steps_of(K), T4 = quads_of(K), G = N / 16;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)G * T4 * 64) return;
  const int lane = (int)(idx % 64);
  const int64_t r = idx / 64;
  const int t4 = (int)(r % T4), g = (int)(r / T4);
  const int n = 16 * g + (lane & 15);
  uint32_t sword = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = 4 * t4 + j;
    if (t < T) {
      const int kb = 4 * t + (lane >> 4);
      uint32_t x[16];
      load_block(W + (size_t)n * K + (size_t)kb * kBlock, x);
      uint32_t qq[4];
      const uint32_t sc = quant_block(x, qq);
      *reinterpret_cast<uint4*>(Wp + wp_payload_off(g, t, lane, T)) = make_uint4(qq[0], qq[1], qq[2], qq[3]);
      sword |= sc << (8 * j);
    }
  }
  *reinterpret_cast<uint32_t*>(Wp + payload_bytes(N, K) + wp_scale_off(g, t4, lane, T4)) = sword;
}

// Inverse of the preshuffle: canonical payload [N, K/2] and scales [N, K/32].
__global__ __launch_bounds__(256) void k_unprepare(const uint8_t* __restrict__ Wp,
                                                    uint8_t* __restrict__ q,
                                                    uint8_t* __restrict__ s, int N, int K) {
  const int T = steps_of(K), T4 = quads_of(K), G = N / 16, KB = K / kBlock;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)G * T * 64) return;
  const int lane = (int)(idx % 64);
  const int64_t r = idx / 64;
  const int t = (int)(r % T), g = (int)(r / T);
  const int n = 16 * g + (lane & 15), kb = 4 * t + (lane >> 4);
  const uint4 v = *reinterpret_cast<const uint4*>(Wp + wp_payload_off(g, t, lane, T));
  *reinterpret_cast<uint4*>(q + (size_t)n * (K / 2) + (size_t)kb * 16) = v;
  const uint32_t sword =
      *reinterpret_cast<const uint32_t*>(Wp + payload_bytes(N, K) + wp_scale_off(g, t >> 2, lane, T4));
  s[(size_t)n * KB + kb] = (uint8_t)(sword >> (8 * (t & 3)));
}

// ====================================================================== small-M GEMM
//
// For decode-sized M (<= 16 * MT). A CTA owns NG column groups (16 * NG output columns)
// and the whole K range; its WK waves split the K steps, each wave streaming its share of
// the prepared weight straight from HBM into registers (no reuse, so no LDS staging), while
// its own activation blocks are quantized once into LDS. The wave partial sums are added in
// LDS in a fixed wave order (deterministic), then rounded to bf16 and stored for rows < M.
//
// LDS: quantized activations [M][K/2 + 16] (the 16-byte pad staggers rows across banks),
// then their scales [M][K/32]; reused for the cross-wave reduction.
template <int MT, int NG, int WK, int PD>
__global__ __launch_bounds__(64 * WK) void k_gemm_skinny(const uint16_t* __restrict__ A,
                                                         const uint8_t* __restrict__ Wp,
                                                         uint16_t* __restrict__ C, int M, int N,
                                                         int K) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int T = steps_of(K), T4 = quads_of(K), KB = K / kBlock;
  const int RS = K / 2 + 16;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g0 = blockIdx.x * NG;
  const uint8_t* __restrict__ Wsc = Wp + payload_bytes(N, K);
  uint8_t* aq = smem;
  uint8_t* as = smem + (size_t)M * RS;

  const int per = (T + WK - 1) / WK;
  const int t0 = min(T, w * per), t1 = min(T, t0 + per);
  const int S = t1 - t0;

  uint4 wq[PD][NG];
  uint32_t wsb[PD][NG];
  auto load_chunk = [&](int tb) {
    const int nh = min(PD, t1 - tb);
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      if (i < nh) {
        const int t = tb + i;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          wq[i][g] = load16_nt(Wp + wp_payload_off(g0 + g, t, lane, T));
          wsb[i][g] = __builtin_nontemporal_load(Wsc + wp_scale_off(g0 + g, t >> 2, lane, T4) + (t & 3));
        }
      }
    }
  };

  if (S > 0) load_chunk(t0);

  // Quantize this wave's activation blocks (rows < M, blocks 4*t0 .. 4*t1-1) into LDS.
  {
    const int nbw = 4 * S;
    const int nb = M * nbw;
    for (int b = lane; b < nb; b += 64) {
      const int m = b / nbw, kb = 4 * t0 + b % nbw;
      uint32_t x[16];
      load_block(A + (size_t)m * K + (size_t)kb * kBlock, x);
      uint32_t q[4];
      const uint32_t s = quant_block(x, q);
      *reinterpret_cast<uint4*>(aq + (size_t)m * RS + kb * 16) = make_uint4(q[0], q[1], q[2], q[3]);
      as[(size_t)m * KB + kb] = (uint8_t)s;
    }
  }
  __syncthreads();

  v4f acc[NG][MT];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[g][mt] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int tb = t0; tb < t1; tb += PD) {
    const int nh = min(PD, t1 - tb);
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      if (i < nh) {
        const int t = tb + i;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = 16 * mt + (lane & 15);
          const int kb = 4 * t + (lane >> 4);
          uint4 b = make_uint4(0u, 0u, 0u, 0u);
          uint32_t sb = 0u;
          if (m < M) {
            b = *reinterpret_cast<const uint4*>(aq + (size_t)m * RS + kb * 16);
            sb = as[(size_t)m * KB + kb];
          }
#pragma unroll
          for (int g = 0; g < NG; ++g) acc[g][mt] = mfma_fp4(wq[i][g], b, acc[g][mt], wsb[i][g], sb);
        }
      }
    }
    if (tb + PD < t1) load_chunk(tb + PD);
  }

  auto store = [&](int g, int mt, const v4f& v) {
    const int m = 16 * mt + (lane & 15);
    const int n = 16 * (g0 + g) + 4 * (lane >> 4);
    if (m < M) *reinterpret_cast<uint2*>(C + (size_t)m * N + n) = pack4_bf16(v[0], v[1], v[2], v[3]);
  };

  if constexpr (WK == 1) {
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) store(g, mt, acc[g][mt]);
  } else {
    __syncthreads();  // every wave is done with the activation region
    v4f* red = reinterpret_cast<v4f*>(smem);  // [WK][NG*MT][64]
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) red[(w * NG * MT + g * MT + mt) * 64 + lane] = acc[g][mt];
    __syncthreads();
    for (int p = w; p < NG * MT; p += WK) {
      v4f sum = red[p * 64 + lane];
      for (int ww = 1; ww < WK; ++ww) sum += red[(ww * NG * MT + p) * 64 + lane];
      store(p / MT, p % MT, sum);
    }
  }
}

// ====================================================================== tiled GEMM
//
// For larger M. A CTA owns a BM x BN output tile (BM = 16 * MT rows, BN = 16 * NG * WN
// columns); its WN waves split the columns. Each 128-wide K step: every thread loads and
// quantizes its share of the BM x 128 activation tile (one 32-block per thread at BM=64),
// writing operand-ordered payload and scales into one of two LDS buffers; each wave loads
// its NG weight operands straight from global memory (a contiguous 1 KiB per operand) one
// step ahead, then reads MT activation operands from LDS and issues NG * MT MFMAs.
template <int MT, int NG, int WN>
__global__ __launch_bounds__(64 * WN) void k_gemm_tile(const uint16_t* __restrict__ A,
                                                       const uint8_t* __restrict__ Wp,
                                                       uint16_t* __restrict__ C, int M, int N,
                                                       int K) {
  constexpr int BM = 16 * MT, BN = 16 * NG * WN, NTH = 64 * WN;
  constexpr int NBLK = 4 * BM;
  constexpr int BPT = (NBLK + NTH - 1) / NTH;
  __shared__ __align__(16) uint8_t sq[2][MT * 64 * 16];
  __shared__ __align__(16) uint8_t ss[2][MT * 64];

  const int T = steps_of(K), T4 = quads_of(K);
  const int n_tiles = N / BN;
  const int bm = blockIdx.x / n_tiles, bn = blockIdx.x % n_tiles;
  const int m0 = bm * BM;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int gw0 = (bn * BN) / 16 + w * NG;
  const uint8_t* __restrict__ Wsc = Wp + payload_bytes(N, K);

  uint32_t areg[BPT][16];
  auto load_a = [&](int t) {
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int b = threadIdx.x + i * NTH;
      if (b < NBLK) {
        const int m = m0 + (b >> 2);
        if (m < M) load_block(A + (size_t)m * K + (size_t)t * kStepK + (b & 3) * kBlock, areg[i]);
        else zero_block(areg[i]);
      }
    }
  };
  auto quant_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int b = threadIdx.x + i * NTH;
      if (b < NBLK) {
        const int r = b >> 2, kbl = b & 3;
        const int slot = (r >> 4) * 64 + (r & 15) + 16 * kbl;
        uint32_t q[4];
        const uint32_t s = quant_block(areg[i], q);
        *reinterpret_cast<uint4*>(&sq[buf][slot * 16]) = make_uint4(q[0], q[1], q[2], q[3]);
        ss[buf][slot] = (uint8_t)s;
      }
    }
  };
  uint4 wq[2][NG];
  uint32_t wsc[2][NG];
  auto load_w = [&](int t, int slot) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      wq[slot][g] = load16_nt(Wp + wp_payload_off(gw0 + g, t, lane, T));
      wsc[slot][g] = Wsc[wp_scale_off(gw0 + g, t >> 2, lane, T4) + (t & 3)];
    }
  };

  v4f acc[NG][MT];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[g][mt] = v4f{0.f, 0.f, 0.f, 0.f};

  auto step = [&](int t, int cur, int nxt) {
    quant_store(t & 1);
    if (t + 1 < T) {
      load_a(t + 1);
      load_w(t + 1, nxt);
    }
    __syncthreads();
    uint4 b[MT];
    uint32_t sb[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      b[mt] = *reinterpret_cast<const uint4*>(&sq[t & 1][(mt * 64 + lane) * 16]);
      sb[mt] = ss[t & 1][mt * 64 + lane];
    }
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[g][mt] = mfma_fp4(wq[cur][g], b[mt], acc[g][mt], wsc[cur][g], sb[mt]);
  };

  load_a(0);
  load_w(0, 0);
  for (int t = 0; t < T; t += 2) {
    step(t, 0, 1);
    if (t + 1 < T) step(t + 1, 1, 0);
  }

#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m0 + 16 * mt + (lane & 15);
      const int n = 16 * (gw0 + g) + 4 * (lane >> 4);
      if (m < M)
        *reinterpret_cast<uint2*>(C + (size_t)m * N + n) =
            pack4_bf16(acc[g][mt][0], acc[g][mt][1], acc[g][mt][2], acc[g][mt][3]);
    }
  }
}

// ====================================================================== grouped MoE GEMM1
//
// Expert-segmented A4W4 GEMM: output row r (expert-sorted) = Q(A[row_token[r]]) Q(W_e)^T.
// Work item = (a, c): the a-th expert with at least one row, and NG column groups. Grid size
// is min(E, R_max) * (N / (16 NG)); each CTA finds its expert by a block-wide scan of the
// segment table, so no host sync or workspace is needed and empty experts cost nothing.
// Inside, the small-M scheme: WK waves split K, each keeping its whole share of the expert's
// weight columns in registers while the CTA walks the expert's rows in chunks of 16 * MT;
// each chunk's rows are gathered by token index and quantized into LDS.
// Malformed tables are clamped (segments to [0, R_max], tokens outside [0, T) read as zero
// rows), so every access stays in bounds.
template <int MT, int NG, int WK, int PD>
__global__ __launch_bounds__(64 * WK) void k_gemm_grouped(const uint16_t* __restrict__ A,
                                                          const int32_t* __restrict__ row_token,
                                                          const int32_t* __restrict__ offs, int E,
                                                          int R_max, const uint8_t* __restrict__ Wall,
                                                          uint16_t* __restrict__ C, int Ttok, int N,
                                                          int K) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int NTH = 64 * WK, CH = 16 * MT;
  __shared__ int s_scan[NTH];
  __shared__ int s_e, s_lo, s_hi;
  const int n_chunks = N / (16 * NG);
  const int a = blockIdx.x / n_chunks, c = blockIdx.x % n_chunks;
  const int tid = threadIdx.x;

  // ---- find the a-th non-empty segment
  auto seg = [&](int e, int& lo, int& hi) {
    lo = min(max(offs[e], 0), R_max);
    hi = min(max(offs[e + 1], lo), R_max);
  };
  const int ept = (E + NTH - 1) / NTH;
  int local = 0;
  for (int i = 0; i < ept; ++i) {
    const int e = tid * ept + i;
    if (e < E) { int lo, hi; seg(e, lo, hi); local += (hi > lo); }
  }
  s_scan[tid] = local;
  if (tid == 0) s_e = -1;
  __syncthreads();
  for (int d = 1; d < NTH; d <<= 1) {
    const int v = (tid >= d) ? s_scan[tid - d] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  {
    int rank = s_scan[tid] - local;  // active segments before this thread's range
    if (a >= rank && a < rank + local) {
      for (int i = 0; i < ept; ++i) {
        const int e = tid * ept + i;
        if (e < E) {
          int lo, hi; seg(e, lo, hi);
          if (hi > lo) {
            if (rank == a) { s_e = e; s_lo = lo; s_hi = hi; }
            ++rank;
          }
        }
      }
    }
  }
  __syncthreads();
  const int e = s_e;
  if (e < 0) return;
  const int lo = s_lo, cnt = s_hi - s_lo;

  const int T = steps_of(K), T4 = quads_of(K), KB = K / kBlock;
  const int RS = K / 2 + 16;
  const int lane = tid & 63, w = tid >> 6;
  const int g0 = c * NG;
  const uint8_t* __restrict__ Wp = Wall + (size_t)e * (payload_bytes(N, K) + scale_region_bytes(N, K));
  const uint8_t* __restrict__ Wsc = Wp + payload_bytes(N, K);
  uint8_t* aq = smem;
  uint8_t* as = smem + (size_t)CH * RS;

  const int per = (T + WK - 1) / WK;
  const int t0 = min(T, w * per), t1 = min(T, t0 + per);
  const int S = t1 - t0;
  const bool resident = S <= PD;

  uint4 wq[PD][NG];
  uint32_t wsb[PD][NG];
  auto load_chunk = [&](int tb) {
    const int nh = min(PD, t1 - tb);
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      if (i < nh) {
        const int t = tb + i;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          wq[i][g] = load16_nt(Wp + wp_payload_off(g0 + g, t, lane, T));
          wsb[i][g] = __builtin_nontemporal_load(Wsc + wp_scale_off(g0 + g, t >> 2, lane, T4) + (t & 3));
        }
      }
    }
  };
  if (S > 0 && resident) load_chunk(t0);

  for (int r0 = 0; r0 < cnt; r0 += CH) {
    const int Mc = min(CH, cnt - r0);
    __syncthreads();  // the previous chunk is done with LDS
    {
      const int nbw = 4 * S;
      const int nb = Mc * nbw;
      for (int b = lane; b < nb; b += 64) {
        const int m = b / nbw, kb = 4 * t0 + b % nbw;
        const int tok = row_token[lo + r0 + m];
        uint32_t x[16];
        if (tok >= 0 && tok < Ttok) load_block(A + (size_t)tok * K + (size_t)kb * kBlock, x);
        else zero_block(x);
        uint32_t q[4];
        const uint32_t s = quant_block(x, q);
        *reinterpret_cast<uint4*>(aq + (size_t)m * RS + kb * 16) = make_uint4(q[0], q[1], q[2], q[3]);
        as[(size_t)m * KB + kb] = (uint8_t)s;
      }
    }
    __syncthreads();

    v4f acc[NG][MT];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[g][mt] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int tb = t0; tb < t1; tb += PD) {
      if (!resident) load_chunk(tb);
      const int nh = min(PD, t1 - tb);
#pragma unroll
      for (int i = 0; i < PD; ++i) {
        if (i < nh) {
          const int t = tb + i;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const int m = 16 * mt + (lane & 15);
            const int kb = 4 * t + (lane >> 4);
            uint4 b = make_uint4(0u, 0u, 0u, 0u);
            uint32_t sb = 0u;
            if (m < Mc) {
              b = *reinterpret_cast<const uint4*>(aq + (size_t)m * RS + kb * 16);
              sb = as[(size_t)m * KB + kb];
            }
#pragma unroll
            for (int g = 0; g < NG; ++g) acc[g][mt] = mfma_fp4(wq[i][g], b, acc[g][mt], wsb[i][g], sb);
          }
        }
      }
    }

    auto store = [&](int g, int mt, const v4f& v) {
      const int m = 16 * mt + (lane & 15);
      const int n = 16 * (g0 + g) + 4 * (lane >> 4);
      if (m < Mc)
        *reinterpret_cast<uint2*>(C + (size_t)(lo + r0 + m) * N + n) = pack4_bf16(v[0], v[1], v[2], v[3]);
    };
    __syncthreads();  // every wave is done with the activation region
    v4f* red = reinterpret_cast<v4f*>(smem);  // [WK][NG*MT][64]
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) red[(w * NG * MT + g * MT + mt) * 64 + lane] = acc[g][mt];
    __syncthreads();
    for (int p = w; p < NG * MT; p += WK) {
      v4f sum = red[p * 64 + lane];
      for (int ww = 1; ww < WK; ++ww) sum += red[(ww * NG * MT + p) * 64 + lane];
      store(p / MT, p % MT, sum);
    }
  }
}

// ====================================================================== launchers

hipError_t launch_quant_act(const void* a, int64_t M, int64_t K, void* q, void* s, hipStream_t st) {
  const int64_t nb = M * (K / kBlock);
  if (nb == 0) return hipSuccess;
  const int64_t grid = (nb + 255) / 256;
  hipLaunchKernelGGL(k_quant_act, dim3((unsigned)grid), dim3(256), 0, st,
                     static_cast<const uint16_t*>(a), static_cast<uint8_t*>(q), static_cast<uint8_t*>(s), nb);
  return hipGetLastError();
}

hipError_t launch_prepare(const void* w, int64_t N, int64_t K, void* wp, hipStream_t st) {
  const int64_t n = (N / 16) * quads_of((int)K) * 64;
  hipLaunchKernelGGL(k_prepare, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(w), static_cast<uint8_t*>(wp), (int)N, (int)K);
  return hipGetLastError();
}

hipError_t launch_unprepare(const void* wp, int64_t N, int64_t K, void* q, void* s, hipStream_t st) {
  const int64_t n = (N / 16) * steps_of((int)K) * 64;
  hipLaunchKernelGGL(k_unprepare, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     static_cast<const uint8_t*>(wp), static_cast<uint8_t*>(q), static_cast<uint8_t*>(s),
                     (int)N, (int)K);
  return hipGetLastError();
}

namespace {

constexpr int kSkinnyPD = 16;
constexpr size_t kMaxLds = 160 * 1024;  // LDS per CU (and per workgroup) on gfx950

// Raise a kernel's dynamic-LDS limit to the full 160 KiB once per device. `done` is the
// caller's per-kernel bitmask of devices already configured.
hipError_t ensure_lds_limit(const void* kern, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

size_t skinny_lds_bytes(int M, int K, int MT, int NG, int WK) {
  const size_t act = (size_t)M * (K / 2 + 16) + (size_t)M * (K / kBlock);
  const size_t red = (size_t)WK * NG * MT * 64 * 16;
  return act > red ? act : red;
}

template <int MT, int NG, int WK>
hipError_t run_skinny(const void* a, const void* wp, void* c, int M, int N, int K, hipStream_t st) {
  auto kern = k_gemm_skinny<MT, NG, WK, kSkinnyPD>;
  static std::atomic<uint64_t> configured{0};
  const size_t lds = skinny_lds_bytes(M, K, MT, NG, WK);
  if (lds > 65536) {
    hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), configured);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(N / (16 * NG))), dim3(64 * WK), lds, st,
                     static_cast<const uint16_t*>(a), static_cast<const uint8_t*>(wp),
                     static_cast<uint16_t*>(c), M, N, K);
  return hipGetLastError();
}

template <int MT, int NG, int WN>
hipError_t run_tile(const void* a, const void* wp, void* c, int M, int N, int K, hipStream_t st) {
  constexpr int BM = 16 * MT, BN = 16 * NG * WN;
  const int64_t grid = (int64_t)((M + BM - 1) / BM) * (N / BN);
  hipLaunchKernelGGL((k_gemm_tile<MT, NG, WN>), dim3((unsigned)grid), dim3(64 * WN), 0, st,
                     static_cast<const uint16_t*>(a), static_cast<const uint8_t*>(wp),
                     static_cast<uint16_t*>(c), M, N, K);
  return hipGetLastError();
}

}  // namespace

// The largest M the small-M kernel takes, and its LDS need at that M.
int skinny_max_m() { return 32; }

hipError_t launch_gemm(const void* a, const void* wp, void* c, int64_t M64, int64_t N64, int64_t K64,
                       hipStream_t st) {
  const int M = (int)M64, N = (int)N64, K = (int)K64;
  const int T = steps_of(K);
  const int G = N / 16;
  if (M <= 32 && skinny_lds_bytes(M, K, 2, 1, 8) <= kMaxLds) {
    const int WK = (G < 256) ? 8 : (T >= 8 ? 4 : 2);
    if (M <= 16) {
      if (WK == 8) return run_skinny<1, 1, 8>(a, wp, c, M, N, K, st);
      if (WK == 4) return run_skinny<1, 1, 4>(a, wp, c, M, N, K, st);
      return run_skinny<1, 1, 2>(a, wp, c, M, N, K, st);
    }
    if (WK == 8) return run_skinny<2, 1, 8>(a, wp, c, M, N, K, st);
    if (WK == 4) return run_skinny<2, 1, 4>(a, wp, c, M, N, K, st);
    return run_skinny<2, 1, 2>(a, wp, c, M, N, K, st);
  }
  const int64_t tiles_wide = (int64_t)((M + 63) / 64) * (N / 256);
  if (tiles_wide >= 512) return run_tile<4, 4, 4>(a, wp, c, M, N, K, st);
  return run_tile<4, 1, 4>(a, wp, c, M, N, K, st);
}

namespace {

template <int MT, int NG, int WK>
hipError_t run_grouped(const void* a, const int32_t* rt, const int32_t* offs, int E, int R_max,
                       const void* wp, void* c, int T, int N, int K, hipStream_t st) {
  auto kern = k_gemm_grouped<MT, NG, WK, kSkinnyPD>;
  static std::atomic<uint64_t> configured{0};
  const size_t lds = skinny_lds_bytes(16 * MT, K, MT, NG, WK);
  if (lds > 65536) {
    hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), configured);
    if (e != hipSuccess) return e;
  }
  const int64_t slots = (int64_t)(E < R_max ? E : R_max);
  const int64_t grid = slots * (N / (16 * NG));
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * WK), lds, st, static_cast<const uint16_t*>(a),
                     rt, offs, E, R_max, static_cast<const uint8_t*>(wp), static_cast<uint16_t*>(c), T, N, K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_grouped(const void* a, const int32_t* row_token, const int32_t* offsets, int64_t E,
                               int64_t R_max, const void* wp, void* c, int64_t T, int64_t N, int64_t K,
                               int64_t rows_hint, hipStream_t st) {
  const int e = (int)E, r = (int)R_max, t = (int)T, n = (int)N, k = (int)K;
  if (skinny_lds_bytes(32, k, 2, 4, 4) > kMaxLds) return hipErrorInvalidValue;
  if (rows_hint <= 16) return run_grouped<1, 1, 4>(a, row_token, offsets, e, r, wp, c, t, n, k, st);
  if (rows_hint <= 32) return run_grouped<2, 1, 4>(a, row_token, offsets, e, r, wp, c, t, n, k, st);
  return run_grouped<2, 4, 4>(a, row_token, offsets, e, r, wp, c, t, n, k, st);
}

}  // namespace mx
