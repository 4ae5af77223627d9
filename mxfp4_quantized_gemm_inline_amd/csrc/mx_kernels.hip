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
#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <utility>

#include "mx_device.h"

#include <type_traits>
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

// One thread per (column group g, step t, lane): quantizes the 32-block that lane owns in
// group g at step t and writes it and its byte of the quad's scale word in place (one block
// per thread keeps four times the loads in flight of a thread per quad: the quantize-once
// GEMM at M = 512 went from 35.8 to 34.3 us at 8448 x 7168). Rows n >= valid (padding up to a whole quad of groups) are
// not read and encode as zero blocks with scale byte 0. The same kernel lays out activation rows in this layout for the
// quantize-once GEMM (rows = M padded to a multiple of 64, valid = M).
__global__ __launch_bounds__(256) void k_prepare(const uint16_t* __restrict__ W,
                                                  uint8_t* __restrict__ Wp, int N, int K, int valid) {
  const int T = steps_of(K), G = N / 16;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)G * T * 64) return;
  const int lane = (int)(idx % 64);
  const int64_t r = idx / 64;
  const int t = (int)(r % T), g = (int)(r / T);
  const int n = 16 * g + (lane & 15), kb = 4 * t + (lane >> 4);
  uint32_t x[16];
  if (n < valid) load_block(W + (size_t)n * K + (size_t)kb * kBlock, x);
  else zero_block(x);
  uint32_t qq[4];
  const uint32_t sc = quant_block(x, qq);
  *reinterpret_cast<uint4*>(Wp + wp_payload_off(g, t, lane, T)) = make_uint4(qq[0], qq[1], qq[2], qq[3]);
  // byte g % 4 of the quad's scale word; the other three bytes are written by the threads of
  // the quad's other groups
  Wp[payload_bytes(N, K) + wp_scale_off(g >> 2, t, lane, T) + (g & 3)] = (uint8_t)sc;
}

// Inverse of the preshuffle: canonical payload [N, K/2] and scales [N, K/32].
__global__ __launch_bounds__(256) void k_unprepare(const uint8_t* __restrict__ Wp,
                                                    uint8_t* __restrict__ q,
                                                    uint8_t* __restrict__ s, int N, int K) {
  const int T = steps_of(K), G = N / 16, KB = K / kBlock;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)G * T * 64) return;
  const int lane = (int)(idx % 64);
  const int64_t r = idx / 64;
  const int t = (int)(r % T), g = (int)(r / T);
  const int n = 16 * g + (lane & 15), kb = 4 * t + (lane >> 4);
  const uint4 v = *reinterpret_cast<const uint4*>(Wp + wp_payload_off(g, t, lane, T));
  *reinterpret_cast<uint4*>(q + (size_t)n * (K / 2) + (size_t)kb * 16) = v;
  const uint32_t sword =
      *reinterpret_cast<const uint32_t*>(Wp + payload_bytes(N, K) + wp_scale_off(g >> 2, t, lane, T));
  s[(size_t)n * KB + kb] = (uint8_t)(sword >> (8 * (g & 3)));
}

// ====================================================================== streaming GEMM (small and mid M)
//
// StreamCTA is the CTA-level building block shared by the dense small-M GEMM and the
// grouped GEMM: WK waves compute 16 * NG output columns for up to 16 * MT rows over a range
// of 128-wide K steps, splitting the steps between waves. Each wave streams its share of
// the prepared weight straight from HBM into registers, PD steps at a time (the weight has
// no reuse here, so it is not staged in LDS), quantizes its own activation blocks into LDS
// (QB blocks per lane per batch, loads issued before any is used), runs its MFMAs, and the
// wave partial sums are added in LDS in a fixed wave order.
//
// Weight loads are branch-free (steps past the wave's range re-load its last step and are
// never multiplied), and the first activation batch is issued before them, so the compiler's
// in-order wait counts let the weight stream stay in flight while the quantizer runs.
//
// LDS: quantized activations [R][TS * 64 + 16] (the 16-byte pad staggers rows across banks),
// then their scales [R][4 TS], R = the rows a launch stages (at most 16 MT; reads of rows
// past the valid count are clamped to the last one); reused for the cross-wave reduction.
constexpr int kSkinnyPD = 16;
// The dense streaming kernel affords twice the weight operands in flight (it holds no
// resident weight chunk): at 8448 x 7168 a wave's seven steps of four column groups then go
// out at once (M = 8: 12.6 -> 11.6 us, M = 16: 15.0 -> 13.6 us).
constexpr int kStreamPD = 32;

// Rows of a dense row-major A.
struct DenseRows {
  const uint16_t* A;
  int K;
  __device__ __forceinline__ const uint16_t* ptr(int m, bool& valid) const {
    valid = true;
    return A + (size_t)m * K;
  }
};

// Rows gathered by token index; an index outside [0, T) reads as an all-zero row (its
// load goes to row 0 and the quantized block is replaced by zeros).
struct GatherRows {
  const uint16_t* A;
  const int32_t* tok;
  int base, T, K;
  __device__ __forceinline__ const uint16_t* ptr(int m, bool& valid) const {
    const int t = tok[base + m];
    valid = t >= 0 && t < T;
    return A + (size_t)(valid ? t : 0) * K;
  }
};

template <int MT, int NG, int WK, int PD, int QB>
struct StreamCTA {
  // With one activation block per lane, every lane stores (lanes past the last block store
  // its bytes again), so no branch guards the store and the compiler keeps the block's load
  // ahead of the weight loads: the quantization waits for it alone and the weight stream
  // stays in flight behind it (8448 x 7168 M=1: 10.0 -> 9.1 us; 1536 x 7168 M=1 4.9 -> 4.35
  // us). With four blocks per lane the branch stays (the same form measured 0.2-1.8 us
  // slower there: more registers live across the weight loads, and at 64 x 4 blocks a
  // pile-up of lanes on one LDS address or a modulo per block to avoid it).
  static constexpr bool kGuarded = QB > 1;
  int lane, T, g0, ks0, t0, t1, S, RS, SB;
  const uint8_t* __restrict__ Wp;
  const uint8_t* __restrict__ Wsc;
  uint8_t* aq;
  uint8_t* as;
  uint4 wq[PD][NG];
  uint32_t wsb[PD][NG];

  __device__ __forceinline__ void init(const uint8_t* wp, int N, int K, int g0_, int ks0_, int ks1, int TS,
                                       int R, uint8_t* smem) {
    lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    T = steps_of(K);
    g0 = g0_;
    ks0 = ks0_;
    const int slice = ks1 - ks0;
    const int per = (slice + WK - 1) / WK;
    t0 = ks0 + min(slice, w * per);
    t1 = min(ks1, t0 + per);
    S = t1 - t0;
    RS = TS * 64 + 16;
    SB = 4 * TS;
    Wp = wp;
    Wsc = wp + payload_bytes(N, K);
    aq = smem;
    as = smem + (size_t)R * RS;
  }

  __device__ __forceinline__ void load_w(int tb) {
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      // t1 - 1 >= 0 whenever K has a step, also for a wave with no step (t1 = t0 >= 1 then);
      // the clamp at 0 only keeps the unguarded form's register allocation as measured
      const int t = kGuarded ? min(tb + i, t1 - 1) : max(0, min(tb + i, t1 - 1));
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        wq[i][g] = load16_nt(Wp + wp_payload_off(g0 + g, t, lane, T));
        // the scale byte of group g0+g sits in byte (g0+g)%4 of its quad's word
        wsb[i][g] = __builtin_nontemporal_load(Wsc + wp_scale_off((g0 + g) >> 2, t, lane, T) + ((g0 + g) & 3));
      }
    }
  }

  // Quantize rows [0, Mc) of this wave's blocks 4*t0 .. 4*t1-1 into LDS. `after_first`
  // runs once, right after the first batch's loads are issued. With several blocks per lane
  // and a `weights_always` call (the weight loads issued on every path), a wave whose blocks
  // fit one batch takes the single-batch form below.
  template <class Rows, class F, class G = std::nullptr_t>
  __device__ __forceinline__ void quant(const Rows& rows, int Mc, F&& after_first, G&& weights_always = nullptr) {
    const int nbw = 4 * S, nb = Mc * nbw;
    if (nb <= 0) {
      after_first();
      return;
    }
    const int q64 = 64 / nbw, r64 = 64 % nbw;
    int m = lane / nbw, r = lane % nbw;  // coordinates of block b = lane
    if constexpr (kGuarded && !std::is_same_v<std::decay_t<G>, std::nullptr_t>) {
      if (nb <= 64 * QB) {
        // one batch: every load of it first (block coordinates computed branch-free), then
        // the weight loads, and no branch around the stores, so the quantization waits for
        // the activation loads alone; lanes past the last block write into the 16 spare
        // bytes that end row Mc - 1 (never read)
        uint32_t x[QB][16];
        int mm[QB], rr[QB];
        bool val[QB], spare[QB];
        const uint16_t* src[QB];
#pragma unroll
        for (int j = 0; j < QB; ++j) {
          const bool ok = j * 64 + lane < nb;
          mm[j] = ok ? m : Mc - 1;
          rr[j] = ok ? r : nbw - 1;
          spare[j] = !ok;
          src[j] = rows.ptr(mm[j], val[j]) + (size_t)(4 * t0 + rr[j]) * kBlock;
          m += q64;
          r += r64;
          const int wrap = r >= nbw ? 1 : 0;
          r -= wrap * nbw;
          m += wrap;
        }
#pragma unroll
        for (int j = 0; j < QB; ++j) load_block(src[j], x[j]);
        __builtin_amdgcn_sched_barrier(0);
        weights_always();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < QB; ++j) {
          uint32_t q[4];
          uint32_t sc = quant_block(x[j], q);
          if (!val[j]) { q[0] = q[1] = q[2] = q[3] = 0u; sc = 0u; }
          const int kbl = 4 * (t0 - ks0) + rr[j];  // block index within the slice
          uint8_t* const row = aq + (size_t)mm[j] * RS;
          uint8_t* const pq = spare[j] ? row + RS - 16 : row + kbl * 16;
          uint8_t* const ps = spare[j] ? row + RS - 1 : as + (size_t)mm[j] * SB + kbl;
          *reinterpret_cast<uint4*>(pq) = make_uint4(q[0], q[1], q[2], q[3]);
          *ps = (uint8_t)sc;
        }
        return;
      }
    }
    bool first = true;
    for (int base = 0; base < nb; base += 64 * QB) {
      uint32_t x[QB][16];
      int mm[QB], rr[QB];
      bool val[QB];
      if constexpr (kGuarded) {
#pragma unroll
        for (int j = 0; j < QB; ++j) {
          const bool ok = base + j * 64 + lane < nb;
          mm[j] = ok ? m : Mc - 1;  // lanes past the last block re-load it and store nothing
          rr[j] = ok ? r : nbw - 1;
          const uint16_t* row = rows.ptr(mm[j], val[j]);
          load_block(row + (size_t)(4 * t0 + rr[j]) * kBlock, x[j]);
          mm[j] = ok ? m : -1;
          m += q64;
          r += r64;
          if (r >= nbw) { r -= nbw; ++m; }
        }
        if (first) {
          after_first();
          first = false;
        }
      } else {
        // lanes past the last block re-load it and store its bytes again
        const bool ok = base + lane < nb;
        mm[0] = ok ? m : Mc - 1;
        rr[0] = ok ? r : nbw - 1;
        load_block(rows.ptr(mm[0], val[0]) + (size_t)(4 * t0 + rr[0]) * kBlock, x[0]);
        m += q64;
        r += r64;
        if (r >= nbw) { r -= nbw; ++m; }
        if (first) {
          // the activation load stays ahead of the weight loads in the instruction stream
          __builtin_amdgcn_sched_barrier(0);
          after_first();
          __builtin_amdgcn_sched_barrier(0);
          first = false;
        }
      }
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        uint32_t q[4];
        uint32_t sc = quant_block(x[j], q);
        if (!val[j]) { q[0] = q[1] = q[2] = q[3] = 0u; sc = 0u; }
        if (kGuarded && mm[j] < 0) continue;
        const int kbl = 4 * (t0 - ks0) + rr[j];  // block index within the slice
        *reinterpret_cast<uint4*>(aq + (size_t)mm[j] * RS + kbl * 16) = make_uint4(q[0], q[1], q[2], q[3]);
        as[(size_t)mm[j] * SB + kbl] = (uint8_t)sc;
      }
    }
  }

  // acc += this wave's steps for rows [0, Mc) (rows past Mc read row Mc-1 and are never stored).
  // With `resident`, the weight chunk loaded at t0 is reused; otherwise chunks are (re)loaded.
  __device__ __forceinline__ void mma(int Mc, bool resident, v4f (&acc)[NG][MT]) {
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[g][mt] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int tb = t0; tb < t1; tb += PD) {
      if (!resident && tb != t0) load_w(tb);
      const int nh = min(PD, t1 - tb);
#pragma unroll
      for (int i = 0; i < PD; ++i) {
        if (i < nh) {
          const int kbl = 4 * (tb + i - ks0) + (lane >> 4);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const int m = min(16 * mt + (lane & 15), Mc - 1);
            const uint4 b = *reinterpret_cast<const uint4*>(aq + (size_t)m * RS + kbl * 16);
            const uint32_t sb = as[(size_t)m * SB + kbl];
#pragma unroll
            for (int g = 0; g < NG; ++g) acc[g][mt] = mfma_fp4(wq[i][g], b, acc[g][mt], wsb[i][g], sb);
          }
        }
      }
    }
  }

  // Sum the wave partials in wave order through LDS (which must be free) and hand each
  // (g, mt) 4-column group to store(g, mt, value).
  template <class Store>
  __device__ __forceinline__ void reduce_store(v4f (&acc)[NG][MT], uint8_t* smem, Store&& store) {
    if constexpr (WK == 1) {
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) store(g, mt, acc[g][mt]);
    } else {
      const int w = threadIdx.x >> 6;
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
};

// Dense small-M GEMM: CTA (x, y) owns column groups [x NG, x NG + NG) and K slice y of TS
// steps. One slice: bf16 C directly; several: FP32 partials to P[slice][M][N], added in
// slice order by k_splitk_reduce (deterministic).
template <int MT, int NG, int WK, int PD, int QB>
__global__ __launch_bounds__(64 * WK) void k_gemm_stream(const uint16_t* __restrict__ A,
                                                         const uint8_t* __restrict__ Wp,
                                                         uint16_t* __restrict__ C,
                                                         float* __restrict__ P, int M, int N, int K,
                                                         int TS) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int T = steps_of(K);
  const int ks0 = min(T, (int)blockIdx.y * TS), ks1 = min(T, ks0 + TS);
  // column chunks dealt to the XCDs in contiguous ranges: the CTAs that share a weight scale
  // word (four column groups) mostly share an L2
  int unused, cg;
  tile_coords(blockIdx.x, gridDim.x, 1, gridDim.x, 1, unused, cg);
  StreamCTA<MT, NG, WK, PD, QB> cta;
  cta.init(Wp, N, K, cg * NG, ks0, ks1, TS, min(M, 16 * MT), smem);
  const DenseRows rows{A, K};
  // unconditional where the quantization should wait for the activation loads alone (a load
  // issued on one branch only makes the compiler wait for every load at the join); a wave
  // with no step then loads its last step's neighbour, never used
  using CTA = StreamCTA<MT, NG, WK, PD, QB>;
  cta.quant(rows, M, [&] { if (!CTA::kGuarded || cta.S > 0) cta.load_w(cta.t0); },
            [&] { cta.load_w(cta.t0); });
  __syncthreads();
  v4f acc[NG][MT];
  cta.mma(M, false, acc);
  if constexpr (WK > 1) __syncthreads();  // every wave is done with the activation region
  const int lane = threadIdx.x & 63;
  cta.reduce_store(acc, smem, [&](int g, int mt, const v4f& v) {
    const int m = 16 * mt + (lane & 15);
    const int n = 16 * (cg * NG + g) + 4 * (lane >> 4);
    if (m < M) {
      if (P) *reinterpret_cast<v4f*>(P + ((size_t)blockIdx.y * M + m) * N + n) = v;
      else *reinterpret_cast<uint2*>(C + (size_t)m * N + n) = pack4_bf16(v[0], v[1], v[2], v[3]);
    }
  });
}

// C = bf16(sum over slices s = 0..S-1, in order, of P[s]); four elements per thread. The
// slices are loaded eight at a time, all eight loads in flight before the first add (a
// load-add loop waits out one memory latency per slice); slices past S re-load the last one
// and are not added.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ P,
                                                       uint16_t* __restrict__ C, int64_t MN, int S) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= MN) return;
  v4f acc = *reinterpret_cast<const v4f*>(P + i);
  for (int s0 = 1; s0 < S; s0 += 8) {
    v4f x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = *reinterpret_cast<const v4f*>(P + (size_t)min(s0 + u, S - 1) * MN + i);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < S) acc += x[u];
  }
  *reinterpret_cast<uint2*>(C + i) = pack4_bf16(acc[0], acc[1], acc[2], acc[3]);
}

// ====================================================================== tiled GEMM (large M)
//
// A CTA owns a BM x BN output tile, BM = 16 * MT * WM rows and BN = 16 * NG * WN columns,
// computed by WM x WN waves of MT x NG MFMA tiles each. Every 128-wide K step, all threads
// quantize their share of the BM x 128 activation tile (one or more 32-blocks per thread)
// into one of two LDS buffers in MFMA operand order; each wave reads its weight operands
// straight from global memory (a contiguous 1 KiB each) and its activation operands from
// LDS. Global loads run PF steps ahead of the MFMAs (activations in PF register slots,
// weights in PF + 1). A tile whose columns run past N (BN not dividing N) masks whole
// column groups. Tiles are dealt to CTAs in the XCD-aware order of tile_coords.
template <int WM, int WN, int MT, int NG>
struct TileShape {
  static constexpr int MTC = MT * WM;  // 16-row tiles per CTA
  static constexpr int BM = 16 * MTC, BN = 16 * NG * WN;
  static constexpr int NW = WM * WN, NTH = 64 * NW;
  static constexpr int BPT = MTC / NW;  // 32-block quads per thread per step
  // LDS: two buffers of quantized activation operands (SQ each) and their scales (SS each),
  // the scales stored as [lane][16-row tile] bytes so a lane's scales for four tiles are one
  // word; after the K loop the same memory stages the bf16 output tile (rows padded by 16
  // bytes against bank conflicts).
  static constexpr int SQ = MTC * 1024, SS = 64 * MTC;
  static constexpr int CROW = BN * 2 + 16, CSTAGE = BM * CROW;
  static constexpr int SMEM = 2 * (SQ + SS) > CSTAGE ? 2 * (SQ + SS) : CSTAGE;
  static_assert(MTC % NW == 0, "every wave quantizes whole 16-row tiles");
  static_assert(MT % 4 == 0, "a wave's tiles cover whole scale words");
};

// Activation rows of one CTA tile. Dense: tile row r is the row at base + r * K (bf16), with
// base wave-uniform, so a lane keeps only a 32-bit offset per row (K < 2^24 keeps it exact).
struct TileRowsDense {
  const uint8_t* base;
  int K;
  static constexpr bool kGather = false, kMx = false;
};
// Gathered: tile row r is A[tok[r]]; a token outside [0, T) reads as an all-zero row.
struct TileRowsGather {
  const uint8_t* A;
  const int32_t* tok;
  int T, K;
  static constexpr bool kGather = true, kMx = false;
};
// Already quantized: tile row r is MXFP4 row r (canonical payload q [rows, K/2] and scales
// s [rows, K/32], both offset to the tile's first row); no quantization takes place.
struct TileRowsMx {
  const uint8_t* q;
  const uint8_t* s;
  int K;
  static constexpr bool kGather = false, kMx = true;
};

// Fused GEMM1 epilogue ("[gfx1250] Fuse A4W4 stage1 FP4 quantization", Summary): the
// activation h = SiLU(c), or SiLU(gate) * up with the gate columns in the first half of the
// GEMM1 output and the up columns in the second, formed in FP32 from the accumulators and
// quantized to MXFP4 along its columns (32-blocks, E8M0 scale from the FP32 block amax),
// written as canonical payload [rows, Nh/2] and scales [rows, Nh/32].
constexpr int kActSilu = 0, kActSwiglu = 1;
struct ActOut {
  uint8_t* q = nullptr;  // packed E2M1 of the tile's first row
  uint8_t* s = nullptr;  // E8M0 scales of the tile's first row
  int Nh = 0;            // columns of h
};

// The tiled main loop and epilogue for one BM x BN output tile: Mrows (1..BM) valid rows
// from `rows`, weight column tile bn of the prepared weight Wp, output rows written at
// Cout + r * N for r < Mrows (columns past N masked). Only K steps [tb, te) are summed; with
// Pout the FP32 sums go to Pout + r * N (one K slice's partial tile) instead of bf16 to Cout.
// With ACT >= 0 the tile's output is the fused activation + quantization into `ao` instead:
// for SwiGLU the first WN/2 waves compute gate columns and the others the matching up
// columns, so the CTA's BN weight columns yield BN/2 columns of h (h tile bn); for SiLU the
// column mapping is the plain one and h tile bn is output tile bn.
template <int WM, int WN, int MT, int NG, int PF, int ACT = -1, class Rows>
__device__ __forceinline__ void tile_core(const Rows& rows, int Mrows, const uint8_t* __restrict__ Wp,
                                          uint16_t* __restrict__ Cout, float* __restrict__ Pout, int N,
                                          int K, int bn, int tb, int te, uint8_t* __restrict__ smem,
                                          const ActOut& ao = ActOut{}) {
  using S = TileShape<WM, WN, MT, NG>;
  constexpr int MTC = S::MTC, BM = S::BM, BN = S::BN, NW = S::NW, BPT = S::BPT;
  constexpr int SQ = S::SQ, SS = S::SS, CROW = S::CROW;
  auto sq = [&](int buf, int off) { return smem + buf * SQ + off; };
  auto ss = [&](int buf, int off) { return smem + 2 * SQ + buf * SS + off; };

  const int T = steps_of(K), G = N / 16;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w / WN, wn = w % WN;
  static_assert(ACT < 0 || WN % 2 == 0, "the fused epilogue pairs the two halves of the waves");
  const int gw0 = ACT == kActSwiglu
                      ? (wn < WN / 2 ? bn * (BN / 32) + wn * NG : G / 2 + bn * (BN / 32) + (wn - WN / 2) * NG)
                      : bn * (BN / 16) + wn * NG;
  const uint8_t* __restrict__ Wsc = Wp + payload_bytes(N, K);

  // Loads are branch-free so the compiler can count them: tile rows past Mrows re-read the
  // last valid row and column groups past N re-read the last group; neither result is ever
  // stored. Lane 4r+j of wave v quantizes, for i < BPT, the whole 32-block j of row r of
  // the 16-row tile v + NW i (four 16-byte loads; a quad covers the row's 256 contiguous
  // bytes of the step). In LDS a tile holds its 16 x 4 operand blocks row-major with the
  // block index XOR-swizzled by the row; the quant stores (16 bytes per lane) and the MFMA
  // reads (lane = row + 16 block) then fall on distinct banks.
  uint32_t aoff[BPT];
  const uint8_t* aptr[BPT];
  bool avalid[BPT];
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const int r = min(16 * (w + NW * i) + (lane >> 2), Mrows - 1);
    if constexpr (Rows::kMx) {  // payload byte offset of the lane's block at step 0; its scale follows from r
      aoff[i] = (uint32_t)r * (uint32_t)(rows.K / 2) + (uint32_t)(lane & 3) * 16u;
      aptr[i] = rows.s + (size_t)r * (rows.K / kBlock) + (lane & 3);
    } else if constexpr (!Rows::kGather) {
      aoff[i] = (uint32_t)r * (uint32_t)rows.K * 2u + (uint32_t)(lane & 3) * (kBlock * 2);
    } else {
      const int tk = rows.tok[r];
      avalid[i] = tk >= 0 && tk < rows.T;
      aptr[i] = rows.A + (size_t)(avalid[i] ? tk : 0) * rows.K * 2 + (lane & 3) * (kBlock * 2);
    }
  }
  auto swz = [](int rr) { return ((rr >> 1) ^ (rr >> 2)) & 3; };
  const uint32_t st_off = (uint32_t)(((lane >> 2) * 4 + ((lane & 3) ^ swz(lane >> 2))) * 16);
  const uint32_t st_sc = (uint32_t)(((lane >> 2) + 16 * (lane & 3)) * MTC);  // this block's operand lane
  const uint32_t ld_off = (uint32_t)(((lane & 15) * 4 + ((lane >> 4) ^ swz(lane & 15))) * 16);
  constexpr int NQ = (NG + 3) / 4;  // scale words per step: one per column-group quad
  const uint8_t* wbase[NG];
  const uint8_t* sbase[NQ];
#pragma unroll
  for (int g = 0; g < NG; ++g) wbase[g] = Wp + (size_t)min(gw0 + g, G - 1) * T * 1024;
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) sbase[qi] = Wsc + (size_t)min((gw0 >> 2) + qi, G / 4 - 1) * T * 256;
  const uint32_t wlane = lane * 16, slane = lane * 4;
  const int sbyte = gw0 & 3;  // byte of group gw0 in its scale word (0 when NG % 4 == 0)

  // a lane's activation block per slot: 16 bf16 words, or (already quantized) 4 payload
  // words and the scale byte
  constexpr int AW = Rows::kMx ? 5 : 16;
  uint32_t areg[PF][BPT][AW];
  uint4 wq[PF + 1][NG];
  uint32_t wsw[PF + 1][NQ];

  auto load_a = [&](int t, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
    if constexpr (Rows::kMx) {
#pragma unroll
      for (int i = 0; i < BPT; ++i) {
        const uint4 u = *reinterpret_cast<const uint4*>(rows.q + (size_t)t * (kStepK / 2) + aoff[i]);
        areg[SL][i][0] = u.x; areg[SL][i][1] = u.y; areg[SL][i][2] = u.z; areg[SL][i][3] = u.w;
        areg[SL][i][4] = aptr[i][(size_t)t * (kStepK / kBlock)];
      }
    } else if constexpr (!Rows::kGather) {
      const uint8_t* base = rows.base + (size_t)t * kStepK * 2;
#pragma unroll
      for (int i = 0; i < BPT; ++i) load_block_at(base, aoff[i], areg[SL][i]);
    } else {
#pragma unroll
      for (int i = 0; i < BPT; ++i) load_block_at(aptr[i] + (size_t)t * kStepK * 2, 0u, areg[SL][i]);
    }
  };
  auto load_w = [&](int t, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
#pragma unroll
    for (int g = 0; g < NG; ++g) wq[SL][g] = *reinterpret_cast<const uint4*>(wbase[g] + (size_t)t * 1024 + wlane);
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) wsw[SL][qi] = *reinterpret_cast<const uint32_t*>(sbase[qi] + (size_t)t * 256 + slane);
  };

  v4f acc[NG][MT];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[g][mt] = v4f{0.f, 0.f, 0.f, 0.f};

  // prologue: steps 0 .. PF-1 in flight (clamped to the last step when T < PF)
  static_for<PF>([&](auto p) {
    load_a(min(tb + (int)decltype(p)::value, te - 1), p);
    load_w(min(tb + (int)decltype(p)::value, te - 1), p);
  });

  auto step = [&](int t, auto sa_c, auto sw_c) {
    constexpr int SA = decltype(sa_c)::value, SW = decltype(sw_c)::value;
    const int buf = t & 1;
    // Keep each step's quantization inside its step: hoisted into the previous step, it
    // would wait there on loads issued only one step earlier and void the prefetch depth.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int tile = w + NW * i;
      uint32_t q[4];
      uint32_t sc;
      if constexpr (Rows::kMx) {
        q[0] = areg[SA][i][0]; q[1] = areg[SA][i][1]; q[2] = areg[SA][i][2]; q[3] = areg[SA][i][3];
        sc = areg[SA][i][4];
      } else {
        sc = quant_block(areg[SA][i], q);
      }
      if constexpr (Rows::kGather) {  // a row with no valid token quantizes to zero
#pragma unroll
        for (int c = 0; c < 4; ++c) q[c] = avalid[i] ? q[c] : 0u;
        sc = avalid[i] ? sc : 0u;
      }
      *reinterpret_cast<uint4*>(sq(buf, tile * 1024 + st_off)) = make_uint4(q[0], q[1], q[2], q[3]);
      *ss(buf, st_sc + tile) = (uint8_t)sc;
    }
    const int tn = min(t + PF, te - 1);  // past the end: a harmless re-load of the last step
    load_a(tn, sa_c);
    load_w(tn, std::integral_constant<int, (SW + PF) % (PF + 1)>{});
    __syncthreads();
    uint4 b[MT];
    uint32_t sbw[MT / 4];  // byte mt % 4 of word mt / 4: the scale of this wave's tile mt
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      b[mt] = *reinterpret_cast<const uint4*>(sq(buf, (wm * MT + mt) * 1024 + ld_off));
#pragma unroll
    for (int j = 0; j < MT / 4; ++j)
      sbw[j] = *reinterpret_cast<const uint32_t*>(ss(buf, lane * MTC + wm * MT + 4 * j));
    static_for<NG>([&](auto g_c) {
      constexpr int g = decltype(g_c)::value;
      static_for<MT>([&](auto m_c) {
        constexpr int mt = decltype(m_c)::value;
        if constexpr (NG % 4 == 0) {  // aligned quads: the group's byte is a compile-time op_sel
          acc[g][mt] = mfma_fp4_sel<g & 3, mt & 3>(wq[SW][g], b[mt], acc[g][mt], wsw[SW][g >> 2], sbw[mt >> 2]);
        } else {
          acc[g][mt] = mfma_fp4_sel<0, mt & 3>(wq[SW][g], b[mt], acc[g][mt], wsw[SW][0] >> (8 * (sbyte + g)),
                                               sbw[mt >> 2]);
        }
      });
    });
  };

  constexpr int U = PF * (PF + 1);
  int t = tb;
  for (; t + U <= te; t += U) {
    static_for<U>([&](auto i) {
      constexpr int I = decltype(i)::value;
      step(t + I, std::integral_constant<int, I % PF>{}, std::integral_constant<int, I % (PF + 1)>{});
    });
  }
  static_for<U - 1>([&](auto i) {
    constexpr int I = decltype(i)::value;
    if (t + I < te) step(t + I, std::integral_constant<int, I % PF>{}, std::integral_constant<int, I % (PF + 1)>{});
  });

  if constexpr (ACT >= 0) {
    // Stage FP32 values in LDS as [BM][HC + 4] (16-byte row pad), half of the tile's
    // columns at a time (the same bytes as the bf16 output staging), then each thread
    // quantizes one 32-column block of one row.
    constexpr int HC = BN / 2, HROW = HC + 4, NB = HC / 32;
    static_assert(BM * HROW * 4 <= S::SMEM, "the staged half tile fits the LDS");
    float* hb = reinterpret_cast<float*>(smem);
    const int half = wn / (WN / 2), cw = (wn % (WN / 2)) * NG;
    // 16-byte chunk ch of a staged row sits at chunk position sw(ch): XOR-swizzled within
    // its 32-float block by the block index, so the quantizer's lanes, which read chunk i
    // of consecutive blocks together, mostly fall on distinct banks.
    auto sw = [](int ch) { return (ch & ~7) | ((ch ^ (ch >> 3)) & 7); };
    auto at = [&](int g, int mt) {
      return hb + (16 * (wm * MT + mt) + (lane & 15)) * HROW + 4 * sw(4 * (cw + g) + (lane >> 4));
    };
    // SiLU(x) = x * sigmoid(x) with e = exp(-|x|) in (0, 1] (no overflow): sigmoid is
    // 1 / (1 + e) for x >= 0 and e / (1 + e) below; v_exp_f32 and v_rcp_f32 (1 ulp each),
    // relative error at most (|x| + 8) * 2^-23 with the rounding of the exponent argument.
    auto silu = [](float x) {
      const float e = __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f);  // log2(e)
      const float r = __builtin_amdgcn_rcpf(1.0f + e);
      return x * (x >= 0.f ? r : e * r);
    };
    auto quantize = [&](int col0) {  // h columns [col0, col0 + HC) of this tile's rows
      for (int id = threadIdx.x; id < BM * NB; id += 64 * NW) {
        const int r = id / NB, b = id % NB;
        if (r >= Mrows) continue;
        const float* p = hb + r * HROW;
        float v[32];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const v4f x = *reinterpret_cast<const v4f*>(p + 4 * sw(8 * b + i));
          v[4 * i] = x[0]; v[4 * i + 1] = x[1]; v[4 * i + 2] = x[2]; v[4 * i + 3] = x[3];
        }
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
        const uint32_t ex = (__builtin_bit_cast(uint32_t, amax) >> 23) & 0xffu;
        const uint32_t sb = ex > 2u ? ex - 2u : 0u;  // e = floor(log2 amax) - 2, clamped at -127
        const float sc = __builtin_bit_cast(float, sb ? (sb << 23) : 0x00400000u);
        uint32_t q[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t w4 = 0;
          w4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w4, v[8 * j + 0], v[8 * j + 1], sc, 0);
          w4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w4, v[8 * j + 2], v[8 * j + 3], sc, 1);
          w4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w4, v[8 * j + 4], v[8 * j + 5], sc, 2);
          w4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w4, v[8 * j + 6], v[8 * j + 7], sc, 3);
          q[j] = w4;
        }
        *reinterpret_cast<uint4*>(ao.q + (size_t)r * (ao.Nh / 2) + (col0 + 32 * b) / 2) = make_uint4(q[0], q[1], q[2], q[3]);
        ao.s[(size_t)r * (ao.Nh / 32) + col0 / 32 + b] = (uint8_t)sb;
      }
    };
    __syncthreads();  // every wave has finished reading the operand buffers
    if constexpr (ACT == kActSwiglu) {
      if (half == 1) {  // up columns to LDS
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<v4f*>(at(g, mt)) = acc[g][mt];
      } else {  // meanwhile the gate waves take SiLU of their accumulators in place
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[g][mt][j] = silu(acc[g][mt][j]);
      }
      __syncthreads();
      if (half == 0)  // h = SiLU(gate) * up, in place
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            float* p = at(g, mt);
            const v4f u = *reinterpret_cast<const v4f*>(p);
            v4f h;
#pragma unroll
            for (int j = 0; j < 4; ++j) h[j] = acc[g][mt][j] * u[j];
            *reinterpret_cast<v4f*>(p) = h;
          }
      __syncthreads();
      quantize(bn * HC);
    } else {
      for (int ph = 0; ph < 2; ++ph) {
        if (half == ph)
#pragma unroll
          for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              v4f h;
#pragma unroll
              for (int j = 0; j < 4; ++j) h[j] = silu(acc[g][mt][j]);
              *reinterpret_cast<v4f*>(at(g, mt)) = h;
            }
        __syncthreads();
        quantize(bn * BN + ph * HC);
        __syncthreads();
      }
    }
    return;
  }

  if (Pout) {  // a K slice: FP32 partial sums, 16 bytes per lane (four columns of one row)
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = 16 * (wm * MT + mt) + (lane & 15);
        if (r < Mrows && gw0 + g < G)
          *reinterpret_cast<v4f*>(Pout + (size_t)r * N + 16 * (gw0 + g) + 4 * (lane >> 4)) = acc[g][mt];
      }
    return;
  }

  // Epilogue: each lane holds four consecutive columns of one row per MFMA tile; stage the
  // tile in LDS as bf16, then every wave store writes 16 bytes per lane along whole rows.
  __syncthreads();  // every wave has finished reading the operand buffers
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = 16 * (wm * MT + mt) + (lane & 15);
      const int cl = 16 * (wn * NG + g) + 4 * (lane >> 4);
      *reinterpret_cast<uint2*>(smem + r * CROW + cl * 2) =
          pack4_bf16(acc[g][mt][0], acc[g][mt][1], acc[g][mt][2], acc[g][mt][3]);
    }
  __syncthreads();
  constexpr int CPR = BN / 8;  // 16-byte chunks per tile row
  static_assert((BM * CPR) % (64 * NW) == 0, "every thread stores the same number of chunks");
  const int n0 = bn * BN;
#pragma unroll
  for (int i = 0; i < BM * CPR / (64 * NW); ++i) {
    const int id = threadIdx.x + i * 64 * NW;
    const int r = id / CPR, ch = id % CPR;
    const int n = n0 + 8 * ch;
    if (r < Mrows && n < N) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * CROW + ch * 16);
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(Cout + (size_t)r * N + n));
    }
  }
}

template <int WM, int WN, int MT, int NG, int PF, int OCC>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(OCC, 8)))
void k_gemm_tile(const uint16_t* __restrict__ A, const uint8_t* __restrict__ Wp, uint16_t* __restrict__ C,
                 float* __restrict__ P, int M, int N, int K, int GM, int TS) {
  using S = TileShape<WM, WN, MT, NG>;
  __shared__ __align__(16) uint8_t smem[S::SMEM];
  const int tiles_m = (M + S::BM - 1) / S::BM, tiles_n = (N + S::BN - 1) / S::BN;
  int bm, bn;
  tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, GM, bm, bn);
  const int m0 = bm * S::BM;
  // K slice blockIdx.y of TS steps; with P, its FP32 partial tile goes to P[slice]
  const int T = steps_of(K), tb = min(T, (int)blockIdx.y * TS), te = min(T, tb + TS);
  float* Pout = P ? P + ((size_t)blockIdx.y * M + m0) * N : nullptr;
  const TileRowsDense rows{reinterpret_cast<const uint8_t*>(A) + (size_t)m0 * K * 2, K};
  tile_core<WM, WN, MT, NG, PF>(rows, min(S::BM, M - m0), Wp, C + (size_t)m0 * N, Pout, N, K, bn, tb, te, smem);
}

// ====================================================================== short-K sweep GEMM (large M)
//
// When K is at most eight 128-wide steps, a CTA's activation rows fit the LDS whole once
// quantized (BM x K/2 payload bytes and BM x K/32 scale bytes: 68 KiB for 128 rows at
// K = 1024). A CTA then quantizes its BM rows over the whole K once and sweeps J adjacent
// column tiles of BN columns. Inside a column tile the waves only read activation
// operands from LDS and stream their weight operands from global memory; the weight
// stream runs PF steps ahead without a break at column-tile boundaries, so the K loop
// holds no barrier. Each tile's bf16 output is staged in one of two LDS buffers and
// stored while the next tiles' MFMAs run. Vector-memory stores and loads retire in issue
// order, so a load issued after a tile's stores cannot be waited on before those stores
// complete: with PF beyond one tile's steps, the first such wait comes PF - T steps into
// the tile after next.
//
// LDS: activation payload [T][16-row tile][1 KiB operand block] (the XOR-swizzled operand
// layout of tile_core), scales [T][operand lane][16-row tile] bytes, then two output
// staging buffers [BM][BN + 8] bf16.
template <int WM, int WN, int MT, int NG, int T, int PF>
struct SweepShape {
  static constexpr int MTC = MT * WM, BM = 16 * MTC, BN = 16 * NG * WN, NW = WM * WN, NTH = 64 * NW;
  static constexpr int IPW = T * MTC / NW;  // (step, 16-row tile) items each wave quantizes
  static constexpr int AQ = T * MTC * 1024, AS = T * 64 * MTC;
  static constexpr int CROW = BN * 2 + 16, CS = BM * CROW;
  static constexpr int SMEM = AQ + AS + 2 * CS;
  static constexpr int R = PF + 1;  // weight register slots, indexed by the flattened step
  static_assert((T * MTC) % NW == 0, "every wave quantizes the same number of items");
  static_assert(MT == 4, "a wave's four row tiles share one activation scale word");
  static_assert(NG == 2 || NG == 4, "a wave's column groups sit in one weight scale word");
  static_assert(SMEM <= 160 * 1024, "the quantized rows and the output staging fit the LDS");
};

// One CTA's work: Mrows (1..BM) activation rows from `rows` (bf16 rows to quantize, or
// MXFP4 rows to copy), column tiles bn0 .. bn0 + J - 1 of the prepared weight Wp, output
// rows at Cout + r * N for r < Mrows; column tiles past bn_last are computed from re-read
// weights and not stored.
template <int WM, int WN, int MT, int NG, int T, int PF, int J, class Rows>
__device__ __forceinline__ void sweep_core(const Rows& rows, int Mrows, const uint8_t* __restrict__ Wp,
                                           uint16_t* __restrict__ Cout, int N, int bn0, int bn_last,
                                           uint8_t* smem) {
  using S = SweepShape<WM, WN, MT, NG, T, PF>;
  constexpr int MTC = S::MTC, BM = S::BM, NW = S::NW, NTH = S::NTH, R = S::R, BN = S::BN;
  constexpr int K = T * kStepK;
  uint8_t* const aq = smem;
  uint8_t* const as = smem + S::AQ;
  uint8_t* const cs0 = smem + S::AQ + S::AS;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w / WN, wn = w % WN;

  // Weight operands of flattened step u = j T + t (column tile bn0 + j, step t): NG 1 KiB
  // payload tiles and the scale word of their column-group quad. The wave's groups start
  // at byte (wn NG) % 4 of that word; the shift that brings them to byte 0 is applied
  // where the word is used, so no arithmetic waits on a load in flight.
  const uint8_t* __restrict__ Wsc = Wp + payload_bytes(N, K);
  const int sshift = 8 * ((wn * NG) & 3);
  uint4 wq[R][NG];
  uint32_t wsw[R];
  auto load_w = [&](int u, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
    const int bn = min(bn0 + u / T, bn_last), t = u % T;
    const int gw0 = bn * (BN / 16) + wn * NG;
    const uint8_t* p = Wp + ((size_t)gw0 * T + t) * 1024 + lane * 16;
#pragma unroll
    for (int g = 0; g < NG; ++g) wq[SL][g] = *reinterpret_cast<const uint4*>(p + (size_t)g * T * 1024);
    wsw[SL] = *reinterpret_cast<const uint32_t*>(Wsc + ((size_t)(gw0 >> 2) * T + t) * 256 + lane * 4);
  };

  static_for<PF>([&](auto p) { load_w((int)decltype(p)::value, p); });

  // Quantize: item i = (step t, 16-row tile) = (i / MTC, i % MTC); lane 4r + j takes the
  // 32-block j of row r of that tile at that step. All of a wave's loads are issued before
  // the first block is quantized. Rows past Mrows re-read the last valid row and are never
  // stored.
  auto swz = [](int rr) { return ((rr >> 1) ^ (rr >> 2)) & 3; };  // tile_core's operand swizzle
  {
    const uint32_t st_off = (uint32_t)(((lane >> 2) * 4 + ((lane & 3) ^ swz(lane >> 2))) * 16);
    const uint32_t st_sc = (uint32_t)(((lane >> 2) + 16 * (lane & 3)) * MTC);
    // a lane's block per item: 16 bf16 words, or (already quantized) 4 payload words and the
    // scale byte
    constexpr int AW = Rows::kMx ? 5 : 16;
    uint32_t x[S::IPW][AW];
#pragma unroll
    for (int k = 0; k < S::IPW; ++k) {
      const int it = w + NW * k, t = it / MTC, tile = it % MTC;
      const int r = min(16 * tile + (lane >> 2), Mrows - 1);
      if constexpr (Rows::kMx) {
        const uint4 u = *reinterpret_cast<const uint4*>(rows.q + (size_t)r * (K / 2) + t * (kStepK / 2) + (lane & 3) * 16);
        x[k][0] = u.x; x[k][1] = u.y; x[k][2] = u.z; x[k][3] = u.w;
        x[k][4] = rows.s[(size_t)r * (K / kBlock) + t * (kStepK / kBlock) + (lane & 3)];
      } else {
        load_block_at(rows.base, (uint32_t)r * (uint32_t)(K * 2) + (uint32_t)(t * kStepK * 2 + (lane & 3) * 64), x[k]);
      }
    }
    // keep every load ahead of the first quantization (the scheduler would otherwise
    // interleave them and serialize their latencies)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < S::IPW; ++k) {
      const int it = w + NW * k, t = it / MTC, tile = it % MTC;
      uint32_t q[4];
      uint32_t sc;
      if constexpr (Rows::kMx) {
        q[0] = x[k][0]; q[1] = x[k][1]; q[2] = x[k][2]; q[3] = x[k][3];
        sc = x[k][4];
      } else {
        sc = quant_block(x[k], q);
      }
      *reinterpret_cast<uint4*>(aq + (t * MTC + tile) * 1024 + st_off) = make_uint4(q[0], q[1], q[2], q[3]);
      as[t * 64 * MTC + st_sc + tile] = (uint8_t)sc;
    }
  }
  __syncthreads();

  const uint32_t ld_off = (uint32_t)(((lane & 15) * 4 + ((lane >> 4) ^ swz(lane & 15))) * 16);
  // Every CTA runs all J column tiles: one past the last column tile (a partial last
  // chunk) is computed from re-read weights and not stored. A guard around the whole tile
  // would make the loads inside it join with their skipped paths and wait there.
  static_for<J>([&](auto j_c) {
    constexpr int j = decltype(j_c)::value;
    const int bn = bn0 + j;
    {
      v4f acc[NG][MT];
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[g][mt] = v4f{0.f, 0.f, 0.f, 0.f};
      static_for<T>([&](auto t_c) {
        constexpr int t = decltype(t_c)::value, u = j * T + t;
        // a step boundary the scheduler may not cross: it would sink each prefetch down to
        // its use, PF steps later, and wait on it there
        __builtin_amdgcn_sched_barrier(0);
        load_w(u + PF, std::integral_constant<int, (u + PF) % R>{});
        uint4 b[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          b[mt] = *reinterpret_cast<const uint4*>(aq + (t * MTC + wm * MT + mt) * 1024 + ld_off);
        const uint32_t sbw = *reinterpret_cast<const uint32_t*>(as + (t * 64 + lane) * MTC + wm * MT);
        const uint32_t sww = NG == 4 ? wsw[u % R] : wsw[u % R] >> sshift;
        static_for<NG>([&](auto g_c) {
          constexpr int g = decltype(g_c)::value;
          static_for<MT>([&](auto m_c) {
            constexpr int mt = decltype(m_c)::value;
            acc[g][mt] = mfma_fp4_sel<g, mt>(wq[u % R][g], b[mt], acc[g][mt], sww, sbw);
          });
        });
      });
      // Stage the tile as bf16 in buffer j % 2 (its previous contents, tile j - 2, were read
      // by every wave before the barrier that followed the staging of tile j - 1), then
      // store whole rows, 16 bytes per lane; the stores drain under the next tiles.
      uint8_t* const cs = cs0 + (j & 1) * S::CS;
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int r = 16 * (wm * MT + mt) + (lane & 15);
          const int cl = 16 * (wn * NG + g) + 4 * (lane >> 4);
          *reinterpret_cast<uint2*>(cs + r * S::CROW + cl * 2) =
              pack4_bf16(acc[g][mt][0], acc[g][mt][1], acc[g][mt][2], acc[g][mt][3]);
        }
      __syncthreads();
      constexpr int CPR = BN / 8, CPT = BM * CPR / NTH;
      static_assert((BM * CPR) % NTH == 0, "every thread stores the same number of chunks");
      u32x4 v[CPT];  // all of a thread's LDS reads before its first (row-guarded) store
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int id = threadIdx.x + i * NTH;
        v[i] = *reinterpret_cast<const u32x4*>(cs + (id / CPR) * S::CROW + (id % CPR) * 16);
      }
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int id = threadIdx.x + i * NTH;
        const int r = id / CPR, c16 = id % CPR;
        if (r < Mrows && bn <= bn_last)
          __builtin_nontemporal_store(v[i], reinterpret_cast<u32x4*>(Cout + (size_t)r * N + bn * BN + 8 * c16));
      }
    }
  });
}

template <int WM, int WN, int MT, int NG, int T, int PF, int J>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(2, 8)))
void k_gemm_sweep(const uint16_t* __restrict__ A, const uint8_t* __restrict__ Wp, uint16_t* __restrict__ C,
                  int M, int N, int GM) {
  using S = SweepShape<WM, WN, MT, NG, T, PF>;
  extern __shared__ __align__(16) uint8_t smem[];
  const int tiles_m = (M + S::BM - 1) / S::BM, tiles_n = N / S::BN, chunks = (tiles_n + J - 1) / J;
  int bm, ch;
  tile_coords(blockIdx.x, tiles_m * chunks, tiles_m, chunks, GM, bm, ch);
  const int m0 = bm * S::BM, bn0 = ch * J;
  const TileRowsDense rows{reinterpret_cast<const uint8_t*>(A) + (size_t)m0 * (T * kStepK) * 2, T * kStepK};
  sweep_core<WM, WN, MT, NG, T, PF, J>(rows, min(S::BM, M - m0), Wp, C + (size_t)m0 * N, N, bn0,
                                       min(bn0 + J, tiles_n) - 1, smem);
}

// ====================================================================== grouped MoE GEMM1, tiled
//
// For segments of tens of rows or more. Each expert's rows are cut into BM-row tiles and
// every (expert, column tile, row tile) unit is one CTA running the tiled main loop with
// its rows gathered by token index, so an expert's weight is streamed once per row tile
// (once in all for a segment of at most BM rows) rather than once per 16 or 32 rows. The
// grid is an upper bound on the units ((active experts + R_max / BM) x column tiles); each
// CTA ranks the experts' unit counts with a block scan to find its unit, and the surplus
// CTAs exit. One expert's units are consecutive and dealt to one XCD (as in tile_coords),
// so its column tiles share the gathered rows and its row tiles the weight in that L2.
// The unit (expert, row tile, column tile) of this CTA: the grid is an upper bound on the
// units; the CTA ranks the experts' unit counts with a wave-shuffle scan (s_scan: an int per wave, s_unit:
// 4 ints of LDS) and finds its own. False for a surplus CTA. Every value is CTA-uniform.
// Exclusive prefix sum, in thread order, of v over the CTA's NTH threads; `total` receives
// the CTA-wide sum. Each wave scans with lane shuffles (no barrier), then the wave totals
// meet in s_w (one int per wave) behind one barrier. Every thread must call it.
template <int NTH>
__device__ __forceinline__ int cta_exclusive_scan(int v, int* s_w, int& total) {
  constexpr int NW = NTH / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_w[w] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int t = s_w[i];
    before += i < w ? t : 0;
    total += t;
  }
  return before + x - v;
}

struct GroupedUnit {
  int e, r0, Mrows, bn;
};
template <int NTH, int BM>
__device__ __forceinline__ bool grouped_unit(const int32_t* __restrict__ offs, int E, int R_max, int tiles_n,
                                             int* s_scan, int* s_unit, GroupedUnit& unit) {
  const int tid = threadIdx.x;
  const int total = gridDim.x;
  const int L = (blockIdx.x % 8) * (total / 8) + min((int)(blockIdx.x % 8), total % 8) + blockIdx.x / 8;
  auto seg = [&](int e, int& lo, int& hi) {
    lo = min(max(offs[e], 0), R_max);
    hi = min(max(offs[e + 1], lo), R_max);
  };
  const int ept = (E + NTH - 1) / NTH;
  int local = 0;
  for (int i = 0; i < ept; ++i) {
    const int e = tid * ept + i;
    if (e < E) { int lo, hi; seg(e, lo, hi); local += (hi - lo + BM - 1) / BM * tiles_n; }
  }
  if (tid == 0) s_unit[0] = -1;
  int all_units;
  {
    int u = cta_exclusive_scan<NTH>(local, s_scan, all_units);  // units before this thread's experts
    if (L >= u && L < u + local) {
      for (int i = 0; i < ept; ++i) {
        const int e = tid * ept + i;
        if (e >= E) break;
        int lo, hi; seg(e, lo, hi);
        const int units = (hi - lo + BM - 1) / BM * tiles_n;
        if (L < u + units) { s_unit[0] = e; s_unit[1] = lo; s_unit[2] = hi - lo; s_unit[3] = u; break; }
        u += units;
      }
    }
  }
  __syncthreads();
  // uniform across the CTA: keep them (and every address derived from them) scalar
  const int e = __builtin_amdgcn_readfirstlane(s_unit[0]);
  if (e < 0) return false;  // surplus CTA: the grid over-counts the units
  const int lo = __builtin_amdgcn_readfirstlane(s_unit[1]), cnt = __builtin_amdgcn_readfirstlane(s_unit[2]);
  const int tiles_e = (cnt + BM - 1) / BM;
  const int rem = L - __builtin_amdgcn_readfirstlane(s_unit[3]), bn = rem / tiles_e, mt = rem % tiles_e;
  const int r0 = lo + mt * BM, Mrows = min(BM, cnt - mt * BM);
  unit = GroupedUnit{e, r0, Mrows, bn};
  return true;
}

// With ACT >= 0 the output is the fused activation + MXFP4 quantization (tile_core) into
// Hq [R_max, Nh/2] and Hs [R_max, Nh/32] instead of C.
template <int WM, int WN, int MT, int NG, int PF, int OCC, int ACT = -1>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(OCC, 8)))
void k_gemm_grouped_tile(const uint16_t* __restrict__ A, const int32_t* __restrict__ row_token,
                         const int32_t* __restrict__ offs, int E, int R_max, const uint8_t* __restrict__ Wall,
                         uint16_t* __restrict__ C, int Ttok, int N, int K, uint8_t* __restrict__ Hq,
                         uint8_t* __restrict__ Hs, int Nh) {
  using S = TileShape<WM, WN, MT, NG>;
  constexpr int NTH = S::NTH, BM = S::BM, BN = S::BN;
  __shared__ __align__(16) uint8_t smem[S::SMEM];
  __shared__ int s_scan[NTH];
  __shared__ int s_unit[4];  // expert, segment start, segment rows, its first unit
  const int tid = threadIdx.x;
  GroupedUnit u;
  if (!grouped_unit<NTH, BM>(offs, E, R_max, (N + BN - 1) / BN, s_scan, s_unit, u)) return;
  const int e = u.e, r0 = u.r0, Mrows = u.Mrows, bn = u.bn;
  uint16_t* Cout = ACT >= 0 ? nullptr : C + (size_t)r0 * N;
  ActOut ao;
  if constexpr (ACT >= 0) ao = ActOut{Hq + (size_t)r0 * (Nh / 2), Hs + (size_t)r0 * (Nh / 32), Nh};

  if (Ttok <= 0) {  // no activations at all: every row is Q(0) W^T = 0
    if constexpr (ACT >= 0) {  // and h = 0: zero codes, zero scales
      const int hc = ACT == kActSwiglu ? BN / 2 : BN, c0 = bn * hc;
      for (int i = tid; i < Mrows * (hc / 32); i += NTH) {
        const int r = i / (hc / 32), b = i % (hc / 32);
        *reinterpret_cast<uint4*>(ao.q + (size_t)r * (Nh / 2) + (c0 + 32 * b) / 2) = make_uint4(0u, 0u, 0u, 0u);
        ao.s[(size_t)r * (Nh / 32) + c0 / 32 + b] = 0;
      }
      return;
    }
    const int n0 = bn * BN, ncol = min(BN, N - n0);
    for (int i = tid; i < Mrows * (ncol / 8); i += NTH) {
      const int r = i / (ncol / 8), ch = i % (ncol / 8);
      *reinterpret_cast<uint4*>(Cout + (size_t)r * N + n0 + 8 * ch) = make_uint4(0u, 0u, 0u, 0u);
    }
    return;
  }
  const TileRowsGather rows{reinterpret_cast<const uint8_t*>(A), row_token + r0, Ttok, K};
  tile_core<WM, WN, MT, NG, PF, ACT>(rows, Mrows, Wall + (size_t)e * prepared_bytes(N, K), Cout, nullptr, N, K, bn,
                                     0, steps_of(K), smem, ao);
}

// The second MoE GEMM: the same units over already-quantized MXFP4 rows (expert-sorted,
// canonical payload Aq [R_max, K/2] and scales As [R_max, K/32]); bf16 rows of C.
template <int WM, int WN, int MT, int NG, int PF, int OCC>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(OCC, 8)))
void k_gemm_grouped_tile_mx(const uint8_t* __restrict__ Aq, const uint8_t* __restrict__ As,
                            const int32_t* __restrict__ offs, int E, int R_max, const uint8_t* __restrict__ Wall,
                            uint16_t* __restrict__ C, int N, int K) {
  using S = TileShape<WM, WN, MT, NG>;
  __shared__ __align__(16) uint8_t smem[S::SMEM];
  __shared__ int s_scan[S::NTH];
  __shared__ int s_unit[4];
  GroupedUnit u;
  if (!grouped_unit<S::NTH, S::BM>(offs, E, R_max, (N + S::BN - 1) / S::BN, s_scan, s_unit, u)) return;
  const TileRowsMx rows{Aq + (size_t)u.r0 * (K / 2), As + (size_t)u.r0 * (K / kBlock), K};
  tile_core<WM, WN, MT, NG, PF>(rows, u.Mrows, Wall + (size_t)u.e * prepared_bytes(N, K), C + (size_t)u.r0 * N,
                                nullptr, N, K, u.bn, 0, steps_of(K), smem);
}

// The second MoE GEMM at short K (at most eight 128-wide steps): the units are (expert,
// 128-row tile, chunk of J 128-column tiles); each CTA copies its MXFP4 rows into LDS once
// and sweeps its column tiles (sweep_core), so a unit's lookup, pipeline fill and epilogue
// are paid once per J column tiles and a tile's stores drain under the next tiles.
template <int T, int PF, int J>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 8)))
void k_gemm_grouped_sweep_mx(const uint8_t* __restrict__ Aq, const uint8_t* __restrict__ As,
                             const int32_t* __restrict__ offs, int E, int R_max, const uint8_t* __restrict__ Wall,
                             uint16_t* __restrict__ C, int N) {
  using S = SweepShape<2, 4, 4, 2, T, PF>;
  constexpr int K = T * kStepK;
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_scan[S::NTH];
  __shared__ int s_unit[4];
  const int tiles_n = N / S::BN, chunks = (tiles_n + J - 1) / J;
  GroupedUnit u;
  if (!grouped_unit<S::NTH, S::BM>(offs, E, R_max, chunks, s_scan, s_unit, u)) return;
  const int bn0 = u.bn * J;
  const TileRowsMx rows{Aq + (size_t)u.r0 * (K / 2), As + (size_t)u.r0 * (K / kBlock), K};
  sweep_core<2, 4, 4, 2, T, PF, J>(rows, u.Mrows, Wall + (size_t)u.e * prepared_bytes(N, K), C + (size_t)u.r0 * N,
                                   N, bn0, min(bn0 + J, tiles_n) - 1, smem);
}

// Top-k weighted combine: out[t, n] = sum_k w[t, k] * y[rows[t, k], n] in FP32 in k order,
// rounded once to bf16; a row index outside [0, R) contributes nothing. One thread per token
// and 8 columns (16-byte loads and store).
__global__ __launch_bounds__(256) void k_moe_combine(const uint16_t* __restrict__ y, int R,
                                                     const int32_t* __restrict__ rows,
                                                     const float* __restrict__ wts, int T, int topk, int N,
                                                     uint16_t* __restrict__ out) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cpr = N / 8;
  if (id >= (int64_t)T * cpr) return;
  const int t = (int)(id / cpr), c = (int)(id % cpr) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < topk; ++k) {
    const int r = rows[(size_t)t * topk + k];
    if (r < 0 || r >= R) continue;
    const float wk = wts[(size_t)t * topk + k];
    const uint4 v = *reinterpret_cast<const uint4*>(y + (size_t)r * N + c);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += wk * __builtin_bit_cast(float, u[i] << 16);
      acc[2 * i + 1] += wk * __builtin_bit_cast(float, u[i] & 0xffff0000u);
    }
  }
  const uint2 lo = pack4_bf16(acc[0], acc[1], acc[2], acc[3]), hi = pack4_bf16(acc[4], acc[5], acc[6], acc[7]);
  *reinterpret_cast<uint4*>(out + (size_t)t * N + c) = make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// ====================================================================== grouped MoE GEMM1
//
// Expert-segmented A4W4 GEMM: output row r (expert-sorted) = Q(A[row_token[r]]) Q(W_e)^T.
// Work item = (a, c): the a-th expert with at least one row, and NG column groups. Grid size
// is min(E, R_max) * (N / (16 NG)); each CTA finds its expert by a block-wide scan of the
// segment table, so no host sync or workspace is needed and empty experts cost nothing.
// Inside, the streaming scheme (StreamCTA): WK waves split K, each keeping its share of the
// expert's weight columns in registers while the CTA walks the expert's rows in chunks of
// 16 * MT, gathering each chunk's rows by token index into the quantizer.
// Malformed tables are clamped (segments to [0, R_max], tokens outside [0, T) read as zero
// rows), so every access stays in bounds.
template <int MT, int NG, int WK, int PD, int QB, bool RES>
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
  if (tid == 0) s_e = -1;
  int all_active;
  {
    int rank = cta_exclusive_scan<NTH>(local, s_scan, all_active);  // active segments before this thread's range
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
  const int lane = tid & 63;
  const int g0 = c * NG;

  if (Ttok <= 0) {  // no activations at all: every row is Q(0) W^T = 0
    for (int i = tid; i < cnt * 4 * NG; i += NTH) {
      const int r = i / (4 * NG), q = i % (4 * NG);
      *reinterpret_cast<uint2*>(C + (size_t)(lo + r) * N + 16 * g0 + 4 * q) = make_uint2(0u, 0u);
    }
    return;
  }

  const int T = steps_of(K);
  const uint8_t* __restrict__ Wp = Wall + (size_t)e * prepared_bytes(N, K);
  StreamCTA<MT, NG, WK, PD, QB> cta;
  cta.init(Wp, N, K, g0, 0, T, T, 16 * MT, smem);
  // RES: every wave's whole K share fits in its PD weight registers (checked by the host),
  // so the weight is loaded once and reused for every row chunk.

  for (int r0 = 0; r0 < cnt; r0 += CH) {
    const int Mc = min(CH, cnt - r0);
    __syncthreads();  // the previous chunk is done with LDS
    const GatherRows rows{A, row_token, lo + r0, Ttok, K};
    cta.quant(rows, Mc, [&] { if ((!RES || r0 == 0) && cta.S > 0) cta.load_w(cta.t0); });
    __syncthreads();
    v4f acc[NG][MT];
    cta.mma(Mc, RES, acc);
    __syncthreads();  // every wave is done with the activation region
    cta.reduce_store(acc, smem, [&](int g, int mt, const v4f& v) {
      const int m = 16 * mt + (lane & 15);
      const int n = 16 * (g0 + g) + 4 * (lane >> 4);
      if (m < Mc)
        *reinterpret_cast<uint2*>(C + (size_t)(lo + r0 + m) * N + n) = pack4_bf16(v[0], v[1], v[2], v[3]);
    });
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
  return launch_prepare_rows(w, N, N, K, wp, st);
}

hipError_t launch_prepare_rows(const void* w, int64_t valid, int64_t N, int64_t K, void* wp, hipStream_t st) {
  const int64_t n = (N / 16) * steps_of((int)K) * 64;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_prepare, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(w), static_cast<uint8_t*>(wp), (int)N, (int)K, (int)valid);
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* P, void* c, int64_t M, int64_t N, int S, hipStream_t st) {
  const int64_t MN = M * N;
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((MN / 4 + 255) / 256)), dim3(256), 0, st, P,
                     static_cast<uint16_t*>(c), MN, S);
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

constexpr size_t kMaxLds = 160 * 1024;  // LDS per CU (and per workgroup) on gfx950

// Raise a kernel's dynamic-LDS limit to what the 160 KiB leave beside its static LDS, once
// per device. `done` is the caller's per-kernel bitmask of devices already configured.
hipError_t ensure_lds_limit(const void* kern, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  hipFuncAttributes attr{};
  e = hipFuncGetAttributes(&attr, kern);
  if (e != hipSuccess) return e;
  if (attr.sharedSizeBytes > kMaxLds) return hipErrorInvalidValue;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kMaxLds - attr.sharedSizeBytes));
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// LDS of a StreamCTA staging M rows of a slice of TS steps: quantized rows, their scales, or
// the cross-wave reduction, whichever is larger.
size_t stream_lds_bytes(int M, int TS, int MT, int NG, int WK) {
  const size_t act = (size_t)M * (TS * 64 + 16) + (size_t)M * 4 * TS;
  const size_t red = (size_t)WK * NG * MT * 64 * 16;
  return act > red ? act : red;
}

// ---------------------------------------------------------------- configurations
struct GemmConfig {
  bool tile = false;
  int MT = 1, NG = 1, WK = 4, S = 1;     // streaming kernel (S = K slices)
  int WM = 1, WN = 4, PF = 2, GM = 8;    // tiled kernel (uses MT, NG too)
  int OCC = 1;                           // tiled kernel: minimum waves per SIMD asked of the compiler
  bool sweep = false;                    // short-K sweep kernel (uses J, GM)
  int J = 1;                             // sweep kernel: column tiles per CTA
  bool qo = false;                       // quantize-once path (uses WM, WN, MT, NG, NBUF, OCC, GM)
  int NBUF = 4;                          // quantize-once kernel: LDS stage buffers (register-direct: steps ahead)
  bool qr = false;                       // quantize-once, register-direct kernel (qo too; uses MT, NG, NBUF, GM, S)
  bool qk = false;                       // the same, four waves per tile splitting K (qo too; MT, NG, NBUF, GM, S)
};

#define MX_STREAM_CONFIGS(X) \
  X(1, 1, 2) X(1, 1, 4) X(1, 1, 8) X(1, 2, 4) X(1, 2, 8) X(1, 4, 4) X(1, 4, 8) \
  X(2, 1, 2) X(2, 1, 4) X(2, 1, 8) X(2, 2, 4) X(2, 2, 8) X(2, 4, 4) X(2, 4, 8) \
  X(4, 1, 4) X(4, 1, 8) X(4, 2, 4) X(4, 4, 4) X(8, 1, 4) X(8, 2, 4)

// short-K sweep kernel: (K steps T, weight prefetch depth PF in steps, column tiles per CTA
// J); the CTA is 8 waves of 64 x 32 (128-row tiles, 128-column tiles)
#define MX_SWEEP_CONFIGS(X) \
  X(2, 3, 2) X(2, 3, 4) X(4, 6, 2) X(4, 6, 4) X(6, 9, 2) X(6, 9, 4) X(8, 10, 2) X(8, 10, 4)

#define MX_TILE_CONFIGS(X) \
  X(1, 4, 4, 4, 2, 1) X(2, 4, 4, 4, 2, 1) X(1, 4, 8, 4, 1, 1) X(2, 2, 4, 8, 1, 1) X(1, 4, 4, 2, 2, 1) \
  X(1, 4, 4, 4, 1, 2) X(1, 4, 4, 4, 2, 2) X(2, 4, 4, 4, 1, 1) X(1, 4, 4, 2, 2, 2) X(1, 8, 8, 4, 1, 2) \
  X(1, 4, 4, 1, 2, 1) X(1, 4, 4, 1, 2, 2)

// Weight prefetch depth: enough registers for a wave's whole K share when it fits (4, 8 or
// 16 steps of NG operands, at most `ops` operands: kSkinnyPD for the grouped kernels,
// kStreamPD for the dense streaming one), so no registers go to duplicate loads. This is
// the PD the streaming and grouped launchers instantiate.
int pick_pd(int NG, int steps_per_wave, int ops = kSkinnyPD) {
  const int cap = std::min(16, ops / NG);
  int pd = 4;
  while (pd < steps_per_wave && pd < cap) pd *= 2;
  return pd > cap ? cap : pd;
}

// Activation quant batch of the streaming kernel: one batch when a wave's blocks fit one
// per lane, otherwise four blocks per lane in flight per batch.
int stream_qb(int M, int steps_per_wave) { return M * 4 * steps_per_wave <= 64 ? 1 : 4; }

template <int MT, int NG, int WK, int PD, int QB>
hipError_t launch_stream(const void* a, const void* wp, void* c, float* P, int M, int N, int K, int S,
                         int TS, size_t lds, hipStream_t st) {
  auto kern = k_gemm_stream<MT, NG, WK, PD, QB>;
  static std::atomic<uint64_t> configured{0};
  if (lds > 65536) {
    hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), configured);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(N / (16 * NG)), (unsigned)S), dim3(64 * WK), lds, st,
                     static_cast<const uint16_t*>(a), static_cast<const uint8_t*>(wp),
                     static_cast<uint16_t*>(c), P, M, N, K, TS);
  return hipGetLastError();
}

template <int MT, int NG, int WK, int QB>
hipError_t launch_stream_pd(int pd, const void* a, const void* wp, void* c, float* P, int M, int N, int K,
                            int S, int TS, size_t lds, hipStream_t st) {
  if constexpr (kStreamPD / NG >= 16)
    if (pd >= 16) return launch_stream<MT, NG, WK, 16, QB>(a, wp, c, P, M, N, K, S, TS, lds, st);
  if constexpr (kStreamPD / NG >= 8)
    if (pd >= 8) return launch_stream<MT, NG, WK, 8, QB>(a, wp, c, P, M, N, K, S, TS, lds, st);
  return launch_stream<MT, NG, WK, 4, QB>(a, wp, c, P, M, N, K, S, TS, lds, st);
}

template <int MT, int NG, int WK>
hipError_t run_stream(const void* a, const void* wp, void* c, float* P, int M, int N, int K, int S,
                      hipStream_t st) {
  const int T = steps_of(K);
  const int TS = (T + S - 1) / S;
  const size_t lds = stream_lds_bytes(min(M, 16 * MT), TS, MT, NG, WK);
  if (lds > kMaxLds) return hipErrorInvalidValue;
  const int per = (TS + WK - 1) / WK;
  const int pd = pick_pd(NG, per, kStreamPD);
  hipError_t e = stream_qb(M, per) == 1 ? launch_stream_pd<MT, NG, WK, 1>(pd, a, wp, c, P, M, N, K, S, TS, lds, st)
                                        : launch_stream_pd<MT, NG, WK, 4>(pd, a, wp, c, P, M, N, K, S, TS, lds, st);
  if (e != hipSuccess || S == 1) return e;
  return launch_splitk_reduce(P, c, M, N, S, st);
}

template <int WM, int WN, int MT, int NG, int PF, int OCC>
hipError_t run_tile(const void* a, const void* wp, void* c, float* P, int M, int N, int K, int GM, int S,
                    hipStream_t st) {
  constexpr int BM = 16 * MT * WM, BN = 16 * NG * WN;
  const int64_t grid = ((int64_t)M + BM - 1) / BM * ((N + BN - 1) / BN);
  const int T = steps_of(K);
  if (!P) S = 1;
  const int TS = (T + S - 1) / S;
  S = (T + TS - 1) / TS;  // no empty slices
  hipLaunchKernelGGL((k_gemm_tile<WM, WN, MT, NG, PF, OCC>), dim3((unsigned)grid, (unsigned)S), dim3(64 * WM * WN),
                     0, st, static_cast<const uint16_t*>(a), static_cast<const uint8_t*>(wp),
                     static_cast<uint16_t*>(c), S > 1 ? P : nullptr, M, N, K, GM, TS);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  return launch_splitk_reduce(P, c, M, N, S, st);
}

template <int T, int PF, int J>
hipError_t run_sweep(const void* a, const void* wp, void* c, int M, int N, int K, int GM, hipStream_t st) {
  using S = SweepShape<2, 4, 4, 2, T, PF>;
  if (K != T * kStepK || N % S::BN != 0) return hipErrorInvalidValue;
  auto kern = k_gemm_sweep<2, 4, 4, 2, T, PF, J>;
  static std::atomic<uint64_t> configured{0};
  hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), configured);
  if (e != hipSuccess) return e;
  const int64_t grid = ((int64_t)M + S::BM - 1) / S::BM * ((N / S::BN + J - 1) / J);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(S::NTH), S::SMEM, st, static_cast<const uint16_t*>(a),
                     static_cast<const uint8_t*>(wp), static_cast<uint16_t*>(c), M, N, GM);
  return hipGetLastError();
}

bool sweep_supported(int T, int J) {
#define X(t, pf, j) if (T == t && J == j) return true;
  MX_SWEEP_CONFIGS(X)
#undef X
  return false;
}

int sweep_pf(int T) {
#define X(t, pf, j) if (T == t) return pf;
  MX_SWEEP_CONFIGS(X)
#undef X
  return 0;
}

bool stream_supported(int MT, int NG, int WK) {
#define X(mt, ng, wk) if (MT == mt && NG == ng && WK == wk) return true;
  MX_STREAM_CONFIGS(X)
#undef X
  return false;
}

bool tile_supported(const GemmConfig& c) {
#define X(wm, wn, mt, ng, pf, occ) \
  if (c.WM == wm && c.WN == wn && c.MT == mt && c.NG == ng && c.PF == pf && c.OCC == occ) return true;
  MX_TILE_CONFIGS(X)
#undef X
  return false;
}

hipError_t run_config(const GemmConfig& c, const void* a, const void* wp, void* out, float* P, int M,
                      int N, int K, hipStream_t st) {
  if (c.qr) return launch_gemm_qr(c.MT, c.NG, c.NBUF, c.S, a, wp, out, M, N, K, c.GM, P, st);
  if (c.qk) return launch_gemm_qk(c.MT, c.NG, c.NBUF, c.S, a, wp, out, M, N, K, c.GM, P, st);
  if (c.qo) return launch_gemm_qo(c.WM, c.WN, c.MT, c.NG, c.NBUF, c.OCC, a, wp, out, M, N, K, c.GM, P, st);
  if (c.sweep) {
    const int T = steps_of(K);
#define X(t, pf, j) if (T == t && c.J == j) return run_sweep<t, pf, j>(a, wp, out, M, N, K, c.GM, st);
    MX_SWEEP_CONFIGS(X)
#undef X
    return hipErrorInvalidValue;
  }
  if (!c.tile) {
#define X(mt, ng, wk) \
  if (c.MT == mt && c.NG == ng && c.WK == wk) return run_stream<mt, ng, wk>(a, wp, out, P, M, N, K, c.S, st);
    MX_STREAM_CONFIGS(X)
#undef X
  } else {
#define X(wm, wn, mt, ng, pf, occ) \
  if (c.WM == wm && c.WN == wn && c.MT == mt && c.NG == ng && c.PF == pf && c.OCC == occ) \
    return run_tile<wm, wn, mt, ng, pf, occ>(a, wp, out, P, M, N, K, c.GM, c.S, st);
    MX_TILE_CONFIGS(X)
#undef X
  }
  return hipErrorInvalidValue;
}

int round_up_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Default configuration for a shape, given the workspace the caller offers. The rules come
// from sweeping every compiled configuration over the microbenchmark shapes on MI355X
// (rotating buffer sets larger than the Infinity Cache).
GemmConfig select_config(int M, int N, int K, size_t ws_bytes) {
  GemmConfig c;
  const int T = steps_of(K), G = N / 16;
  auto stream_fits = [&](const GemmConfig& s) {
    const int TS = (T + s.S - 1) / s.S;
    const size_t need = s.S > 1 ? (size_t)s.S * M * N * 4 : 0;
    return need <= ws_bytes && stream_lds_bytes(std::min(M, 16 * s.MT), TS, s.MT, s.NG, s.WK) <= kMaxLds &&
           G % s.NG == 0;
  };
  // long K: the tiled kernel with K slices when the caller offers room for the partials
  const bool split_ok = T >= 16 && (size_t)2 * M * N * 4 <= ws_bytes;
  // 17..32 rows against many column groups and long K (8448 x 7168): 64 x 256 tiles over K
  // slices beat the streaming kernel, whose 132 CTAs leave half the chip idle (16.4 against
  // 19.5 us, cold). The most slices (4 .. 8) whose CTAs still fit one per CU: at 8448 x 7168
  // M=32, 33 tiles x 7 slices of 8 steps, 16.1 -> 14.2 us against four slices (five: 15.7,
  // six: 15.0; eight, 264 CTAs: 18.7 us).
  if (M > 16 && M <= 32 && G >= 512 && T >= 32) {
    const int64_t tiles = (N + 255) / 256;
    int sk = (int)std::max<int64_t>(4, std::min<int64_t>(8, 256 / tiles));
    sk = std::min(sk, T / 6);
    while (sk > 4 && (size_t)sk * M * N * 4 > ws_bytes) --sk;
    if ((size_t)sk * M * N * 4 <= ws_bytes) {
      c.tile = true; c.WM = 1; c.WN = 4; c.MT = 4; c.NG = 4; c.PF = 2; c.GM = 8; c.OCC = 2; c.S = sk;
      return c;
    }
  }
  if (M <= 32 || (M <= 128 && G <= 96 && !split_ok)) {
    // weight-streaming kernel: the weight is read once, straight into registers
    GemmConfig s;
    s.tile = false;
    s.MT = round_up_pow2((M + 15) / 16);
    // long K: eight waves share a CTA's K range, more weight bytes in flight per column
    const bool longk = T >= 16;
    if (M <= 4) {
      s.NG = (G >= 256 && G < 512) ? 2 : 1;
      s.WK = longk ? 8 : 4;
    } else if (M <= 16) {
      // four column groups share each scale word the CTA loads (one scale request per four
      // weight requests instead of one per request)
      s.NG = G >= 512 ? 4 : (G >= 256 ? 2 : 1);
      s.WK = longk ? 8 : 4;
    } else if (M <= 32) {
      s.WK = longk ? 8 : 4;
      if (G >= 512) {
        s.NG = 4;
      } else if (G >= 256 && longk && (size_t)2 * M * N * 4 <= ws_bytes) {
        s.NG = 4;
        s.S = 2;
      } else {
        s.NG = 2;
      }
    } else {
      s.NG = 2;
      s.WK = 4;
    }
    // few column groups (N = 1536): split K so the grid covers the chip
    if (G <= 96) s.S = M <= 16 ? 1 : 4;
    while (!stream_fits(s) && s.S < T && (size_t)(2 * s.S) * M * N * 4 <= ws_bytes) s.S *= 2;
    if (!stream_fits(s)) s.S = 1;
    if (stream_fits(s)) return s;
  }
  // tiled kernel: 64 x 256 tiles when there are enough of them (two steps of prefetch only
  // for long K at moderate sizes), else 64 x 128 tiles at one CTA per SIMD set
  c.tile = true;
  // Many rows and long K: quantize the activations once into the workspace and multiply the
  // two prepared operands (k_gemm_qo), when the caller offers that workspace and the 128 x 128
  // tiles number at least 150. 256 x 256 tiles when one round of them nearly fills the chip
  // (N=7168, K=4224, M=2048: 224 tiles), 128 x 128 otherwise. Measured against the inline
  // kernels (cold buffers): 8448 x 7168 M=2048 141 -> 95 us, M=512 55 -> 35 us; 7168 x 4224
  // M=2048 61 -> 44 us, M=512 26 -> 22 us; 1536 x 7168 M=2048 39 -> 32 us. At M=512 with
  // N=1536 (48 tiles) the inline kernel with K slices stays ahead (21 against 28 us).
  const int64_t t256 = ((int64_t)M + 255) / 256 * ((N + 255) / 256);
  const int64_t t128 = ((int64_t)M + 127) / 128 * ((N + 127) / 128);
  // Slightly more 128 x 128 tiles than one wave per SIMD of the chip (8448 x 7168 at M=2048:
  // 1056): the register-direct kernel on 72-accumulator tiles that fit one round: 128 x 144
  // (944 tiles there: 80.0 -> 68.8 us against 128 x 128 with the tail), else 144 x 128
  // (990 tiles there: 75.8 us); else 128 x 128 with the tiles past one round in four K
  // slices (90 -> 86 us there; with the whole last round 96 us, eight slices 93 us).
  const int64_t tm128 = ((int64_t)M + 127) / 128;
  if (T >= 16 && t128 > 1024 && tm128 * ((N + 143) / 144) <= 1024 && qr_workspace_bytes(M, N, K, 8, 9, 1) <= ws_bytes) {
    c.qo = true; c.qr = true; c.MT = 8; c.NG = 9; c.NBUF = 1; c.GM = 8; c.S = 1;
    return c;
  }
  if (T >= 16 && t128 > 1024 && ((int64_t)M + 143) / 144 * ((N + 127) / 128) <= 1024 &&
      qr_workspace_bytes(M, N, K, 9, 8, 1) <= ws_bytes) {
    c.qo = true; c.qr = true; c.MT = 9; c.NG = 8; c.NBUF = 1; c.GM = 8; c.S = 1;
    return c;
  }
  if (T >= 16 && qr_tail_tiles(M, N, 8, 8) > 0 && qr_workspace_bytes(M, N, K, 8, 8, 4) <= ws_bytes) {
    c.qo = true; c.qr = true; c.MT = 8; c.NG = 8; c.NBUF = 2; c.GM = 8; c.S = 4;
    return c;
  }
  // Too few 128 x 128 tiles for one wave per SIMD but enough for one CTA per CU, at long K:
  // four register-direct waves per tile splitting K, the tile width 16 NG (NG = 6 .. 9) the
  // narrowest whose tiles fit one round of 256 CTAs, when that round holds at least 150.
  // 1536 x 7168 M=2048: 256 tiles of 128 x 96, 28.3 -> 26.0 us (32.2 us on the LDS kernel);
  // 8448 x 7168 M=512: 236 tiles of 128 x 144, 34.3 -> 28.7 us (128 x 128: 264 tiles, two
  // rounds, 40.0 us). At K = 4224 (7168 x 4224 M=512, 256 tiles of 128 x 112) it only ties
  // the LDS kernel.
  // Few 128-row tiles at long K: 128 x 48 tiles, four K quarters per CTA, four steps ahead,
  // no K slices across CTAs, when they number 128 .. 256 (one CTA per CU at most). 8448 x 7168
  // M=128 (176 CTAs): 23.2 -> 19.2 us against the inline 64 x 256 tile over three K slices
  // (128 x 32 tiles, 264 CTAs: 27.6 us); 7168 x 4224 M=128 (150): 16.3 -> 14.9 us against the
  // inline 64 x 64 tile; 1536 x 7168 M=512 (128): 20.0 -> 19.4 us against the inline tile over
  // four K slices. At K = 768 (7168 x 768 M=128 and 512) the inline kernels stay well ahead.
  const int64_t t48 = tm128 * ((N + 47) / 48);
  if (M > 96 && T >= 32 && t48 >= 128 && t48 <= 256 && qk_workspace_bytes(M, N, K, 1) <= ws_bytes) {
    c.qo = true; c.qk = true; c.MT = 8; c.NG = 3; c.NBUF = 4; c.GM = (int)(tm128 < 4 ? tm128 : 4); c.S = 1;
    return c;
  }
  if (M >= 512 && T >= 48 && qk_workspace_bytes(M, N, K, 1) <= ws_bytes) {
    for (int ng = 6; ng <= 9; ++ng) {
      const int64_t tiles = tm128 * ((N + 16 * ng - 1) / (16 * ng));
      if (tiles > 256) continue;
      if (tiles < 150) break;
      c.qo = true; c.qk = true; c.MT = 8; c.NG = ng; c.NBUF = ng == 9 ? 1 : 2; c.GM = 4; c.S = 1;
      return c;
    }
  }
  if (M >= 512 && T >= 16 && t128 >= 150 && qo_act_bytes(M, K) <= ws_bytes) {
    c.qo = true; c.GM = 8; c.OCC = 2;
    if (t256 >= 200 && t256 <= 256) { c.WM = 2; c.WN = 4; c.MT = 8; c.NG = 4; c.NBUF = 4; }
    else { c.WM = 2; c.WN = 2; c.MT = 4; c.NG = 4; c.NBUF = 4; }
    return c;
  }
  // short K and enough rows: each 128-row tile quantized once and swept over four 128-column
  // tiles, when that still gives about 200 CTAs or more (N=7168, K=768, M=2048: 224)
  const int64_t sweeps = ((int64_t)M + 127) / 128 * ((N / 128 + 3) / 4);
  if (sweep_supported(T, 4) && sweeps >= 200) {
    c.sweep = true; c.J = 4; c.GM = 8;
    return c;
  }
  // 128 x 512 tiles (eight waves of 128 x 64) halve the load instructions per output; they
  // pay when one round of them (at most one per CU) nearly fills the chip
  const int64_t tiles512 = ((int64_t)M + 127) / 128 * (N / 512);
  if (N % 512 == 0 && tiles512 >= 160 && tiles512 <= 256) {
    c.WM = 1; c.WN = 8; c.MT = 8; c.NG = 4; c.PF = 1; c.GM = 8; c.OCC = 2;
    return c;
  }
  c.WM = 1; c.WN = 4; c.MT = 4;
  const int64_t tiles256 = ((int64_t)M + 63) / 64 * ((N + 255) / 256);
  const int64_t tiles128 = ((int64_t)M + 63) / 64 * ((N + 127) / 128);
  if (tiles256 >= 150) {
    c.NG = 4; c.GM = 8; c.OCC = 2;
    c.PF = K <= 1024 || G >= 512 || (M >= 1024 && G >= 256) ? 1 : 2;
    return c;
  }
  // few 256-wide tiles but about 200 or more 64 x 64 ones (N=7168 at M=65..128): narrow
  // tiles at two CTAs per CU fill the chip without K slices or their reduce, as long as the
  // bf16 activation rows that every 64-column tile re-reads through L2 stay modest (at most
  // 160 MB in all: 22 MB at 7168 x 768 and 121 MB at 7168 x 4224 for M = 128 gained 13% and
  // 6%; 242 MB at 8448 x 7168 took 41 us against 22.6 us for K slices)
  const int64_t tiles64 = ((int64_t)M + 63) / 64 * (N / 64);
  const int64_t reread = (int64_t)(N / 64) * (((int64_t)M + 63) / 64 * 64) * K * 2;
  if (tiles64 >= 200 && reread <= (int64_t)160 << 20) {
    c.NG = 1; c.PF = 2; c.GM = 8; c.OCC = 2;
    return c;
  }
  if (split_ok) {
    // Few tiles at long K: split K into S slices (at least 6 steps each) so that about 200
    // CTAs run, one per CU or fewer; FP32 partials go to the workspace and k_splitk_reduce
    // adds them in slice order. 64 x 256 tiles unless even eight slices of them are too few.
    const int64_t tiles = tiles256 * 8 >= 150 ? tiles256 : tiles128;
    if (tiles == tiles256) { c.NG = 4; c.PF = 2; c.GM = 8; c.OCC = 2; }
    else { c.NG = 2; c.PF = 2; c.GM = 8; c.OCC = 2; }
    int sk = (int)std::min<int64_t>(8, (200 + tiles / 2) / tiles);
    sk = std::max(1, std::min(sk, T / 6));
    while (sk > 1 && (size_t)sk * M * N * 4 > ws_bytes) --sk;
    c.S = sk;
    return c;
  }
  c.NG = 2; c.PF = 2; c.GM = 16; c.OCC = 1;
  return c;
}

// Tuning only: MX_GEMM_CONFIG="s,MT,NG,WK,S" (streaming), "t,WM,WN,MT,NG,PF,GM[,OCC[,S]]" (tiled,
// S = K slices), "k,J,GM" (short-K sweep, J column tiles per CTA), "q,WM,WN,MT,NG,NBUF,OCC,GM"
// (quantize-once: k_prepare of the activations into the workspace, then k_gemm_qo), "r,MT,NG,D,GM[,S]"
// (the same with the register-direct k_gemm_qr, operands D steps ahead, tail tiles in S K slices),
// "x,MT,NG,D,GM[,S]" (four register-direct waves per tile splitting K, k_gemm_qk, S K slices)
// replaces the default choice. Returns 0 when unset, 1 when applied, -1 when the string
// does not name a compiled configuration (the call then fails rather than silently
// running something else).
int override_config(GemmConfig& c) {
  const char* e = std::getenv("MX_GEMM_CONFIG");
  if (!e || !*e) return 0;
  GemmConfig o;
  int v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (e[0] == 's' && std::sscanf(e, "s,%d,%d,%d,%d", &v[0], &v[1], &v[2], &v[3]) == 4) {
    o.tile = false; o.MT = v[0]; o.NG = v[1]; o.WK = v[2]; o.S = v[3];
    if (!stream_supported(o.MT, o.NG, o.WK) || o.S < 1) return -1;
  } else if (e[0] == 'q' && std::sscanf(e, "q,%d,%d,%d,%d,%d,%d,%d", &v[0], &v[1], &v[2], &v[3], &v[4], &v[5],
                                         &v[6]) == 7) {
    o.tile = true; o.qo = true; o.WM = v[0]; o.WN = v[1]; o.MT = v[2]; o.NG = v[3]; o.NBUF = v[4]; o.OCC = v[5];
    o.GM = v[6] < 1 ? 1 : v[6];
    if (!qo_supported(o.WM, o.WN, o.MT, o.NG, o.NBUF, o.OCC)) return -1;
  } else if (e[0] == 'r' && std::sscanf(e, "r,%d,%d,%d,%d,%d", &v[0], &v[1], &v[2], &v[3], &v[4]) >= 4) {
    o.tile = true; o.qo = true; o.qr = true; o.MT = v[0]; o.NG = v[1]; o.NBUF = v[2]; o.GM = v[3] < 1 ? 1 : v[3];
    o.S = v[4] < 1 ? 1 : v[4];
    if (!qr_supported(o.MT, o.NG, o.NBUF) || o.S > 16) return -1;
  } else if (e[0] == 'x' && std::sscanf(e, "x,%d,%d,%d,%d,%d", &v[0], &v[1], &v[2], &v[3], &v[4]) >= 4) {
    o.tile = true; o.qo = true; o.qk = true; o.MT = v[0]; o.NG = v[1]; o.NBUF = v[2]; o.GM = v[3] < 1 ? 1 : v[3];
    o.S = v[4] < 1 ? 1 : v[4];
    if (!qk_supported(o.MT, o.NG, o.NBUF) || o.S > 16) return -1;
  } else if (e[0] == 'k' && std::sscanf(e, "k,%d,%d", &v[0], &v[1]) == 2) {
    o.tile = true; o.sweep = true; o.J = v[0]; o.GM = v[1] < 1 ? 1 : v[1];
  } else if (e[0] == 't' && std::sscanf(e, "t,%d,%d,%d,%d,%d,%d,%d,%d", &v[0], &v[1], &v[2], &v[3], &v[4], &v[5],
                                         &v[6], &v[7]) >= 6) {
    o.tile = true; o.WM = v[0]; o.WN = v[1]; o.MT = v[2]; o.NG = v[3]; o.PF = v[4]; o.GM = v[5] < 1 ? 1 : v[5];
    o.OCC = v[6] < 1 ? 1 : v[6];
    o.S = v[7] < 1 ? 1 : v[7];
    if (!tile_supported(o)) return -1;
  } else {
    return -1;
  }
  c = o;
  return 1;
}

}  // namespace

// Workspace a configuration needs: split-K partials, or the quantized activations of the
// quantize-once kernel.
size_t config_workspace(const GemmConfig& c, int64_t M, int64_t N, int64_t K) {
  if (c.qr) return qr_workspace_bytes(M, N, K, c.MT, c.NG, c.S);
  if (c.qk) return qk_workspace_bytes(M, N, K, c.S);
  if (c.qo) return qo_act_bytes(M, K);
  return c.S > 1 ? (size_t)c.S * (size_t)M * (size_t)N * 4 : 0;
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0) return 0;
  return config_workspace(select_config((int)M, (int)N, (int)K, (size_t)-1), M, N, K);
}

namespace {

// The configuration a dense call runs: the default choice or the tuning override. False
// when the override names nothing compiled or cannot run this call (a streaming choice
// must cover M, fit its K slice in LDS and its partials in the workspace; a sliced tiled
// choice must fit its partials).
bool resolve_config(int M, int N, int K, size_t ws_bytes, GemmConfig& cfg) {
  cfg = select_config(M, N, K, ws_bytes);
  const int ov = override_config(cfg);
  if (ov < 0) return false;
  if (ov > 0 && cfg.sweep && (!sweep_supported(steps_of(K), cfg.J) || N % 128 != 0)) return false;
  if (ov > 0 && cfg.qo && config_workspace(cfg, M, N, K) > ws_bytes) return false;
  if (ov > 0 && cfg.qr && cfg.S > steps_of(K)) return false;
  // tail K slices run only on 128 x 128 tiles
  if (ov > 0 && cfg.qr && cfg.S > 1 && !(cfg.MT == 8 && cfg.NG == 8) && qr_tail_tiles(M, N, cfg.MT, cfg.NG) > 0)
    return false;
  if (ov > 0 && cfg.qk && 4 * cfg.S > steps_of(K)) return false;
  if (ov > 0 && cfg.tile && !cfg.qo && cfg.S > 1) {
    const int T = steps_of(K);
    if (cfg.S > T) cfg.S = T;
    if ((size_t)cfg.S * M * N * 4 > ws_bytes) return false;
  }
  if (ov > 0 && !cfg.tile) {
    const int T = steps_of(K);
    if (cfg.S > T) cfg.S = T;
    const size_t need = cfg.S > 1 ? (size_t)cfg.S * M * N * 4 : 0;
    const int TS = (T + cfg.S - 1) / cfg.S;
    if (M > 16 * cfg.MT || need > ws_bytes || (N / 16) % cfg.NG != 0 ||
        stream_lds_bytes(std::min(M, 16 * cfg.MT), TS, cfg.MT, cfg.NG, cfg.WK) > kMaxLds)
      return false;
  }
  return true;
}

}  // namespace

hipError_t launch_gemm(const void* a, const void* wp, void* c, int64_t M64, int64_t N64, int64_t K64,
                       void* ws, size_t ws_bytes, hipStream_t st) {
  const int M = (int)M64, N = (int)N64, K = (int)K64;
  if (!ws) ws_bytes = 0;
  GemmConfig cfg;
  if (!resolve_config(M, N, K, ws_bytes, cfg)) return hipErrorInvalidValue;
  return run_config(cfg, a, wp, c, (cfg.S > 1 || cfg.qo) ? static_cast<float*>(ws) : nullptr, M, N, K, st);
}

bool gemm_plan(int64_t M64, int64_t N64, int64_t K64, size_t ws_bytes, char* buf, size_t len) {
  const int M = (int)M64, N = (int)N64, K = (int)K64;
  GemmConfig c;
  if (!resolve_config(M, N, K, ws_bytes, c)) return false;
  if (c.qr) {
    const int tail = c.S > 1 ? qr_tail_tiles(M, N, c.MT, c.NG) : 0;
    char tl[64] = "";
    if (tail > 0) std::snprintf(tl, sizeof tl, " tail=%dx%d + k_qr_tail_reduce", tail, c.S);
    std::snprintf(buf, len, "k_prepare + k_gemm_qr<%d, %d, %d> GM=%d%s", c.MT, c.NG, c.NBUF, c.GM, tl);
  } else if (c.qk) {
    char split[40] = "";
    if (c.S > 1) std::snprintf(split, sizeof split, " S=%d + k_splitk_reduce", c.S);
    std::snprintf(buf, len, "k_prepare + k_gemm_qk<%d, %d, %d> GM=%d%s", c.MT, c.NG, c.NBUF, c.GM, split);
  } else if (c.qo) {
    std::snprintf(buf, len, "k_prepare + k_gemm_qo<%d, %d, %d, %d, %d, %d> GM=%d", c.WM, c.WN, c.MT, c.NG, c.NBUF,
                  c.OCC, c.GM);
  } else if (c.sweep) {
    const int T = steps_of(K);
    std::snprintf(buf, len, "k_gemm_sweep<2, 4, 4, 2, %d, %d, %d> GM=%d", T, sweep_pf(T), c.J, c.GM);
  } else if (c.tile) {
    const int T = steps_of(K), TS = (T + c.S - 1) / c.S, S = (T + TS - 1) / TS;  // as run_tile slices
    char split[40] = "";
    if (S > 1) std::snprintf(split, sizeof split, " S=%d + k_splitk_reduce", S);
    std::snprintf(buf, len, "k_gemm_tile<%d, %d, %d, %d, %d, %d> GM=%d%s", c.WM, c.WN, c.MT, c.NG, c.PF, c.OCC,
                  c.GM, split);
  } else {
    const int T = steps_of(K), TS = (T + c.S - 1) / c.S, per = (TS + c.WK - 1) / c.WK;
    std::snprintf(buf, len, "k_gemm_stream<%d, %d, %d, %d, %d> S=%d%s", c.MT, c.NG, c.WK, pick_pd(c.NG, per, kStreamPD),
                  stream_qb(M, per), c.S, c.S > 1 ? " + k_splitk_reduce" : "");
  }
  return true;
}

namespace {

template <int MT, int NG, int WK, int PD, bool RES>
hipError_t launch_grouped(const void* a, const int32_t* rt, const int32_t* offs, int E, int R_max,
                          const void* wp, void* c, int T, int N, int K, size_t lds, hipStream_t st) {
  auto kern = k_gemm_grouped<MT, NG, WK, PD, (MT == 1 ? 1 : 4), RES>;
  static std::atomic<uint64_t> configured{0};
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

template <int MT, int NG, int WK>
hipError_t run_grouped(const void* a, const int32_t* rt, const int32_t* offs, int E, int R_max,
                       const void* wp, void* c, int T, int N, int K, hipStream_t st) {
  const int steps = steps_of(K);
  const size_t lds = stream_lds_bytes(16 * MT, steps, MT, NG, WK);
  if (lds > kMaxLds) return hipErrorInvalidValue;
  const int per = (steps + WK - 1) / WK;
  const int pd = pick_pd(NG, per);
  if (per > pd) return launch_grouped<MT, NG, WK, kSkinnyPD / NG, false>(a, rt, offs, E, R_max, wp, c, T, N, K, lds, st);
  if constexpr (kSkinnyPD / NG >= 16)
    if (pd >= 16) return launch_grouped<MT, NG, WK, 16, true>(a, rt, offs, E, R_max, wp, c, T, N, K, lds, st);
  if constexpr (kSkinnyPD / NG >= 8)
    if (pd >= 8) return launch_grouped<MT, NG, WK, 8, true>(a, rt, offs, E, R_max, wp, c, T, N, K, lds, st);
  return launch_grouped<MT, NG, WK, 4, true>(a, rt, offs, E, R_max, wp, c, T, N, K, lds, st);
}

// Tiled grouped configurations (WM, WN, MT, NG, PF, OCC).
#define MX_GROUPED_TILE_CONFIGS(X) \
  X(1, 4, 4, 4, 1, 2)              \
  X(2, 4, 4, 4, 1, 1)              \
  X(1, 4, 4, 4, 2, 2)              \
  X(1, 8, 8, 4, 1, 2)

template <int WM, int WN, int MT, int NG, int PF, int OCC>
hipError_t run_grouped_tile(const void* a, const int32_t* rt, const int32_t* offs, int E, int R_max,
                            const void* wp, void* c, int T, int N, int K, hipStream_t st) {
  using S = TileShape<WM, WN, MT, NG>;
  const int64_t active = E < R_max ? E : R_max;
  const int64_t grid = (active + R_max / S::BM) * ((N + S::BN - 1) / S::BN);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gemm_grouped_tile<WM, WN, MT, NG, PF, OCC>), dim3((unsigned)grid), dim3(S::NTH), 0, st,
                     static_cast<const uint16_t*>(a), rt, offs, E, R_max, static_cast<const uint8_t*>(wp),
                     static_cast<uint16_t*>(c), T, N, K, nullptr, nullptr, 0);
  return hipGetLastError();
}

template <int WM, int WN, int MT, int NG, int PF, int OCC>
hipError_t run_grouped_tile_mx(const void* aq, const void* as, const int32_t* offs, int E, int R_max, const void* wp,
                               void* c, int N, int K, hipStream_t st) {
  using S = TileShape<WM, WN, MT, NG>;
  const int64_t active = E < R_max ? E : R_max;
  const int64_t grid = (active + R_max / S::BM) * ((N + S::BN - 1) / S::BN);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gemm_grouped_tile_mx<WM, WN, MT, NG, PF, OCC>), dim3((unsigned)grid), dim3(S::NTH), 0, st,
                     static_cast<const uint8_t*>(aq), static_cast<const uint8_t*>(as), offs, E, R_max,
                     static_cast<const uint8_t*>(wp), static_cast<uint16_t*>(c), N, K);
  return hipGetLastError();
}

template <int WM, int WN, int MT, int NG, int PF, int OCC, int ACT>
hipError_t run_grouped_tile_act(const void* a, const int32_t* rt, const int32_t* offs, int E, int R_max,
                                const void* wp, void* hq, void* hs, int T, int N, int K, hipStream_t st) {
  using S = TileShape<WM, WN, MT, NG>;
  const int64_t active = E < R_max ? E : R_max;
  const int64_t grid = (active + R_max / S::BM) * (N / S::BN);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const int Nh = ACT == kActSwiglu ? N / 2 : N;
  hipLaunchKernelGGL((k_gemm_grouped_tile<WM, WN, MT, NG, PF, OCC, ACT>), dim3((unsigned)grid), dim3(S::NTH), 0, st,
                     static_cast<const uint16_t*>(a), rt, offs, E, R_max, static_cast<const uint8_t*>(wp), nullptr, T,
                     N, K, static_cast<uint8_t*>(hq), static_cast<uint8_t*>(hs), Nh);
  return hipGetLastError();
}

struct GroupedConfig {
  bool tile = false;
  int WM = 1, WN = 4, MT = 1, NG = 1, PF = 1, OCC = 2;
};

bool grouped_tile_supported(const GroupedConfig& g) {
#define X(wm, wn, mt, ng, pf, occ) \
  if (g.WM == wm && g.WN == wn && g.MT == mt && g.NG == ng && g.PF == pf && g.OCC == occ) return true;
  MX_GROUPED_TILE_CONFIGS(X)
#undef X
  return false;
}

// The configuration a grouped call runs. Tuning only: MX_GROUPED_CONFIG="gs,MT,NG"
// (streaming, four waves) or "gt,WM,WN,MT,NG,PF,OCC" (tiled) replaces the default choice;
// false when it names no compiled configuration (the call then fails).
bool resolve_grouped(int E, int R_max, int N, int64_t rows_hint, GroupedConfig& g) {  // any T
  const int G = N / 16;
  const int64_t active = E < R_max ? E : R_max;
  const char* s = std::getenv("MX_GROUPED_CONFIG");
  if (s && *s) {
    int v[6] = {0, 0, 0, 0, 0, 0};
    if (std::sscanf(s, "gt,%d,%d,%d,%d,%d,%d", &v[0], &v[1], &v[2], &v[3], &v[4], &v[5]) == 6) {
      g.tile = true; g.WM = v[0]; g.WN = v[1]; g.MT = v[2]; g.NG = v[3]; g.PF = v[4]; g.OCC = v[5];
      return grouped_tile_supported(g);
    }
    if (std::sscanf(s, "gs,%d,%d", &v[0], &v[1]) == 2) {
      g.tile = false; g.MT = v[0]; g.NG = v[1];
      return (g.MT == 1 || g.MT == 2) && (g.NG == 1 || (g.NG == 4 && G % 4 == 0));
    }
    return false;
  }
  // Tiled (the weight streamed once per 64-row tile) whenever its grid, one CTA per active
  // expert and 256-column tile, can fill the chip; the streaming kernel (more, narrower
  // CTAs) only for a handful of active experts. Segments longer than 64 rows take the
  // 128 x 512 tile, so that one row tile still covers a typical segment and each expert's
  // weight is streamed once rather than twice. Streaming widens to four column groups per
  // CTA as segments grow, amortizing each CTA's serial segment-lookup -> token ->
  // activation chain over more streamed weight.
  if (G % 16 == 0 && active * (G / 16) >= 512) {
    g = (rows_hint > 64 && G % 32 == 0) ? GroupedConfig{true, 1, 8, 8, 4, 1, 2} : GroupedConfig{true, 1, 4, 4, 4, 2, 2};
    return true;
  }
  g.tile = false;
  if (rows_hint <= 16) { g.MT = 1; g.NG = (active < 128 || G % 4 != 0) ? 1 : 4; }
  else { g.MT = 2; g.NG = (rows_hint <= 32 || G % 4 != 0) ? 1 : 4; }
  return true;
}

}  // namespace

hipError_t launch_gemm_grouped(const void* a, const int32_t* row_token, const int32_t* offsets, int64_t E,
                               int64_t R_max, const void* wp, void* c, int64_t T, int64_t N, int64_t K,
                               int64_t rows_hint, hipStream_t st) {
  const int e = (int)E, r = (int)R_max, t = (int)T, n = (int)N, k = (int)K;
  GroupedConfig g;
  if (!resolve_grouped(e, r, n, rows_hint, g)) return hipErrorInvalidValue;
  if (g.tile) {
#define X(wm, wn, mt, ng, pf, occ)                                                                 \
    if (g.WM == wm && g.WN == wn && g.MT == mt && g.NG == ng && g.PF == pf && g.OCC == occ)         \
      return run_grouped_tile<wm, wn, mt, ng, pf, occ>(a, row_token, offsets, e, r, wp, c, t, n, k, st);
    MX_GROUPED_TILE_CONFIGS(X)
#undef X
    return hipErrorInvalidValue;
  }
  if (g.MT == 1 && g.NG == 1) return run_grouped<1, 1, 4>(a, row_token, offsets, e, r, wp, c, t, n, k, st);
  if (g.MT == 1 && g.NG == 4) return run_grouped<1, 4, 4>(a, row_token, offsets, e, r, wp, c, t, n, k, st);
  if (g.MT == 2 && g.NG == 1) return run_grouped<2, 1, 4>(a, row_token, offsets, e, r, wp, c, t, n, k, st);
  if (g.MT == 2 && g.NG == 4) return run_grouped<2, 4, 4>(a, row_token, offsets, e, r, wp, c, t, n, k, st);
  return hipErrorInvalidValue;
}

namespace {

// Fused activation + quantization variants of the tiled grouped kernel (WM, WN, MT, NG, PF, OCC).
#define MX_GROUPED_ACT_CONFIGS(X) \
  X(1, 4, 4, 4, 2, 2)             \
  X(1, 8, 8, 4, 1, 2)             \
  X(1, 4, 4, 2, 2, 2)

// The fused call and the second GEMM always run the tiled grouped kernel (the fused epilogue
// needs a whole row tile of gate and up columns in one CTA; the second GEMM has no streaming
// variant): 128 x 512 tiles for segments longer than 64 rows when N is a multiple of 512;
// 64 x 128 when fewer than 256 CTAs of 64 x 256 would run (`grid256` = min(E, R_max) N / 256;
// the fused call at T = 1: 21.0 -> 17.9 us); 64 x 256 otherwise. MX_GROUPED_CONFIG="gt,..."
// may force another of these configurations (tuning only).
bool resolve_grouped_act(int N, int64_t rows_hint, int64_t grid256, GroupedConfig& g) {
  const char* s = std::getenv("MX_GROUPED_CONFIG");
  if (s && *s) {
    int v[6] = {0, 0, 0, 0, 0, 0};
    if (std::sscanf(s, "gt,%d,%d,%d,%d,%d,%d", &v[0], &v[1], &v[2], &v[3], &v[4], &v[5]) != 6) return false;
    g = GroupedConfig{true, v[0], v[1], v[2], v[3], v[4], v[5]};
  } else if (rows_hint > 64 && N % 512 == 0) {
    g = GroupedConfig{true, 1, 8, 8, 4, 1, 2};
  } else if (grid256 < 256 && N % 128 == 0) {
    g = GroupedConfig{true, 1, 4, 4, 2, 2, 2};
  } else {
    g = GroupedConfig{true, 1, 4, 4, 4, 2, 2};
  }
  const int BN = 16 * g.NG * g.WN;
#define X(wm, wn, mt, ng, pf, occ) \
  if (g.WM == wm && g.WN == wn && g.MT == mt && g.NG == ng && g.PF == pf && g.OCC == occ) return N % BN == 0;
  MX_GROUPED_ACT_CONFIGS(X)
#undef X
  return false;
}

}  // namespace

hipError_t launch_gemm_grouped_act(const void* a, const int32_t* row_token, const int32_t* offsets, int64_t E,
                                   int64_t R_max, const void* wp, void* hq, void* hs, int64_t T, int64_t N,
                                   int64_t K, int act, int64_t rows_hint, hipStream_t st) {
  const int e = (int)E, r = (int)R_max, t = (int)T, n = (int)N, k = (int)K;
  GroupedConfig g;
  if (!resolve_grouped_act(n, rows_hint, std::min(E, R_max) * (N / 256), g)) return hipErrorInvalidValue;
#define X(wm, wn, mt, ng, pf, occ)                                                                        \
  if (g.WM == wm && g.WN == wn && g.MT == mt && g.NG == ng && g.PF == pf && g.OCC == occ)                \
    return act == kActSwiglu                                                                              \
               ? run_grouped_tile_act<wm, wn, mt, ng, pf, occ, kActSwiglu>(a, row_token, offsets, e, r, wp, hq, \
                                                                            hs, t, n, k, st)                   \
               : run_grouped_tile_act<wm, wn, mt, ng, pf, occ, kActSilu>(a, row_token, offsets, e, r, wp, hq, hs, \
                                                                          t, n, k, st);
  MX_GROUPED_ACT_CONFIGS(X)
#undef X
  return hipErrorInvalidValue;
}

namespace {

// Grouped short-K sweep configurations (T, PF, J), 128 x 128 column tiles. More column tiles per
// unit amortize its lookup, pipeline fill and epilogue further (N=3584, K=768, T=4096: J = 4, 7,
// 14 took 512, 451, 424 us).
#define MX_GROUPED_SWEEP_CONFIGS(X) X(2, 3, 4) X(4, 6, 4) X(6, 9, 4) X(6, 9, 7) X(6, 9, 14) X(8, 10, 4)

template <int T, int PF, int J>
hipError_t run_grouped_sweep_mx(const void* aq, const void* as, const int32_t* offs, int E, int R_max, const void* wp,
                                void* c, int N, int K, hipStream_t st) {
  using S = SweepShape<2, 4, 4, 2, T, PF>;
  if (K != T * kStepK || N % S::BN != 0) return hipErrorInvalidValue;
  auto kern = k_gemm_grouped_sweep_mx<T, PF, J>;
  static std::atomic<uint64_t> configured{0};
  hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), configured);
  if (e != hipSuccess) return e;
  const int64_t active = E < R_max ? E : R_max;
  const int64_t grid = (active + R_max / S::BM) * ((N / S::BN + J - 1) / J);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(S::NTH), S::SMEM, st, static_cast<const uint8_t*>(aq),
                     static_cast<const uint8_t*>(as), offs, E, R_max, static_cast<const uint8_t*>(wp),
                     static_cast<uint16_t*>(c), N);
  return hipGetLastError();
}

bool grouped_sweep_supported(int T, int J) {
#define X(t, pf, j) if (T == t && J == j) return true;
  MX_GROUPED_SWEEP_CONFIGS(X)
#undef X
  return false;
}

int grouped_sweep_pf(int T) {
#define X(t, pf, j) if (T == t) return pf;
  MX_GROUPED_SWEEP_CONFIGS(X)
#undef X
  return 0;
}

// The second GEMM's configuration: the sweep kernel (J > 0) when segments exceed 64 rows and
// K is a compiled step count (the most column tiles per unit compiled for it: 14 at K = 768,
// which makes N = 3584 two units per expert), the
// tiled kernel otherwise. Tuning only: MX_GROUPED_CONFIG="gk,J" forces the sweep kernel,
// "gt,..." a tiled configuration; false when the choice cannot run this call.
bool resolve_grouped_mx(int N, int K, int64_t rows_hint, GroupedConfig& g, int& J) {
  const int T = steps_of(K);
  J = 0;
  const char* s = std::getenv("MX_GROUPED_CONFIG");
  if (s && *s && s[0] == 'g' && s[1] == 'k') {
    if (std::sscanf(s, "gk,%d", &J) != 1) return false;
    return grouped_sweep_supported(T, J) && N % 128 == 0;
  }
  if (!(s && *s) && rows_hint > 64 && N % 128 == 0) {
    for (const int j : {14, 7, 4})
      if (grouped_sweep_supported(T, j)) { J = j; return true; }
  }
  return resolve_grouped_act(N, rows_hint, INT64_MAX, g);  // the second GEMM never narrows to 64 x 128
}

}  // namespace

hipError_t launch_gemm_grouped_mx(const void* aq, const void* as, const int32_t* offsets, int64_t E, int64_t R_max,
                                  const void* wp, void* c, int64_t N, int64_t K, int64_t rows_hint, hipStream_t st) {
  const int e = (int)E, r = (int)R_max, n = (int)N, k = (int)K;
  GroupedConfig g;
  int J = 0;
  if (!resolve_grouped_mx(n, k, rows_hint, g, J)) return hipErrorInvalidValue;
  if (J > 0) {
    const int T = steps_of(k);
#define X(t, pf, j) if (T == t && J == j) return run_grouped_sweep_mx<t, pf, j>(aq, as, offsets, e, r, wp, c, n, k, st);
    MX_GROUPED_SWEEP_CONFIGS(X)
#undef X
    return hipErrorInvalidValue;
  }
#define X(wm, wn, mt, ng, pf, occ)                                                          \
  if (g.WM == wm && g.WN == wn && g.MT == mt && g.NG == ng && g.PF == pf && g.OCC == occ)  \
    return run_grouped_tile_mx<wm, wn, mt, ng, pf, occ>(aq, as, offsets, e, r, wp, c, n, k, st);
  MX_GROUPED_ACT_CONFIGS(X)
#undef X
  return hipErrorInvalidValue;
}

bool grouped_mx_plan(int64_t N, int64_t K, int64_t rows_hint, char* buf, size_t len) {
  GroupedConfig g;
  int J = 0;
  if (!resolve_grouped_mx((int)N, (int)K, rows_hint, g, J)) return false;
  if (J > 0) {
    const int T = steps_of((int)K);
    std::snprintf(buf, len, "k_gemm_grouped_sweep_mx<%d, %d, %d>", T, grouped_sweep_pf(T), J);
    return true;
  }
  std::snprintf(buf, len, "k_gemm_grouped_tile_mx<%d, %d, %d, %d, %d, %d>", g.WM, g.WN, g.MT, g.NG, g.PF, g.OCC);
  return true;
}

hipError_t launch_moe_combine(const void* y, int64_t R, const int32_t* rows, const float* w, int64_t T, int64_t topk,
                              int64_t N, void* out, hipStream_t st) {
  const int64_t n = T * (N / 8);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(y), (int)R, rows, w, (int)T, (int)topk, (int)N,
                     static_cast<uint16_t*>(out));
  return hipGetLastError();
}

bool grouped_act_plan(int64_t E, int64_t R_max, int64_t N, int act, int64_t rows_hint, char* buf, size_t len) {
  GroupedConfig g;
  if (!resolve_grouped_act((int)N, rows_hint, std::min(E, R_max) * (N / 256), g)) return false;
  std::snprintf(buf, len, "k_gemm_grouped_tile<%d, %d, %d, %d, %d, %d, %s>", g.WM, g.WN, g.MT, g.NG, g.PF, g.OCC,
                act == kActSwiglu ? "swiglu" : "silu");
  return true;
}

bool grouped_plan(int64_t E, int64_t R_max, int64_t N, int64_t K, int64_t /*T*/, int64_t rows_hint, char* buf,
                  size_t len) {
  GroupedConfig g;
  if (!resolve_grouped((int)E, (int)R_max, (int)N, rows_hint, g)) return false;
  if (g.tile) {
    std::snprintf(buf, len, "k_gemm_grouped_tile<%d, %d, %d, %d, %d, %d>", g.WM, g.WN, g.MT, g.NG, g.PF, g.OCC);
  } else {
    constexpr int WK = 4;
    const int per = (steps_of((int)K) + WK - 1) / WK, pd = pick_pd(g.NG, per);
    const bool res = per <= pd;
    std::snprintf(buf, len, "k_gemm_grouped<%d, %d, %d, %d, %d, %s>", g.MT, g.NG, WK, res ? pd : kSkinnyPD / g.NG,
                  g.MT == 1 ? 1 : 4, res ? "true" : "false");
  }
  return true;
}

}  // namespace mx
