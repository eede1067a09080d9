// Multi-row projection for prefill chunks: C[m][n] = sum_k A[m][k] W[n][k]
// for up to 512 activation rows (engine.zig Engine.prefill: a chunk of token
// columns shares one pass over every weight matrix; decoder.rs AttnWeights:
// weights are row-major [out][in]).
//
// gfx950 design.  A chunk projection streams each weight matrix once and
// does 2 M flops per weight element (4 M with the split-bf16 activations),
// so with M = 128 it sits near the HBM / MFMA ridge.
//  * MFMA v_mfma_f32_32x32x16_bf16: on gfx950 it has twice the flop rate of
//    the 16x16x32 form.
//  * Weights are read from a packed copy made once at init: 32-row x 16-k
//    tiles of 1 KB in MFMA lane order, so every weight load instruction of a
//    wave reads one contiguous kilobyte (coalesced, one page), straight into
//    the B-operand registers.  Row-major fragments would touch 32 rows per
//    instruction and stall the L1 TLB and the address path.
//  * Block = 4 waves over 64 activation rows x 256 weight rows; a wave owns
//    2 weight tiles of 32 rows (for the paired epilogues one tile and its
//    partner rows) for all 64 rows, accumulating 2 x 2 32x32 fp32 tiles.
//  * Activations (split bf16: hi and lo planes, two MFMAs per product) are
//    staged per 64-wide k step into LDS with coalesced loads (8 threads per
//    128-byte row piece), in MFMA fragment order with an XOR swizzle that
//    keeps both the stores and the fragment reads free of bank conflicts.
//  * Two LDS stages and two weight register buffers: the next step's loads
//    are in flight during the current step's MFMAs.  Loads are
//    unconditional (masked lanes read a zero page), so the compiler's wait
//    counts stay exact.
//  * Split-K across blocks fills the compute units when a matrix has few
//    tiles; partials go to Cpart and gemm_reduce sums them in fixed split
//    order.  Without a split the epilogue runs straight from the
//    accumulators.
//  * Grouped form (MoE experts of a prefill chunk; engine.zig Engine.prefill
//    batches a chunk's columns by chosen expert, so each chosen expert's
//    weights are read once): the groups' rows are cut into 32-row tiles (in
//    group order), a block takes one (row tile, weight-tile block) and finds
//    its group from the device-side group counts; the weights are the
//    expert's slice of a packed copy of the stacked [E][rows][K] matrix and
//    the rows are gathered through a_rows (the token row of each (token,
//    expert) pair).  The grid covers the largest possible tile count, and
//    only blocks past the actual count exit: a grid of every group times its
//    largest possible row count, most of whose blocks exit at once, measured
//    close to twice as slow.
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "epilogue.h"

namespace {

constexpr int CK_WAVES = 4;  // waves per block
constexpr int CK_NS = 2;     // 32-row weight tiles per wave
constexpr int CK_STEP = 64;  // k per pipeline step (4 MFMA k groups of 16)
constexpr int CK_ROWS = 64;  // activation rows per block
constexpr int CK_XCDS = 8;   // blocks are dispatched round-robin over 8 XCDs

// 1 KB of zeros: masked-off lanes load from here (16 bytes each), so loads
// need no value select, which would force a wait right after the load.
__device__ u32x4 ck_zero[64];  // never written: zero-initialised

// Activation stage = MFMA A fragments (t, s, plane) of 64 lanes x 16 bytes:
// 32 rows x 16 k, fragment f = (t * 4 + s) * PL + plane at LDS slots f * 64.
// Lane l of a fragment holds row 32 t + l % 32 at k0 + 16 s + 8 g
// (g = l / 32), kept in slot a_swz(l % 32, g, s).
template <int MT, bool SPLIT>
struct AStage {
  static constexpr int PL = SPLIT ? 2 : 1;
  static constexpr int PIECES = MT * 32 * 8 * PL;  // 16-byte pieces per stage
  static constexpr int PER_THREAD = (PIECES + CK_WAVES * WAVE - 1) / (CK_WAVES * WAVE);
  static constexpr int NFRAG = MT * 4 * PL;
};

__device__ __forceinline__ int a_swz(int r32, int g, int s) { return (r32 ^ (2 * (2 * s + g))) + 32 * g; }

// Staging piece -> (row, 16-byte chunk c8 of the row's 128 bytes): each 8
// consecutive pieces are 4 chunks of two adjacent rows (bits 0-1: c8 % 4,
// bit 2: row % 2, bit 3: c8 / 4), so the 8 lanes an LDS cycle serves store
// to 8 different bank groups (one row's 8 chunks would hit only 4 of them
// under the swizzle).  A wave's global loads still cover 8 whole rows.
__device__ __forceinline__ int piece_row(int rem) { return ((rem >> 4) << 1) | ((rem >> 2) & 1); }
__device__ __forceinline__ int piece_c8(int rem) { return (rem & 3) | (((rem >> 3) & 1) << 2); }

// Global -> registers, coalesced: piece e = (plane, row r, 16-byte chunk c8
// of the step's 128 bytes); rows past `rows` and k past kend read zeros.
template <int MT, bool SPLIT>
__device__ __forceinline__ void a_load(const uint16_t *abase, const GemmArgs &g, int rows, int k0, int kend,
                                       u32x4 (&ar)[AStage<MT, SPLIT>::PER_THREAD]) {
  constexpr int PER_PLANE = MT * 256, PIECES = AStage<MT, SPLIT>::PIECES;
#pragma unroll
  for (int i = 0; i < AStage<MT, SPLIT>::PER_THREAD; ++i) {
    const int e = threadIdx.x + i * CK_WAVES * WAVE;
    const int plane = e / PER_PLANE, rem = e - plane * PER_PLANE;
    const int r = piece_row(rem), k = k0 + piece_c8(rem) * 8;
    const bool ok = (PIECES % (CK_WAVES * WAVE) == 0 || e < PIECES) && r < rows && k < kend;
    ar[i] = load16(ok ? static_cast<const void *>(abase + plane * g.a_lo + (int64_t)r * g.lda + k)
                      : static_cast<const void *>(ck_zero + (threadIdx.x & 63)));
  }
}

// Registers -> LDS: chunk c8 of row r is k group g = c8 % 2 of MFMA step
// s = c8 / 2.  The swizzle spreads the 16 lanes of each store cycle (two
// rows x eight chunks) over all 16 bank groups.
template <int MT, bool SPLIT>
__device__ __forceinline__ void a_store(u32x4 *dst, const u32x4 (&ar)[AStage<MT, SPLIT>::PER_THREAD]) {
  constexpr int PER_PLANE = MT * 256, PIECES = AStage<MT, SPLIT>::PIECES, PL = AStage<MT, SPLIT>::PL;
#pragma unroll
  for (int i = 0; i < AStage<MT, SPLIT>::PER_THREAD; ++i) {
    const int e = threadIdx.x + i * CK_WAVES * WAVE;
    const int plane = e / PER_PLANE, rem = e - plane * PER_PLANE;
    const int r = piece_row(rem), c8 = piece_c8(rem);
    const int t = r >> 5, s = c8 >> 1, gk = c8 & 1;
    if (PIECES % (CK_WAVES * WAVE) == 0 || e < PIECES)
      dst[((t * 4 + s) * PL + plane) * WAVE + a_swz(r & 31, gk, s)] = ar[i];
  }
}

// This wave's weight fragments of the step at k0: tile p, k group s (one
// contiguous kilobyte of the packed copy per load).  NT: non-temporal loads
// (a dense chunk reads each weight tile from HBM once, and its other row
// blocks run on the same XCD at the same time: 8B prefill at 128 rows
// 18.5 k -> 19.2 k tok/s); the grouped form keeps plain loads, because the
// row tiles of one group, on other XCDs, re-read the expert's weights from
// the memory-side cache (non-temporal there: MoE expert node 47.5 -> 50.7 us).
template <bool NT>
__device__ __forceinline__ void w_load(const uint16_t *const (&wp)[CK_NS], const bool (&wv)[CK_NS], int k0,
                                       int kend, u32x4 (&w)[CK_NS][4]) {
  const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const bool kok = k0 + 16 * s < kend;
#pragma unroll
    for (int p = 0; p < CK_NS; ++p)
      w[p][s] = (NT ? load16_nt : load16)(kok && wv[p] ? static_cast<const void *>(wp[p] + (k0 / 16 + s) * 512)
                                                    : static_cast<const void *>(ck_zero + lane));
  }
}

// One k step: for each (s, t) the A fragments (hi, lo) from LDS feed
// CK_NS (x2) MFMAs; the next pair's LDS reads are issued before the
// current MFMAs, and scheduling barriers keep the compiler from hoisting
// every read of the step.
template <int MT, bool SPLIT>
__device__ __forceinline__ void mma_step(const u32x4 *src, const u32x4 (&w)[CK_NS][4], const int (&sw)[4],
                                         f32x16 (&acc)[MT][CK_NS]) {
  constexpr int PL = AStage<MT, SPLIT>::PL;
  u32x4 cur[PL], nxt[PL];
#pragma unroll
  for (int pl = 0; pl < PL; ++pl) cur[pl] = src[pl * WAVE + sw[0]];
#pragma unroll
  for (int idx = 0; idx < 4 * MT; ++idx) {
    const int s = idx / MT, t = idx % MT;
    if (idx + 1 < 4 * MT) {
      const int s1 = (idx + 1) / MT, t1 = (idx + 1) % MT;
#pragma unroll
      for (int pl = 0; pl < PL; ++pl) nxt[pl] = src[((t1 * 4 + s1) * PL + pl) * WAVE + sw[s1]];
    }
#pragma unroll
    for (int pl = 0; pl < PL; ++pl)
#pragma unroll
      for (int p = 0; p < CK_NS; ++p) acc[t][p] = mfma32x32x16(as_bf16x8(cur[pl]), as_bf16x8(w[p][s]), acc[t][p]);
    __builtin_amdgcn_sched_barrier(0);
    if (idx + 1 < 4 * MT) {
#pragma unroll
      for (int pl = 0; pl < PL; ++pl) cur[pl] = nxt[pl];
    }
  }
}

// Grouped form: this thread's staging pieces as row pointers (the gather
// resolved once per block; a row past the block's rows reads the zero page)
// and their k offsets within a step.
template <int MT, bool SPLIT>
struct ARows {
  const uint16_t *p[AStage<MT, SPLIT>::PER_THREAD];
  int koff[AStage<MT, SPLIT>::PER_THREAD];
};

template <int MT, bool SPLIT>
__device__ __forceinline__ ARows<MT, SPLIT> a_rows_of(const GemmArgs &g, int row0, int rows) {
  constexpr int PER_PLANE = MT * 256, PIECES = AStage<MT, SPLIT>::PIECES;
  ARows<MT, SPLIT> ra;
#pragma unroll
  for (int i = 0; i < AStage<MT, SPLIT>::PER_THREAD; ++i) {
    const int e = threadIdx.x + i * CK_WAVES * WAVE;
    const int plane = e / PER_PLANE, rem = e - plane * PER_PLANE;
    const int r = piece_row(rem);
    ra.koff[i] = piece_c8(rem) * 8;
    const bool ok = (PIECES % (CK_WAVES * WAVE) == 0 || e < PIECES) && r < rows;
    const int64_t src = ok ? (g.a_rows ? g.a_rows[row0 + r] : row0 + r) : 0;
    ra.p[i] = ok ? g.A + plane * g.a_lo + src * g.lda + ra.koff[i] : nullptr;
  }
  return ra;
}

template <int MT, bool SPLIT>
__device__ __forceinline__ void a_load_rows(const ARows<MT, SPLIT> &ra, int k0, int kend,
                                            u32x4 (&ar)[AStage<MT, SPLIT>::PER_THREAD]) {
#pragma unroll
  for (int i = 0; i < AStage<MT, SPLIT>::PER_THREAD; ++i) {
    const bool ok = ra.p[i] != nullptr && k0 + ra.koff[i] < kend;
    ar[i] = load16(ok ? static_cast<const void *>(ra.p[i] + k0) : static_cast<const void *>(ck_zero + (threadIdx.x & 63)));
  }
}

// Block b -> (unit u = (weight tile, k split), row block mb): the row
// blocks of one unit are CK_XCDS block ids apart, so they are dispatched to
// the same XCD at about the same time and the second one finds the weights
// in that XCD's L2.  GR (grouped, mblocks 1): u = (row tile of 32 MT
// rows, weight tile).
template <int MT, int EPI, bool SPLIT, bool GR, bool PIN>
__global__ __launch_bounds__(CK_WAVES * WAVE, 2) void gemm_chunk_kernel(GemmArgs g, int ntiles16, int mblocks) {
  constexpr int NP = paired<EPI>();
  constexpr int LT = CK_NS / NP;  // logical 32-row tiles per wave
  __shared__ u32x4 a_s[2][AStage<MT, SPLIT>::NFRAG * WAVE];

  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int K = g.K;
  const int ntiles32 = ntiles16 / 2;
  const int nbt = (ntiles32 + CK_WAVES * LT - 1) / (CK_WAVES * LT);
  const int u = (blockIdx.x / (CK_XCDS * mblocks)) * CK_XCDS + blockIdx.x % CK_XCDS;
  const int mb = (blockIdx.x / CK_XCDS) % mblocks;
  int bt, z, row0, rows;
  const uint16_t *Wbase = g.Wp;
  if constexpr (GR) {
    // ksplit is 1: u = row tile t * nbt + tile block.  Wave 0 finds the
    // group of row tile t: an inclusive prefix sum of the groups' tile
    // counts, 64 groups at a time.
    __shared__ int tile_sel[2];
    const int t = u / nbt;
    bt = u - t * nbt;
    if (wave == 0) {
      const int ng = *g.n_groups;
      int base = 0, gsel = -1, tsel = 0;
      for (int c0 = 0; c0 < ng && gsel < 0; c0 += WAVE) {
        const int i = c0 + lane;
        const int cnt = i < ng ? g.group_count[i] : 0;
        const int nt = (cnt + 32 * MT - 1) / (32 * MT);
        int incl = nt;
#pragma unroll
        for (int o = 1; o < WAVE; o <<= 1) {
          const int v = __shfl_up(incl, o, WAVE);
          if (lane >= o) incl += v;
        }
        const bool hit = nt > 0 && t >= base + incl - nt && t < base + incl;
        const unsigned long long m = __ballot(hit);
        const int src = m ? __ffsll((long long)m) - 1 : 0;
        const int first = __shfl(incl - nt, src, WAVE);
        if (m) {
          gsel = c0 + src;
          tsel = t - base - first;
        }
        base += __shfl(incl, WAVE - 1, WAVE);
      }
      if (lane == 0) {
        tile_sel[0] = gsel;
        tile_sel[1] = tsel;
      }
    }
    __syncthreads();
    const int gi = tile_sel[0];
    if (gi < 0) return;
    z = 0;
    row0 = tile_sel[1] * 32 * MT;
    rows = min(32 * MT, g.group_count[gi] - row0);
    row0 += g.group_start[gi];
    Wbase += (int64_t)g.group_expert[gi] * g.w_group_stride;
  } else {
    if (u >= nbt * g.ksplit) return;
    bt = u % nbt;
    z = u / nbt;
    row0 = mb * CK_ROWS;
    rows = min(CK_ROWS, g.M - row0);
  }
  const int nsteps = (K + CK_STEP - 1) / CK_STEP;
  const int per = (nsteps + g.ksplit - 1) / g.ksplit;
  const int s0 = min(nsteps, z * per), s1 = min(nsteps, s0 + per);
  const uint16_t *abase = g.A + (int64_t)row0 * g.lda;
  ARows<MT, SPLIT> ra;
  if constexpr (GR) ra = a_rows_of<MT, SPLIT>(g, row0, rows);
  auto aload = [&](int k0, int kend, u32x4(&ar)[AStage<MT, SPLIT>::PER_THREAD]) {
    if constexpr (GR) a_load_rows<MT, SPLIT>(ra, k0, kend, ar);
    else a_load<MT, SPLIT>(abase, g, rows, k0, kend, ar);
  };

  // this wave's 32-row tiles T (16-row logical tiles 2T, 2T + 1): weight
  // tile p = lt * NP + half, in the packed copy at row tile r0 / 32
  const uint16_t *wp[CK_NS];
  bool wv[CK_NS];
  int tt[LT];
#pragma unroll
  for (int lt = 0; lt < LT; ++lt) {
    const int T = (bt * CK_WAVES + wave) * LT + lt;
    tt[lt] = T;
    const bool ok = T < ntiles32;
    const int r0 = ok ? tile_n0<EPI>(g, 2 * T) : 0;
#pragma unroll
    for (int h = 0; h < NP; ++h) {
      wv[lt * NP + h] = ok;
      wp[lt * NP + h] = Wbase + (ok ? (int64_t)((r0 + h * g.np_off) / 32) * (K / 16) * 512 : 0) + lane * 8;
    }
  }
  int sw[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) sw[s] = a_swz(lane & 31, lane >> 5, s);

  f32x16 acc[MT][CK_NS];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int p = 0; p < CK_NS; ++p)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][p][i] = 0.f;

  u32x4 w0[CK_NS][4], w1[CK_NS][4];
  u32x4 ar[AStage<MT, SPLIT>::PER_THREAD];
  const int kend = min(K, s1 * CK_STEP);
  if (s0 < s1) {
    aload(s0 * CK_STEP, kend, ar);
    w_load<!GR>(wp, wv, s0 * CK_STEP, kend, w0);
    a_store<MT, SPLIT>(a_s[0], ar);
  }
  __syncthreads();
  // Two steps per iteration, activation loads first (the wait before their
  // LDS store then leaves the newer weight loads in flight).  Steps at or
  // past s1 read zeros (k >= kend), so an odd step count adds one zero step.
  // PIN holds that order with scheduling barriers: left to itself the
  // compiler moved weight loads ahead of activation loads, so the
  // activation stores also waited for 2-4 of the step's weight loads.  It
  // pays where few row blocks share a weight tile (128 rows: 8B prefill
  // 19.25 k -> 19.68 k tok/s on one machine, unchanged on a slower one);
  // with 8 row blocks (512 rows) the down projection measured 122 -> 125.5
  // us with it, and the grouped form 1% slower, so those keep the
  // compiler's order.
  auto order = [] {
    if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
  };
  for (int s = s0; s < s1; s += 2) {
    aload((s + 1) * CK_STEP, kend, ar);
    order();
    w_load<!GR>(wp, wv, (s + 1) * CK_STEP, kend, w1);
    order();
    mma_step<MT, SPLIT>(a_s[0], w0, sw, acc);
    a_store<MT, SPLIT>(a_s[1], ar);
    __syncthreads();
    aload((s + 2) * CK_STEP, kend, ar);
    order();
    w_load<!GR>(wp, wv, (s + 2) * CK_STEP, kend, w0);
    order();
    mma_step<MT, SPLIT>(a_s[1], w1, sw, acc);
    a_store<MT, SPLIT>(a_s[0], ar);
    __syncthreads();
  }

  // epilogue: lane l holds rows 32 t + 8 (i / 4) + 4 (l / 32) + i % 4 of
  // column l % 32 of each tile, i.e. logical 16-row tile 2 T + (l % 32) / 16,
  // column c = l % 16
  const int64_t np_cols = (int64_t)ntiles16 * 16;
  const int c = lane & 15;
#pragma unroll
  for (int lt = 0; lt < LT; ++lt) {
    const int b = 2 * tt[lt] + ((lane >> 4) & 1);
    const bool bok = tt[lt] < ntiles32;
    const int n = bok ? tile_n0<EPI>(g, b) + c : 0;
    const bool nok = bok && (EPI == EPI_QKV || n < g.N);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = 32 * t + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        const float v0 = acc[t][lt * NP][i], v1 = acc[t][lt * NP + NP - 1][i];
        const bool ok = nok && m < rows;
        if (g.ksplit > 1) {
          if (ok) {
            float *dst = g.Cpart + ((int64_t)z * g.M + row0 + m) * NP * np_cols + (int64_t)b * 16 + c;
            dst[0] = v0;
            if (NP == 2) dst[np_cols] = v1;
          }
        } else {
          if (ok) epi_apply<EPI>(g, row0 + m, n, v0, v1);
          if (EPI == EPI_LOGITS) {
            // best (value, index) of this logical tile's 16 columns for row
            // m: they sit in the 16 lanes that share l / 16
            float bv = ok ? v0 : -INFINITY;
            int bi = ok ? n : 0x7fffffff;
#pragma unroll
            for (int o = 1; o <= 8; o <<= 1) {
              const float ov = __shfl_xor(bv, o, WAVE);
              const int oi = __shfl_xor(bi, o, WAVE);
              if (better(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
              }
            }
            if (c == 0 && bok && m < rows) {
              g.am.part_val[(int64_t)(row0 + m) * ntiles16 + b] = bv;
              g.am.part_idx[(int64_t)(row0 + m) * ntiles16 + b] = bi;
            }
          }
        }
      }
    }
  }
}

template <int MT, int EPI, bool GR, bool PIN>
hipError_t launch_mt(const GemmArgs &g, int ntiles16, int blocks, int mblocks, hipStream_t st) {
  if (g.a_lo)
    hipLaunchKernelGGL((gemm_chunk_kernel<MT, EPI, true, GR, PIN>), dim3(blocks), dim3(CK_WAVES * WAVE), 0, st, g,
                       ntiles16, mblocks);
  else
    hipLaunchKernelGGL((gemm_chunk_kernel<MT, EPI, false, GR, PIN>), dim3(blocks), dim3(CK_WAVES * WAVE), 0, st, g,
                       ntiles16, mblocks);
  return hipGetLastError();
}

// loads in program order up to CK_PIN_MBLOCKS row blocks per weight tile
constexpr int CK_PIN_MBLOCKS = 2;

template <int EPI>
hipError_t launch_epi(const GemmArgs &g, int ntiles16, int blocks, int mblocks, hipStream_t st) {
  if (std::min(g.M, CK_ROWS) <= 32) return launch_mt<1, EPI, false, true>(g, ntiles16, blocks, mblocks, st);
  if (mblocks <= CK_PIN_MBLOCKS) return launch_mt<2, EPI, false, true>(g, ntiles16, blocks, mblocks, st);
  return launch_mt<2, EPI, false, false>(g, ntiles16, blocks, mblocks, st);
}

// P[((nt * K / 16 + kt) * 64 + l) * 8 + e] = W[32 nt + l % 32][16 kt + 8 (l / 32) + e]
// (W rows ld elements apart): one thread per 16-byte piece; the stores are
// coalesced.
__global__ __launch_bounds__(256) void pack_w32_kernel(const uint16_t *W, int64_t ld, int64_t pieces, int K,
                                                       uint16_t *P) {
  const int kt16 = K / 16;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < pieces; i += (int64_t)gridDim.x * 256) {
    const int l = (int)(i & 63);
    const int64_t tile = i >> 6;
    const int64_t nt = tile / kt16;
    const int kt = (int)(tile - nt * kt16);
    const int64_t row = 32 * nt + (l & 31);
    const u32x4 v = load16(W + row * ld + 16 * kt + 8 * (l >> 5));
    *reinterpret_cast<u32x4 *>(P + i * 8) = v;
  }
}

}  // namespace

bool pack_w32_fits(int64_t rows, int K) { return rows > 0 && rows % 32 == 0 && K > 0 && K % 16 == 0; }

hipError_t launch_pack_w32_ld(const uint16_t *W, int64_t ld, int64_t rows, int K, uint16_t *P, hipStream_t st) {
  if (!pack_w32_fits(rows, K) || ld < K || ld % 8) return hipErrorInvalidValue;
  const int64_t pieces = rows * K / 8;
  const int blocks = (int)std::min<int64_t>((pieces + 255) / 256, 65536);
  hipLaunchKernelGGL(pack_w32_kernel, dim3(blocks), dim3(256), 0, st, W, ld, pieces, K, P);
  return hipGetLastError();
}

hipError_t launch_pack_w32(const uint16_t *W, int64_t rows, int K, uint16_t *P, hipStream_t st) {
  return launch_pack_w32_ld(W, K, rows, K, P, st);
}

int gemm_chunk_tiles(const GemmArgs &g, int epi) {
  const int lt = (epi == EPI_SWIGLU || epi == EPI_QKV) ? CK_NS / 2 : CK_NS;
  return (gemm_ntiles(g, epi) / 2 + CK_WAVES * lt - 1) / (CK_WAVES * lt);
}

int gemm_chunk_mblocks(int rows) { return (rows + CK_ROWS - 1) / CK_ROWS; }

bool gemm_chunk_fits(const GemmArgs &g, int epi) {
  // the packed copy covers every weight row in 32-row tiles
  const int64_t wrows = epi == EPI_SWIGLU ? 2 * (int64_t)g.N : g.N;
  return g.Wp != nullptr && g.M >= 2 && g.M <= 512 && g.A != nullptr && g.x == nullptr && g.n_groups == nullptr &&
         g.a_rows == nullptr && pack_w32_fits(wrows, g.K) && gemm_ntiles(g, epi) % 2 == 0 &&
         (epi == EPI_QKV ? g.np_off % 32 == 0 : g.N % 32 == 0);
}

hipError_t launch_gemm_chunk(const GemmArgs &g, int epi, hipStream_t st) {
  if (!gemm_chunk_fits(g, epi) || g.ksplit < 1 || (epi == EPI_LOGITS && g.ksplit != 1)) return hipErrorInvalidValue;
  const int ntiles16 = gemm_ntiles(g, epi);
  const int units = gemm_chunk_tiles(g, epi) * g.ksplit;
  hipError_t e;
  if (g.wide && gemm_wide_takes(g, epi)) {
    e = launch_gemm_wide(g, epi, ntiles16, units, st);
    if (e != hipSuccess || g.ksplit <= 1) return e;
    return launch_gemm_reduce(g, epi, ntiles16, st);
  }
  const int mblocks = (g.M + CK_ROWS - 1) / CK_ROWS;
  const int blocks = (units + CK_XCDS - 1) / CK_XCDS * CK_XCDS * mblocks;
  switch (epi) {
    case EPI_STORE: e = launch_epi<EPI_STORE>(g, ntiles16, blocks, mblocks, st); break;
    case EPI_ADD: e = launch_epi<EPI_ADD>(g, ntiles16, blocks, mblocks, st); break;
    case EPI_SWIGLU: e = launch_epi<EPI_SWIGLU>(g, ntiles16, blocks, mblocks, st); break;
    case EPI_QKV: e = launch_epi<EPI_QKV>(g, ntiles16, blocks, mblocks, st); break;
    default: e = launch_epi<EPI_LOGITS>(g, ntiles16, blocks, mblocks, st); break;
  }
  if (e != hipSuccess || g.ksplit <= 1) return e;
  return launch_gemm_reduce(g, epi, ntiles16, st);
}

bool gemm_chunk_grouped_fits(const GemmArgs &g, int epi) {
  // each expert's slice of the stacked weights starts at a 32-row tile; the
  // SwiGLU up rows follow the expert's N gate rows
  const int64_t wrows = epi == EPI_SWIGLU ? 2 * (int64_t)g.N : g.N;
  return (epi == EPI_SWIGLU || epi == EPI_STORE) && g.Wp != nullptr && g.A != nullptr && g.x == nullptr &&
         g.n_groups != nullptr && g.group_expert != nullptr && g.group_start != nullptr &&
         g.group_count != nullptr && g.ksplit == 1 && g.N % 32 == 0 && pack_w32_fits(wrows, g.K) &&
         g.w_group_stride == wrows * g.K && (epi != EPI_SWIGLU || g.np_off == g.N);
}

hipError_t launch_gemm_chunk_grouped(const GemmArgs &g, int epi, int pairs, int group_slots, hipStream_t st) {
  if (!gemm_chunk_grouped_fits(g, epi) || pairs < 1 || group_slots < 1) return hipErrorInvalidValue;
  const int ntiles16 = gemm_ntiles(g, epi);
  // sum over groups of ceil(count / 32) <= (pairs + 31 groups) / 32
  const int64_t row_tiles = ((int64_t)pairs + 31 * (int64_t)std::min(group_slots, pairs)) / 32;
  const int64_t blocks = row_tiles * gemm_chunk_tiles(g, epi);
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU) return launch_mt<1, EPI_SWIGLU, true, false>(g, ntiles16, (int)blocks, 1, st);
  return launch_mt<1, EPI_STORE, true, false>(g, ntiles16, (int)blocks, 1, st);
}
