// Multi-row projection for prefill chunks: C[m][n] = sum_k A[m][k] W[n][k]
// for up to 128 activation rows (engine.zig Engine.prefill: a chunk of token
// columns shares one pass over every weight matrix; decoder.rs AttnWeights:
// weights are row-major [out][in]).
//
// gfx950 design.  A chunk projection streams each weight matrix once and
// does 2 M flops per weight element, so with M = 128 it sits on the HBM /
// MFMA ridge: the kernel must keep the weight stream at full HBM rate while
// the matrix cores do the arithmetic.
//  * Block = 4 waves.  Each wave owns 4 weight subtiles of 16 rows (64 rows;
//    for the paired epilogues two tiles and their partner rows) for all M
//    rows, so a weight fragment feeds MT MFMAs and the whole output tile of
//    the wave stays in its accumulators (MT x 4 16x16 fp32 tiles).
//  * Weights go straight from HBM into MFMA B-operand registers.  In a
//    64-wide k step lane l loads the 32 contiguous bytes at k0 + 16 (l / 16)
//    of each of its rows, so the 4 lane groups read each row's full 128-byte
//    line; MFMA j (0, 1) takes the 8 elements at k0 + 16 (l / 16) + 8 j.
//    The next step's weights are in flight while the current step computes
//    (loads are unconditional, past the k range they read zeros through the
//    buffer bound, so the compiler's wait counts stay exact).
//  * Activations (split bf16: hi and lo planes, two MFMAs per product) are
//    staged per k step into LDS by the whole block, in MFMA fragment order
//    with the same k mapping, so each fragment read is one conflict-free
//    64 x 16-byte ds_read.  Two LDS stages: the next step's activations are
//    loaded from L2 during the current step's MFMAs.
//  * Split-K across blocks (a block = one 256-row weight tile and one k
//    range) fills the 256 compute units when a matrix has few tiles;
//    partials go to Cpart and gemm_reduce sums them in fixed split order.
//    Without a split the epilogue runs straight from the accumulators.
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "epilogue.h"

namespace {

constexpr int CK_WAVES = 4;  // waves per block
constexpr int CK_SUB = 4;    // 16-row weight subtiles per wave
constexpr int CK_STEP = 64;  // k per pipeline step
constexpr int CK_ROWS = 64;  // activation rows per block (MT <= 4)
constexpr int CK_XCDS = 8;   // blocks are dispatched round-robin over 8 XCDs

template <int MT, bool SPLIT>
struct Stage {
  static constexpr int PLANES = SPLIT ? 2 : 1;
  static constexpr int PIECES = MT * 16 * 8 * PLANES;  // 16-byte pieces per stage
  static constexpr int PER_THREAD = (PIECES + CK_WAVES * WAVE - 1) / (CK_WAVES * WAVE);
};

// Global -> registers: this thread's pieces of the activation stage at k0
// (rows past M and k past K read zeros through the buffer bound `oob`).
template <int MT, bool SPLIT>
__device__ __forceinline__ void a_load(__amdgpu_buffer_rsrc_t ra, uint32_t oob, const GemmArgs &g, int rows, int k0,
                                       int kend, u32x4 (&ar)[Stage<MT, SPLIT>::PER_THREAD]) {
  constexpr int PER_PLANE = MT * 128;
#pragma unroll
  for (int i = 0; i < Stage<MT, SPLIT>::PER_THREAD; ++i) {
    const int e = threadIdx.x + i * CK_WAVES * WAVE;
    const int plane = e / PER_PLANE, rem = e - plane * PER_PLANE;
    const int r = rem >> 3, k = k0 + (rem & 7) * 8;
    const bool ok = (Stage<MT, SPLIT>::PIECES % (CK_WAVES * WAVE) == 0 || e < Stage<MT, SPLIT>::PIECES) && r < rows && k < kend;
    const uint32_t off = (uint32_t)((plane * g.a_lo + (int64_t)r * g.lda + k) * 2);
    ar[i] = buf_load16(ra, ok ? off : oob);
  }
}

// Registers -> LDS in fragment order: piece (row r, k offset kk, plane) goes
// to fragment (t = r / 16, j = (kk / 8) & 1, plane), lane r % 16 + 16 (kk / 16).
template <int MT, bool SPLIT>
__device__ __forceinline__ void a_store(u32x4 *dst, const u32x4 (&ar)[Stage<MT, SPLIT>::PER_THREAD]) {
  constexpr int PER_PLANE = MT * 128, PL = Stage<MT, SPLIT>::PLANES;
#pragma unroll
  for (int i = 0; i < Stage<MT, SPLIT>::PER_THREAD; ++i) {
    const int e = threadIdx.x + i * CK_WAVES * WAVE;
    const int plane = e / PER_PLANE, rem = e - plane * PER_PLANE;
    const int r = rem >> 3, kk = (rem & 7) * 8;
    const int t = r >> 4, j = (kk >> 3) & 1, ln = (r & 15) + 16 * (kk >> 4);
    if (Stage<MT, SPLIT>::PIECES % (CK_WAVES * WAVE) == 0 || e < Stage<MT, SPLIT>::PIECES)
      dst[((t * 2 + j) * PL + plane) * WAVE + ln] = ar[i];
  }
}

// This wave's weight fragments of the k step at k0: subtile p, half j
// (byte offsets wo[p] of the lane's row and k group; invalid rows carry `oob`).
template <int NSUB>
__device__ __forceinline__ void w_load(__amdgpu_buffer_rsrc_t rw, uint32_t oob, const uint32_t (&wo)[NSUB], int k0,
                                       int K, int q, u32x4 (&w)[NSUB][2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bool kok = k0 + 16 * q + 8 * j < K;
#pragma unroll
    for (int p = 0; p < NSUB; ++p) w[p][j] = buf_load16(rw, (kok && wo[p] != oob) ? wo[p] + (k0 + 8 * j) * 2 : oob);
  }
}

// One k step: for each (j, t) the A fragments (hi, lo) from LDS feed
// 4 (x2) MFMAs; the next pair's LDS reads are issued before the current
// MFMAs, and scheduling barriers keep the compiler from hoisting every read
// of the step (which would cost a register per read).
template <int MT, bool SPLIT>
__device__ __forceinline__ void mma_step(const u32x4 *src, const u32x4 (&w)[CK_SUB][2], int lane,
                                         f32x4 (&acc)[MT][CK_SUB]) {
  constexpr int PL = Stage<MT, SPLIT>::PLANES;
  u32x4 cur[PL], nxt[PL];
#pragma unroll
  for (int pl = 0; pl < PL; ++pl) cur[pl] = src[pl * WAVE + lane];
#pragma unroll
  for (int idx = 0; idx < 2 * MT; ++idx) {
    const int j = idx / MT, t = idx % MT;  // fragment (t, j) sits at (t * 2 + j) * PL
    if (idx + 1 < 2 * MT) {
      const int j1 = (idx + 1) / MT, t1 = (idx + 1) % MT;
#pragma unroll
      for (int pl = 0; pl < PL; ++pl) nxt[pl] = src[((t1 * 2 + j1) * PL + pl) * WAVE + lane];
    }
#pragma unroll
    for (int pl = 0; pl < PL; ++pl)
#pragma unroll
      for (int p = 0; p < CK_SUB; ++p) acc[t][p] = mfma16x16x32(as_bf16x8(cur[pl]), as_bf16x8(w[p][j]), acc[t][p]);
    __builtin_amdgcn_sched_barrier(0);
    if (idx + 1 < 2 * MT) {
#pragma unroll
      for (int pl = 0; pl < PL; ++pl) cur[pl] = nxt[pl];
    }
  }
}

// Block b -> (unit u = (weight tile, k split), row block mb): the row
// blocks of one unit are CK_XCDS block ids apart, so they are dispatched to
// the same XCD at about the same time and the second one finds the weights
// in that XCD's L2.
template <int MT, int EPI, bool SPLIT>
__global__ __launch_bounds__(CK_WAVES * WAVE, 2) void gemm_chunk_kernel(GemmArgs g, int ntiles16, int mblocks) {
  constexpr int NP = paired<EPI>();
  constexpr int LT = CK_SUB / NP;  // logical 16-row tiles per wave
  constexpr int PIECES = Stage<MT, SPLIT>::PIECES;
  __shared__ u32x4 a_s[2][PIECES];

  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int c = lane & 15, q = lane >> 4;
  const int K = g.K;
  const int nbt = (ntiles16 + CK_WAVES * LT - 1) / (CK_WAVES * LT);
  const int u = (blockIdx.x / (CK_XCDS * mblocks)) * CK_XCDS + blockIdx.x % CK_XCDS;
  const int mb = (blockIdx.x / CK_XCDS) % mblocks;
  if (u >= nbt * g.ksplit) return;
  const int bt = u % nbt, z = u / nbt;
  const int row0 = mb * CK_ROWS, rows = min(CK_ROWS, g.M - row0);
  const int nsteps = (K + CK_STEP - 1) / CK_STEP;
  const int per = (nsteps + g.ksplit - 1) / g.ksplit;
  const int s0 = min(nsteps, z * per), s1 = min(nsteps, s0 + per);

  // buffer resources: weights (all rows of the matrix) and the activation planes
  const int64_t wrows = EPI == EPI_SWIGLU ? 2 * (int64_t)g.N : g.N;
  const uint32_t w_oob = (uint32_t)(wrows * K * 2);
  const __amdgpu_buffer_rsrc_t rw = buf_rsrc(g.W, w_oob);
  const uint32_t a_oob = (uint32_t)(((SPLIT ? g.a_lo : 0) + (int64_t)g.M * g.lda) * 2);
  const __amdgpu_buffer_rsrc_t ra = buf_rsrc(g.A + (int64_t)row0 * g.lda, a_oob);

  // this wave's weight rows: subtile p = lt * NP + half
  uint32_t wo[CK_SUB];
  int tb[LT];
#pragma unroll
  for (int lt = 0; lt < LT; ++lt) {
    const int b = (bt * CK_WAVES + wave) * LT + lt;
    tb[lt] = b;
    const int n = b < ntiles16 ? tile_n0<EPI>(g, b) + c : 0;
    const bool ok = b < ntiles16 && (EPI == EPI_QKV || n < g.N);
#pragma unroll
    for (int h = 0; h < NP; ++h)
      wo[lt * NP + h] = ok ? (uint32_t)(((int64_t)(n + h * g.np_off) * K + 16 * q) * 2) : w_oob;
  }

  f32x4 acc[MT][CK_SUB];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int p = 0; p < CK_SUB; ++p) acc[t][p] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 w0[CK_SUB][2], w1[CK_SUB][2];
  u32x4 ar[Stage<MT, SPLIT>::PER_THREAD];
  const int kend = min(K, s1 * CK_STEP);
  if (s0 < s1) {
    a_load<MT, SPLIT>(ra, a_oob, g, rows, s0 * CK_STEP, kend, ar);
    w_load<CK_SUB>(rw, w_oob, wo, s0 * CK_STEP, kend, q, w0);
    a_store<MT, SPLIT>(a_s[0], ar);
  }
  __syncthreads();
  // Two steps per iteration, activation loads first (the wait before their
  // LDS store then leaves the newer weight loads in flight).  No conditional
  // loads: steps at or past s1 read zeros (k >= kend), so an odd step count
  // adds one zero step.
  for (int s = s0; s < s1; s += 2) {
    a_load<MT, SPLIT>(ra, a_oob, g, rows, (s + 1) * CK_STEP, kend, ar);
    w_load<CK_SUB>(rw, w_oob, wo, (s + 1) * CK_STEP, kend, q, w1);
    mma_step<MT, SPLIT>(a_s[0], w0, lane, acc);
    a_store<MT, SPLIT>(a_s[1], ar);
    __syncthreads();
    a_load<MT, SPLIT>(ra, a_oob, g, rows, (s + 2) * CK_STEP, kend, ar);
    w_load<CK_SUB>(rw, w_oob, wo, (s + 2) * CK_STEP, kend, q, w0);
    mma_step<MT, SPLIT>(a_s[1], w1, lane, acc);
    a_store<MT, SPLIT>(a_s[0], ar);
    __syncthreads();
  }

  // epilogue: lane (c, q) holds rows 16 t + 4 q + i, column c of each subtile
  const int64_t np_cols = (int64_t)ntiles16 * 16;
#pragma unroll
  for (int lt = 0; lt < LT; ++lt) {
    const int b = tb[lt];
    const bool bok = b < ntiles16;
    const int n = bok ? tile_n0<EPI>(g, b) + c : 0;
    const bool nok = bok && (EPI == EPI_QKV || n < g.N);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * t + 4 * q + i;
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
            // best (value, index) of this tile's 16 columns for row m: the
            // columns of a row sit in the 16 lanes that share q
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

template <int MT, int EPI>
hipError_t launch_mt(const GemmArgs &g, int ntiles16, int blocks, int mblocks, hipStream_t st) {
  if (g.a_lo)
    hipLaunchKernelGGL((gemm_chunk_kernel<MT, EPI, true>), dim3(blocks), dim3(CK_WAVES * WAVE), 0, st, g, ntiles16,
                       mblocks);
  else
    hipLaunchKernelGGL((gemm_chunk_kernel<MT, EPI, false>), dim3(blocks), dim3(CK_WAVES * WAVE), 0, st, g, ntiles16,
                       mblocks);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const GemmArgs &g, int ntiles16, int blocks, int mblocks, hipStream_t st) {
  const int mt = gemm_mtiles(std::min(g.M, CK_ROWS));
  switch (mt) {
    case 1: return launch_mt<1, EPI>(g, ntiles16, blocks, mblocks, st);
    case 2: return launch_mt<2, EPI>(g, ntiles16, blocks, mblocks, st);
    default: return launch_mt<4, EPI>(g, ntiles16, blocks, mblocks, st);
  }
}

}  // namespace

int gemm_chunk_tiles(const GemmArgs &g, int epi) {
  const int lt = (epi == EPI_SWIGLU || epi == EPI_QKV) ? CK_SUB / 2 : CK_SUB;
  return (gemm_ntiles(g, epi) + CK_WAVES * lt - 1) / (CK_WAVES * lt);
}

int gemm_chunk_mblocks(int rows) { return (rows + CK_ROWS - 1) / CK_ROWS; }

bool gemm_chunk_fits(const GemmArgs &g, int epi) {
  // byte offsets into the weight matrix and the activation planes are 32-bit
  const int64_t wrows = epi == EPI_SWIGLU ? 2 * (int64_t)g.N : g.N;
  const int64_t a_elems = (g.a_lo ? g.a_lo : 0) + (int64_t)g.M * g.lda;
  return g.M >= 1 && g.M <= 128 && g.A != nullptr && g.x == nullptr && g.n_groups == nullptr && g.a_rows == nullptr &&
         g.K % 8 == 0 && wrows * g.K * 2 < (int64_t)UINT32_MAX - 64 && a_elems * 2 < (int64_t)UINT32_MAX - 64;
}

hipError_t launch_gemm_chunk(const GemmArgs &g, int epi, hipStream_t st) {
  if (!gemm_chunk_fits(g, epi) || g.ksplit < 1 || (epi == EPI_LOGITS && g.ksplit != 1)) return hipErrorInvalidValue;
  const int ntiles16 = gemm_ntiles(g, epi);
  const int units = gemm_chunk_tiles(g, epi) * g.ksplit;
  const int mblocks = gemm_chunk_mblocks(g.M);
  const int blocks = (units + CK_XCDS - 1) / CK_XCDS * CK_XCDS * mblocks;
  hipError_t e;
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
