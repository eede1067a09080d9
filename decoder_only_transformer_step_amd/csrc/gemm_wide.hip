// Multi-row projection for wide prefill chunks (256 to 512 rows):
// C[m][n] = sum_k A[m][k] W[n][k] (engine.zig Engine.prefill: a chunk of
// token columns shares one pass over every weight matrix; cortiq_engine
// pipeline.rs prefill_chunk(): tall panels keep the matrix units busy).
//
// gfx950 design: at 256+ rows the product is compute-bound, so the tile is
// sized for MFMA work per byte moved:
//  * Block = 8 waves (two per SIMD) over 256 activation rows x 256 weight
//    rows; wave (wm, wn) owns rows 128 wm .. and weight rows 64 wn .. : 4 x 2
//    tiles of 32 x 32 (v_mfma_f32_32x32x16_bf16), 128 fp32 accumulators per
//    lane.  (4 waves of 4 x 4 tiles need all 256 accumulation registers and
//    spill.)
//  * Both operands are staged per 32-wide k step into LDS (two stages of
//    48 KB): the activations (split bf16, hi and lo planes) in MFMA fragment
//    order with the XOR swizzle of the 64-row chunk kernel, the weights as
//    the packed 32-row x 16-k tiles of 1 KB (each tile is already one
//    fragment in lane order, so its copy and its reads are contiguous).
//    Every fragment is then one conflict-free 1 KB LDS read.
//  * Per 32-wide k step a wave issues 32 MFMAs (16 with one plane) against
//    20 fragment reads; the next step's global loads are in flight during
//    them.  Loads are unconditional (masked lanes read a zero page).
//  * Per MFMA a block moves half the global bytes of the 64-row kernel.
//  * Split-K and the epilogues are the chunk kernel's: partials in Cpart
//    reduced by gemm_reduce in split order, or epi_apply in place.  QKV
//    always goes through the partials (its bias, RoPE and cache-append
//    epilogue over 64 values per lane would spill here).
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "epilogue.h"

namespace {

constexpr int GW_WAVES = 8;
constexpr int GW_TJ = 2;     // 32-row weight tiles per wave
constexpr int GW_BM = 256;   // activation rows per block
constexpr int GW_TILES = 8;  // 32-row weight tiles per block (256 weight rows)
constexpr int GW_XCDS = 8;

__device__ u32x4 gw_zero[64];  // never written: zero-initialised

__device__ __forceinline__ int gw_swz(int r32, int g, int s) { return (r32 ^ (2 * (2 * s + g))) + 32 * g; }

template <bool SPLIT>
struct GwLay {
  static constexpr int PL = SPLIT ? 2 : 1;
  static constexpr int A_SLOTS = 2 * 8 * PL * WAVE;     // 2 k16 groups x 8 row tiles x planes x 64 lanes
  static constexpr int B_SLOTS = 2 * GW_TILES * WAVE;   // 2 k16 groups x 8 weight tiles x 64 lanes
  static constexpr int STAGE = A_SLOTS + B_SLOTS;       // 16-byte slots per stage
  static constexpr int AP = A_SLOTS / (GW_WAVES * WAVE);  // activation pieces per thread
  static constexpr int BP = B_SLOTS / (GW_WAVES * WAVE);  // weight pieces per thread
};

template <int EPI, bool SPLIT>
__global__ __launch_bounds__(GW_WAVES * WAVE, 1) void gemm_wide_kernel(GemmArgs g, int ntiles16, int mblocks) {
  using L = GwLay<SPLIT>;
  constexpr int PL = L::PL, NP = paired<EPI>();
  constexpr int LTB = GW_TILES / NP;  // logical 32-row tiles per block
  extern __shared__ u32x4 lds[];

  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE, wm = wave / 4, wn = wave % 4;
  const int K = g.K;
  const int ntiles32 = ntiles16 / 2;
  const int nbt = (ntiles32 + LTB - 1) / LTB;
  // block -> (unit u = (weight block, k split), row block mb): the row
  // blocks of one unit are GW_XCDS block ids apart (one XCD, one L2)
  const int u = (blockIdx.x / (GW_XCDS * mblocks)) * GW_XCDS + blockIdx.x % GW_XCDS;
  const int mb = (blockIdx.x / GW_XCDS) % mblocks;
  if (u >= nbt * g.ksplit) return;
  const int bt = u % nbt, z = u / nbt;
  const int row0 = mb * GW_BM, rows = min(GW_BM, g.M - row0);
  const int nsteps = (K + 31) / 32;
  const int per = (nsteps + g.ksplit - 1) / g.ksplit;
  const int s0 = min(nsteps, z * per), s1 = min(nsteps, s0 + per);
  const int kend = min(K, s1 * 32);
  const uint16_t *abase = g.A + (int64_t)row0 * g.lda;

  // weight staging: thread piece i = kilobyte tile chunk c = p / 64 of the
  // step (k16 group c % 2, block tile c / 2), lane p % 64 of it
  const uint16_t *wsrc[L::BP];
  bool wok[L::BP];
  int wdst[L::BP];
#pragma unroll
  for (int i = 0; i < L::BP; ++i) {
    const int p = threadIdx.x + i * GW_WAVES * WAVE, c = p / WAVE, lc = p % WAVE;
    const int kg = c & 1, j = c >> 1;
    const int T = bt * LTB + j / NP;  // logical tile, half j % NP
    const bool ok = T < ntiles32;
    const int r0 = ok ? tile_n0<EPI>(g, 2 * T) + (j % NP) * g.np_off : 0;
    wok[i] = ok;
    wsrc[i] = g.Wp + (int64_t)(r0 / 32) * (K / 16) * 512 + kg * 512 + lc * 8;
    wdst[i] = L::A_SLOTS + (kg * GW_TILES + j) * WAVE + lc;
  }
  // activation staging: piece (plane, row r, 16-byte chunk c4 of the step's
  // 64 bytes), 4 threads per row piece
  int adst[L::AP];
#pragma unroll
  for (int i = 0; i < L::AP; ++i) {
    const int p = threadIdx.x + i * GW_WAVES * WAVE;
    const int plane = p / (GW_BM * 4), rem = p % (GW_BM * 4), r = rem >> 2, c4 = rem & 3;
    const int kg = c4 >> 1, gk = c4 & 1;
    adst[i] = ((kg * 8 + (r >> 5)) * PL + plane) * WAVE + gw_swz(r & 31, gk, kg);
  }
  // two register sets: a step's loads go out two steps before its LDS store
  u32x4 ra0[L::AP], rb0[L::BP], ra1[L::AP], rb1[L::BP];
  auto gload = [&](int step, u32x4 (&ra)[L::AP], u32x4 (&rb)[L::BP]) {
    const int k0 = step * 32;
#pragma unroll
    for (int i = 0; i < L::AP; ++i) {
      const int p = threadIdx.x + i * GW_WAVES * WAVE;
      const int plane = p / (GW_BM * 4), rem = p % (GW_BM * 4), r = rem >> 2, c4 = rem & 3;
      const int k = k0 + c4 * 8;
      const bool ok = r < rows && k < kend;
      ra[i] = load16(ok ? static_cast<const void *>(abase + plane * g.a_lo + (int64_t)r * g.lda + k)
                        : static_cast<const void *>(gw_zero + lane));
    }
#pragma unroll
    for (int i = 0; i < L::BP; ++i) {
      const int kg = ((threadIdx.x + i * GW_WAVES * WAVE) / WAVE) & 1;
      const bool ok = wok[i] && k0 + 16 * kg < kend;
      rb[i] = load16(ok ? static_cast<const void *>(wsrc[i] + (int64_t)step * 1024)
                        : static_cast<const void *>(gw_zero + lane));
    }
  };
  auto sstore = [&](u32x4 *st, const u32x4 (&ra)[L::AP], const u32x4 (&rb)[L::BP]) {
#pragma unroll
    for (int i = 0; i < L::AP; ++i) st[adst[i]] = ra[i];
#pragma unroll
    for (int i = 0; i < L::BP; ++i) st[wdst[i]] = rb[i];
  };

  f32x16 acc[4][GW_TJ];
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int tj = 0; tj < GW_TJ; ++tj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[ti][tj][e] = 0.f;

  int sw[2];
#pragma unroll
  for (int kg = 0; kg < 2; ++kg) sw[kg] = gw_swz(lane & 31, lane >> 5, kg);
  // one 32-wide k step from stage st: per k16 group, the wave's 4 x PL
  // activation fragments and 4 weight fragments, then 16 x PL MFMAs
  auto mma = [&](const u32x4 *st) {
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
      u32x4 a[4][PL], b[GW_TJ];
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int pl = 0; pl < PL; ++pl) a[ti][pl] = st[((kg * 8 + wm * 4 + ti) * PL + pl) * WAVE + sw[kg]];
#pragma unroll
      for (int tj = 0; tj < GW_TJ; ++tj) b[tj] = st[L::A_SLOTS + (kg * GW_TILES + wn * GW_TJ + tj) * WAVE + lane];
#pragma unroll
      for (int pl = 0; pl < PL; ++pl)
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
          for (int tj = 0; tj < GW_TJ; ++tj)
            acc[ti][tj] = mfma32x32x16(as_bf16x8(a[ti][pl]), as_bf16x8(b[tj]), acc[ti][tj]);
    }
  };

  if (s0 < s1) {
    gload(s0, ra0, rb0);
    sstore(lds, ra0, rb0);
    gload(s0 + 1, ra0, rb0);
  }
  __syncthreads();
  // two steps per iteration, loads unconditional: steps at or past s1 read
  // zeros (k >= kend), so an odd step count adds one zero step
  for (int s = s0; s < s1; s += 2) {
    gload(s + 2, ra1, rb1);
    mma(lds);
    sstore(lds + L::STAGE, ra0, rb0);
    __syncthreads();
    gload(s + 3, ra0, rb0);
    mma(lds + L::STAGE);
    sstore(lds, ra1, rb1);
    __syncthreads();
  }

  // epilogue: physical tile tj of the wave is block tile j = GW_TJ wn + tj
  // (logical tile j / NP, half j % NP); lane l holds rows
  // 32 t + 8 (i / 4) + 4 (l / 32) + i % 4 of column l % 32, i.e. logical
  // 16-row tile 2 T + (l % 32) / 16, column l % 16
  const int64_t np_cols = (int64_t)ntiles16 * 16;
  const int c = lane & 15;
#pragma unroll
  for (int tj = 0; tj < GW_TJ; tj += NP) {
    const int j = wn * GW_TJ + tj;
    const int T = bt * LTB + j / NP;
    const int b = 2 * T + ((lane >> 4) & 1);
    const bool bok = T < ntiles32;
    const int n = bok ? tile_n0<EPI>(g, b) + c : 0;
    const bool nok = bok && (EPI == EPI_QKV || n < g.N);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = 32 * (wm * 4 + ti) + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        const float v0 = acc[ti][tj][i], v1 = acc[ti][tj + NP - 1][i];
        if (!(nok && m < rows)) continue;
        if (g.ksplit > 1 || EPI == EPI_QKV) {  // QKV: partials only (gemm_reduce applies its epilogue)
          float *dst = g.Cpart + ((int64_t)z * g.M + row0 + m) * NP * np_cols + (int64_t)b * 16 + c;
          dst[0] = v0;
          if (NP == 2) dst[np_cols] = v1;
        } else {
          epi_apply<EPI>(g, row0 + m, n, v0, v1);
        }
      }
    }
  }
}

template <int EPI, bool SPLIT>
hipError_t gw_launch(const GemmArgs &g, int ntiles16, int blocks, int mblocks, hipStream_t st) {
  constexpr size_t bytes = 2 * (size_t)GwLay<SPLIT>::STAGE * sizeof(u32x4);
  static bool attr = false;
  if (!attr) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_wide_kernel<EPI, SPLIT>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((gemm_wide_kernel<EPI, SPLIT>), dim3(blocks), dim3(GW_WAVES * WAVE), bytes, st, g, ntiles16,
                     mblocks);
  return hipGetLastError();
}

template <int EPI>
hipError_t gw_launch_e(const GemmArgs &g, int ntiles16, int blocks, int mblocks, hipStream_t st) {
  return g.a_lo ? gw_launch<EPI, true>(g, ntiles16, blocks, mblocks, st)
                : gw_launch<EPI, false>(g, ntiles16, blocks, mblocks, st);
}

}  // namespace

int gemm_wide_mblocks(int rows) { return (rows + GW_BM - 1) / GW_BM; }

bool gemm_wide_takes(const GemmArgs &g, int epi) {
  return g.M >= GEMM_WIDE_MIN_ROWS && epi != EPI_LOGITS && g.K % 32 == 0 && !(epi == EPI_QKV && g.ksplit <= 1);
}

// Launch over `units` (weight blocks x k splits) and the row blocks; the
// caller checked gemm_chunk_fits and sets g.ksplit.
hipError_t launch_gemm_wide(const GemmArgs &g, int epi, int ntiles16, int units, hipStream_t st) {
  const int mblocks = gemm_wide_mblocks(g.M);
  const int blocks = (units + GW_XCDS - 1) / GW_XCDS * GW_XCDS * mblocks;
  switch (epi) {
    case EPI_STORE: return gw_launch_e<EPI_STORE>(g, ntiles16, blocks, mblocks, st);
    case EPI_ADD: return gw_launch_e<EPI_ADD>(g, ntiles16, blocks, mblocks, st);
    case EPI_SWIGLU: return gw_launch_e<EPI_SWIGLU>(g, ntiles16, blocks, mblocks, st);
    case EPI_QKV: return gw_launch_e<EPI_QKV>(g, ntiles16, blocks, mblocks, st);
    default: return hipErrorInvalidValue;
  }
}
