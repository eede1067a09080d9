// Projection of 2-8 activation rows with bf16 weights: C[m][n] = sum_k A[m][k] W[n][k],
// each weight row streamed once for all rows (pipeline.rs forward_pair and
// measure_pair_fusion: one pass over the weights serves a drafted position
// together with the current one; pipeline.rs module doc: a small batch of
// sequences decodes in one pass the same way).
//
// gfx950 design: the access shape of the batch-1 GEMV (every wave load
// instruction reads one contiguous kilobyte of a weight row), with the
// activations of all M rows held in registers instead of LDS:
//  * K is split over the block's waves in 512-element steps: wave w owns
//    steps w SPW .. w SPW + SPW - 1 of every weight row and keeps the fp32
//    activations of those steps, for all M rows, in registers (8 per lane,
//    row and step).  A 16-byte weight load then feeds 8 M FMAs with no LDS
//    read; an LDS-resident activation needs 2 M LDS reads per weight load.
//  * The block walks groups of 8 weight rows (8 items, or 4 row pairs for
//    the paired epilogues; 4 rows where the activations take more
//    registers), one step at a time through two register buffers, so the next stage's loads are in flight during the current
//    stage's FMAs.
//  * After a group, each lane holds 8 M (or 4 M) partial sums.  They are reduced
//    across the wave by halving exchanges (each round a lane keeps half of
//    its values and adds its partner's copy of them: 8 M - 1 shuffles leave
//    one finished value per lane, against 6 per value for separate
//    butterflies), then across the waves through LDS in wave order, so the
//    result does not depend on scheduling.
//  * Prologue: the fused RMSNorm (x and gamma: per-row sums of squares over
//    the block's waves, then each wave scales its own slice) or split-bf16
//    activations (hi + lo).  Epilogues as the other multi-row kernels
//    (epi_apply); with EPI_LOGITS each block also leaves its best (value,
//    index) per row for the argmax pass.
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "epilogue.h"

namespace {

constexpr int GR_MAXW = 8;  // waves per block

// weight rows per group: 8, or 4 where 4 rows' activations over 4 steps
// per wave would not leave room for two 8-row stage buffers
template <int MR, int SPW>
constexpr int gr_rg() {
  return MR * SPW >= 16 ? 4 : 8;
}

__device__ u32x4 gr_zero[64];  // never written: zero-initialised

// weight rows of item `it` (as the batch-1 GEMV pairs them)
template <int EPI>
__device__ __forceinline__ void gr_item_rows(const GemmArgs &g, int it, int &r0, int &r1) {
  if (EPI == EPI_QKV) {
    const int half = g.qkv.d / 2;
    const int hh = it / half, i = it - hh * half;
    r0 = hh * g.qkv.d + i;
    r1 = r0 + half;
  } else if (EPI == EPI_SWIGLU) {
    r0 = it;
    r1 = it + g.np_off;
  } else {
    r0 = r1 = it;
  }
}

// Element offsets of the group's RG weight rows (row r: item gi IG + r / NR,
// half r % NR); rows of items past n_items are marked -1.
template <int EPI, int RG>
__device__ __forceinline__ void gr_rows(const GemmArgs &g, int gi, int n_items, int64_t (&off)[RG]) {
  constexpr int NR = paired<EPI>(), IG = RG / NR;
#pragma unroll
  for (int q = 0; q < IG; ++q) {
    const int it = gi * IG + q;
    int r0, r1;
    gr_item_rows<EPI>(g, it < n_items ? it : 0, r0, r1);
#pragma unroll
    for (int h = 0; h < NR; ++h) off[q * NR + h] = it < n_items ? (int64_t)(h ? r1 : r0) * g.K : -1;
  }
}

// Loads of one stage: step s of the group's rows (lanes past K and invalid
// rows read the zero page, so no load sits under a branch).
template <int RG>
__device__ __forceinline__ void gr_load(const GemmArgs &g, const int64_t (&off)[RG], int s, int lane,
                                        u32x4 (&w)[RG]) {
  const int k = s * 512 + lane * 8;
#pragma unroll
  for (int r = 0; r < RG; ++r)
    w[r] = load16_nt(off[r] >= 0 && k < g.K ? static_cast<const void *>(g.W + off[r] + k)
                                          : static_cast<const void *>(gr_zero + lane));
}

template <int RG, int MR>
__device__ __forceinline__ void gr_fma(float (&acc)[RG][MR], const u32x4 (&w)[RG], const float (&a)[MR][8]) {
#pragma unroll
  for (int r = 0; r < RG; ++r) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float t = acc[r][m];
      t = fmaf(bf16_lo(w[r][0]), a[m][0], t);
      t = fmaf(bf16_hi(w[r][0]), a[m][1], t);
      t = fmaf(bf16_lo(w[r][1]), a[m][2], t);
      t = fmaf(bf16_hi(w[r][1]), a[m][3], t);
      t = fmaf(bf16_lo(w[r][2]), a[m][4], t);
      t = fmaf(bf16_hi(w[r][2]), a[m][5], t);
      t = fmaf(bf16_lo(w[r][3]), a[m][6], t);
      t = fmaf(bf16_hi(w[r][3]), a[m][7], t);
      acc[r][m] = t;
    }
  }
}

template <int EPI, int MR, int SPW>
__global__ __launch_bounds__(GR_MAXW * WAVE) void gemv_rows_kernel(GemmArgs g, int n_items) {
  constexpr int RG = gr_rg<MR, SPW>(), NR = paired<EPI>(), IG = RG / NR, V = RG * MR;
  constexpr int LV = V == 8 ? 3 : V == 16 ? 4 : V == 32 ? 5 : 6;  // log2 V
  constexpr int GPI = SPW == 1 ? 2 : 1;             // groups per iteration: an even number of stages
  static_assert(V == (1 << LV), "RG M values per lane");
  __shared__ float red[2][GR_MAXW][V];
  __shared__ float ssr[GR_MAXW][MR];
  __shared__ float lbv[GR_MAXW * WAVE];
  __shared__ int lbi[GR_MAXW * WAVE];

  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int nw = blockDim.x / WAVE;
  const int K = g.K;
  const int ngrp = (n_items + IG - 1) / IG;
  const int s0 = wave * SPW;  // this wave's first step

  // activation slice: a[j][m][e] = row m at k = (s0 + j) 512 + 8 lane + e
  // (rows past M and k past K are zero)
  float a[SPW][MR][8];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int k = (s0 + j) * 512 + lane * 8;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const bool ok = m < g.M && k < K;
      if (g.x) {
        const float *src = ok ? g.x + (int64_t)m * g.lda + k : reinterpret_cast<const float *>(gr_zero + lane);
        const f32x4 v0 = loadf4(src), v1 = loadf4(ok ? src + 4 : src);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[j][m][e] = v0[e];
          a[j][m][4 + e] = v1[e];
        }
      } else {
        const uint16_t *hp = g.A + (int64_t)m * g.lda + k;
        const u32x4 h = load16(ok ? static_cast<const void *>(hp) : static_cast<const void *>(gr_zero + lane));
        const u32x4 l = load16(ok && g.a_lo ? static_cast<const void *>(hp + g.a_lo)
                                            : static_cast<const void *>(gr_zero + lane));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[j][m][2 * e] = bf16_lo(h[e]) + bf16_lo(l[e]);
          a[j][m][2 * e + 1] = bf16_hi(h[e]) + bf16_hi(l[e]);
        }
      }
    }
  }
  if (g.x) {
    // RMSNorm (engine.zig rmsnormColumn): per-row mean square over the
    // block's waves in wave order, then (x * inv) * gamma on this slice
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < SPW; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += a[j][m][e] * a[j][m][e];
      ss = wave_sum(ss);
      if (lane == 0) ssr[wave][m] = ss;
    }
    __syncthreads();
    float inv[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float t = 0.f;
      for (int w = 0; w < nw; ++w) t += ssr[w][m];
      inv[m] = 1.0f / sqrtf(t / (float)K + g.eps);
    }
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int k = (s0 + j) * 512 + lane * 8;
      const float *gp = k < K ? g.gamma + k : reinterpret_cast<const float *>(gr_zero + lane);
      const f32x4 g0 = loadf4(gp), g1 = loadf4(k < K ? gp + 4 : gp);
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[j][m][e] = (a[j][m][e] * inv[m]) * g0[e];
          a[j][m][4 + e] = (a[j][m][4 + e] * inv[m]) * g1[e];
        }
    }
  }

  // this thread's epilogue slot (item q of the group, row m) and, for the
  // logits, its running best over the block's groups
  const int tq = threadIdx.x / MR, tm = threadIdx.x % MR;
  float bv = -INFINITY;
  int bi = 0x7fffffff;

  int64_t off[RG], offn[RG];
  u32x4 wA[RG], wB[RG];
  int gi = blockIdx.x;
  gr_rows<EPI, RG>(g, gi < ngrp ? gi : ngrp, n_items, off);
  gr_load(g, off, s0, lane, wA);
  int buf = 0;

  // one group: its SPW stages (the first in `first`), then the reductions
  auto group = [&](int gcur, u32x4 (&first)[RG], u32x4 (&second)[RG]) {
    float acc[RG][MR];
#pragma unroll
    for (int r = 0; r < RG; ++r)
#pragma unroll
      for (int m = 0; m < MR; ++m) acc[r][m] = 0.f;
    const int gnext = gcur + (int)gridDim.x;
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      u32x4 (&cur)[RG] = (j & 1) ? second : first;
      u32x4 (&nxt)[RG] = (j & 1) ? first : second;
      if (j + 1 < SPW) {
        gr_load(g, off, s0 + j + 1, lane, nxt);
      } else {
        // the next group's first stage (a block past the last group reads
        // the zero page: every row marked invalid)
        gr_rows<EPI, RG>(g, gnext < ngrp ? gnext : ngrp, n_items, offn);
        gr_load(g, offn, s0, lane, nxt);
      }
      gr_fma<RG, MR>(acc, cur, a[j]);
    }
    // reduce across the wave: value i = r MR + m; after round q a lane keeps
    // the half selected by its bit (32 >> q), so it ends with value
    // lane >> (6 - LV)
    float v[V];
#pragma unroll
    for (int r = 0; r < RG; ++r)
#pragma unroll
      for (int m = 0; m < MR; ++m) v[r * MR + m] = acc[r][m];
#pragma unroll
    for (int q = 0; q < LV; ++q) {
      const int d = 32 >> q, n = V >> q;
      const bool up = (lane & d) != 0;
#pragma unroll
      for (int i = 0; i < n / 2; ++i) {
        const float send = up ? v[i] : v[i + n / 2];
        const float keep = up ? v[i + n / 2] : v[i];
        v[i] = keep + __shfl_xor(send, d, WAVE);
      }
    }
#pragma unroll
    for (int d = 32 >> LV; d >= 1; d >>= 1) v[0] += __shfl_xor(v[0], d, WAVE);
    if ((lane & ((64 >> LV) - 1)) == 0) red[buf][wave][lane >> (6 - LV)] = v[0];
    __syncthreads();
    // across the waves, in wave order, then the epilogue
    if (threadIdx.x < IG * MR) {
      float v0 = 0.f, v1 = 0.f;
      for (int w = 0; w < nw; ++w) {
        v0 += red[buf][w][(tq * NR) * MR + tm];
        if (NR == 2) v1 += red[buf][w][(tq * NR + 1) * MR + tm];
      }
      const int it = gcur * IG + tq;
      if (it < n_items && tm < g.M) {
        int r0, r1;
        gr_item_rows<EPI>(g, it, r0, r1);
        epi_apply<EPI>(g, tm, r0, v0, NR == 2 ? v1 : v0);
        if (EPI == EPI_LOGITS && better(v0, r0, bv, bi)) {
          bv = v0;
          bi = r0;
        }
      }
    }
    buf ^= 1;
#pragma unroll
    for (int r = 0; r < RG; ++r) off[r] = offn[r];
  };

  for (; gi < ngrp; gi += GPI * (int)gridDim.x) {
    if (SPW & 1) {
      group(gi, wA, wB);
      if (GPI == 2 && gi + (int)gridDim.x < ngrp) group(gi + (int)gridDim.x, wB, wA);
    } else {
      group(gi, wA, wB);
    }
  }

  if (EPI == EPI_LOGITS) {
    // this block's best (value, index) per row, over its groups' items
    lbv[threadIdx.x] = threadIdx.x < IG * MR ? bv : -INFINITY;
    lbi[threadIdx.x] = threadIdx.x < IG * MR ? bi : 0x7fffffff;
    __syncthreads();
    if (threadIdx.x < MR && (int)threadIdx.x < g.M) {
      float b = -INFINITY;
      int ix = 0x7fffffff;
      for (int q = 0; q < IG; ++q)
        if (better(lbv[q * MR + threadIdx.x], lbi[q * MR + threadIdx.x], b, ix)) {
          b = lbv[q * MR + threadIdx.x];
          ix = lbi[q * MR + threadIdx.x];
        }
      g.am.part_val[(int64_t)threadIdx.x * gridDim.x + blockIdx.x] = b;
      g.am.part_idx[(int64_t)threadIdx.x * gridDim.x + blockIdx.x] = ix;
    }
  }
}

// steps per wave for K (at most 8 waves per block), 0 if K is too long
int gr_spw(int K, int mr) {
  const int nsteps = (K + 511) / 512;
  const int spw = nsteps <= GR_MAXW ? 1 : nsteps <= 2 * GR_MAXW ? 2 : nsteps <= 4 * GR_MAXW ? 4 : 0;
  if (mr == 8 && spw != 1) return 0;  // 8 rows keep one step per wave (registers)
  return spw;
}

int gr_mr(int M) { return M <= 2 ? 2 : M <= 4 ? 4 : 8; }

int gr_items(const GemmArgs &g, int epi) { return epi == EPI_QKV ? g.N / 2 : g.N; }

int gr_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    hipDeviceProp_t p;
    cus = (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&p, dev) == hipSuccess) ? p.multiProcessorCount : 256;
  }
  return cus;
}

// Blocks of `waves` waves of the instantiation that fit one compute unit
// (registers decide), asked of the runtime once per instantiation and size.
template <int EPI, int MR, int SPW>
int gr_fit(int waves) {
  static int fit[GR_MAXW + 1] = {};
  if (!fit[waves]) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemv_rows_kernel<EPI, MR, SPW>, waves * WAVE, 0) != hipSuccess)
      n = 1;
    fit[waves] = std::max(1, n);
  }
  return fit[waves];
}

template <int EPI, int MR>
int gr_fit_spw(int spw, int waves) {
  if (spw == 1) return gr_fit<EPI, MR, 1>(waves);
  if constexpr (MR != 8) return spw == 2 ? gr_fit<EPI, MR, 2>(waves) : gr_fit<EPI, MR, 4>(waves);
  return 1;
}

int gr_fit_epi(int epi, int mr, int spw, int waves) {
  auto by_mr = [&](auto f2, auto f4, auto f8) { return mr == 2 ? f2() : mr == 4 ? f4() : f8(); };
  switch (epi) {
#define GR_FIT_CASE(E)                                                                                    \
  case E:                                                                                                 \
    return by_mr([&] { return gr_fit_spw<E, 2>(spw, waves); }, [&] { return gr_fit_spw<E, 4>(spw, waves); }, \
                 [&] { return gr_fit_spw<E, 8>(spw, waves); });
    GR_FIT_CASE(EPI_STORE)
    GR_FIT_CASE(EPI_ADD)
    GR_FIT_CASE(EPI_SWIGLU)
    GR_FIT_CASE(EPI_QKV)
    GR_FIT_CASE(EPI_LOGITS)
#undef GR_FIT_CASE
    default: return 1;
  }
}

template <int EPI, int MR>
void gr_launch_spw(const GemmArgs &g, int spw, int waves, int grid, hipStream_t st) {
  const int n_items = gr_items(g, EPI);
  if (spw == 1) {
    hipLaunchKernelGGL((gemv_rows_kernel<EPI, MR, 1>), dim3(grid), dim3(waves * WAVE), 0, st, g, n_items);
  } else if constexpr (MR != 8) {  // 8 rows keep one step per wave
    if (spw == 2) hipLaunchKernelGGL((gemv_rows_kernel<EPI, MR, 2>), dim3(grid), dim3(waves * WAVE), 0, st, g, n_items);
    else hipLaunchKernelGGL((gemv_rows_kernel<EPI, MR, 4>), dim3(grid), dim3(waves * WAVE), 0, st, g, n_items);
  }
}

template <int EPI>
void gr_launch_mr(const GemmArgs &g, int mr, int spw, int waves, int grid, hipStream_t st) {
  if (mr == 2) gr_launch_spw<EPI, 2>(g, spw, waves, grid, st);
  else if (mr == 4) gr_launch_spw<EPI, 4>(g, spw, waves, grid, st);
  else gr_launch_spw<EPI, 8>(g, spw, waves, grid, st);
}

}  // namespace

bool gemv_rows_takes(int rows, int K) {
  return rows >= 2 && rows <= GEMV_ROWS_MAX && K >= 8 && K % 8 == 0 && gr_spw(K, gr_mr(rows)) != 0;
}

bool gemv_rows_fits(const GemmArgs &g, int epi) {
  if (!gemv_rows_takes(g.M, g.K) || !g.W || g.Wq || g.n_groups || g.a_rows) return false;
  if (g.x ? !g.gamma : !g.A) return false;
  if (epi == EPI_QKV) return g.qkv.row_pos && g.qkv.row_seq && g.qkv.d % 2 == 0 && g.N % 2 == 0;
  if (epi == EPI_SWIGLU) return g.Hout && g.np_off == g.N;
  if (epi == EPI_LOGITS) return g.C && g.am.part_val && g.am.part_idx;
  return (epi == EPI_STORE || epi == EPI_ADD) && g.C;
}

int gemv_rows_grid(const GemmArgs &g, int epi) {
  const int mr = gr_mr(g.M), spw = gr_spw(g.K, mr);
  const int waves = ((g.K + 511) / 512 + spw - 1) / spw;
  const int rg = mr * spw >= 16 ? 4 : 8;  // gr_rg
  const int ig = rg / ((epi == EPI_SWIGLU || epi == EPI_QKV) ? 2 : 1);
  const int ngrp = (gr_items(g, epi) + ig - 1) / ig;
  // as many blocks as the compute units hold at once (the blocks loop over
  // the groups); logits: at most one argmax partial per row and 16 columns,
  // the count the partial buffers hold for the one-tile GEMM
  int grid = std::max(1, std::min(ngrp, gr_cus() * gr_fit_epi(epi, mr, spw, waves)));
  if (epi == EPI_LOGITS) grid = std::min(grid, (g.N + 15) / 16);
  return grid;
}

hipError_t launch_gemv_rows(const GemmArgs &g, int epi, hipStream_t st) {
  if (!gemv_rows_fits(g, epi)) return hipErrorInvalidValue;
  const int mr = gr_mr(g.M), spw = gr_spw(g.K, mr);
  const int waves = ((g.K + 511) / 512 + spw - 1) / spw;
  const int grid = gemv_rows_grid(g, epi);
  switch (epi) {
    case EPI_STORE: gr_launch_mr<EPI_STORE>(g, mr, spw, waves, grid, st); break;
    case EPI_ADD: gr_launch_mr<EPI_ADD>(g, mr, spw, waves, grid, st); break;
    case EPI_SWIGLU: gr_launch_mr<EPI_SWIGLU>(g, mr, spw, waves, grid, st); break;
    case EPI_QKV: gr_launch_mr<EPI_QKV>(g, mr, spw, waves, grid, st); break;
    default: gr_launch_mr<EPI_LOGITS>(g, mr, spw, waves, grid, st); break;
  }
  return hipGetLastError();
}
