// Projection kernel: C[m][n] = sum_k A[m][k] W[n][k] for the QKV, o_proj,
// gate/up, down, router and lm-head products (engine.zig: every projection
// is a 1x1 conv y = W x per token column; decoder.rs AttnWeights: weights
// are row-major [out][in]).
//
// Design for gfx950 (weights are read exactly once per call, so the kernel
// is bound by HBM bandwidth for decode and small chunks):
//  * One block = 4 wavefronts = one 16-row tile of W (two tiles for the
//    SwiGLU epilogue: gate rows n and up rows n + N).  The 4 waves split the
//    K loop by interleaved 32-wide steps, so at every step the block reads
//    256 contiguous bytes of each weight row.
//  * Weight fragments go straight from HBM into MFMA B-operand registers
//    with 16-byte non-temporal loads (lane l reads row l % 16, k offset
//    8 (l / 16)); activations (tiny, L2-resident) are the A operand, MT
//    tiles of 16 rows each, so one weight fragment feeds MT MFMAs.
//  * v_mfma_f32_16x16x32_bf16 accumulates in fp32; the 4 partial tiles are
//    summed in LDS in fixed wave order (deterministic), then the epilogue
//    (store / residual add / SwiGLU) runs on the block's 256 threads.
//  * Optional split-K across blocks (blockIdx.z) writes fp32 partials that
//    gemm_reduce sums in fixed split order.
//  * Grouped mode (MoE experts): blockIdx.y selects a group (one expert and
//    a contiguous run of rows); the weight base moves to that expert.
#include "common.h"
#include "launch.h"

namespace {

constexpr int NWAVES = 4;

template <int MT, int NP, int U>
__device__ __forceinline__ void gemm_tile(const GemmArgs &g, const uint16_t *W, int row0, int rows,
                                          int mp, int n0, int s0, int s1, f32x4 (&acc)[MT][NP]) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  const int c = lane & 15, quad = lane >> 4;
  const int N = g.N, K = g.K;
  const bool nvalid = (n0 + c) < N;
  const uint16_t *wrow[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) wrow[p] = W + (int64_t)(n0 + c + p * N) * K + quad * 8;
  const uint16_t *arow[MT];
  bool mvalid[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    int m = mp + t * 16 + c;
    mvalid[t] = m < rows;
    int64_t src = 0;
    if (mvalid[t]) src = g.a_rows ? g.a_rows[row0 + m] : (row0 + m);
    arow[t] = g.A + src * g.lda + quad * 8;
  }
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int p = 0; p < NP; ++p) acc[t][p] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int st = s0 + wave; st < s1; st += NWAVES * U) {
    u32x4 wf[U][NP];
    u32x4 af[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int step = st + u * NWAVES;
      const int k = step * 32;
      const bool kv = (step < s1) && (k + quad * 8 < K);
#pragma unroll
      for (int p = 0; p < NP; ++p)
        wf[u][p] = (kv && nvalid) ? load_stream16(wrow[p] + k) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int t = 0; t < MT; ++t)
        af[u][t] = (kv && mvalid[t]) ? load16(arow[t] + k) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int p = 0; p < NP; ++p)
          acc[t][p] = mfma16x16x32(as_bf16x8(af[u][t]), as_bf16x8(wf[u][p]), acc[t][p]);
  }
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

template <int MT, int EPI, int U>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  constexpr int NP = (EPI == EPI_SWIGLU) ? 2 : 1;
  __shared__ f32x4 red[NWAVES][MT][NP][WAVE];

  const uint16_t *W = g.W;
  int row0 = 0, rows = g.M;
  if (g.n_groups) {
    const int gi = blockIdx.y;
    if (gi >= *g.n_groups) return;
    W += (int64_t)g.group_expert[gi] * g.w_group_stride;
    row0 = g.group_start[gi];
    rows = g.group_count[gi];
  }
  const int n0 = blockIdx.x * 16;
  const int steps = (g.K + 31) / 32;
  int s0 = 0, s1 = steps;
  if (g.ksplit > 1) {
    const int per = (steps + g.ksplit - 1) / g.ksplit;
    s0 = blockIdx.z * per;
    s1 = min(steps, s0 + per);
  }
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;

  for (int mp = 0; mp < rows; mp += 16 * MT) {
    f32x4 acc[MT][NP];
    gemm_tile<MT, NP, U>(g, W, row0, rows, mp, n0, s0, s1, acc);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int p = 0; p < NP; ++p) red[wave][t][p][lane] = acc[t][p];
    __syncthreads();
    // thread -> (lane', i): output row 4 (lane' / 16) + i of each m-tile, column lane' % 16
    const int ol = threadIdx.x >> 2, oi = threadIdx.x & 3;
    const int n = n0 + (ol & 15);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = mp + t * 16 + (ol >> 4) * 4 + oi;
      float v[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) s += red[w][t][p][ol][oi];
        v[p] = s;
      }
      if (m < rows && n < g.N) {
        const int64_t orow = row0 + m;
        if (g.ksplit > 1) {
          float *dst = g.Cpart + ((int64_t)blockIdx.z * g.M + orow) * (NP * g.N);
#pragma unroll
          for (int p = 0; p < NP; ++p) dst[n + p * g.N] = v[p];
        } else if (EPI == EPI_STORE) {
          g.C[orow * g.ldc + n] = v[0] + (g.bias ? g.bias[n] : 0.f);
        } else if (EPI == EPI_ADD) {
          g.C[orow * g.ldc + n] += v[0];
        } else {
          g.Hout[orow * g.ldc + n] = (uint16_t)f32_to_bf16_bits(silu_f(v[0]) * v[NP - 1]);
        }
      }
    }
    __syncthreads();
  }
}

template <int EPI>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmArgs g) {
  constexpr int NP = (EPI == EPI_SWIGLU) ? 2 : 1;
  const int64_t total = (int64_t)g.M * g.N;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = e / g.N;
    const int n = (int)(e - m * g.N);
    float v[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      float s = 0.f;
      for (int z = 0; z < g.ksplit; ++z) s += g.Cpart[((int64_t)z * g.M + m) * (NP * g.N) + n + p * g.N];
      v[p] = s;
    }
    if (EPI == EPI_STORE) {
      g.C[m * g.ldc + n] = v[0] + (g.bias ? g.bias[n] : 0.f);
    } else if (EPI == EPI_ADD) {
      g.C[m * g.ldc + n] += v[0];
    } else {
      g.Hout[m * g.ldc + n] = (uint16_t)f32_to_bf16_bits(silu_f(v[0]) * v[NP - 1]);
    }
  }
}

template <int MT, int EPI>
hipError_t launch_mt(const GemmArgs &g, dim3 grid, hipStream_t st) {
  constexpr int NP = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int U = (MT * 1 + NP) <= 3 ? 8 : ((MT + NP) <= 6 ? 4 : 2);
  hipLaunchKernelGGL((gemm_kernel<MT, EPI, U>), grid, dim3(256), 0, st, g);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const GemmArgs &g, int mt, dim3 grid, hipStream_t st) {
  switch (mt) {
    case 1: return launch_mt<1, EPI>(g, grid, st);
    case 2: return launch_mt<2, EPI>(g, grid, st);
    case 4: return launch_mt<4, EPI>(g, grid, st);
    default: return launch_mt<8, EPI>(g, grid, st);
  }
}

}  // namespace

int gemm_mtiles(int rows) {
  if (rows <= 16) return 1;
  if (rows <= 32) return 2;
  if (rows <= 64) return 4;
  return 8;
}

hipError_t launch_gemm(const GemmArgs &g_in, int epi, int max_rows, int n_group_slots,
                       hipStream_t st) {
  GemmArgs g = g_in;
  const int ntiles = (g.N + 15) / 16;
  const int mt = gemm_mtiles(max_rows);
  dim3 grid(ntiles, g.n_groups ? n_group_slots : 1, g.ksplit > 1 ? g.ksplit : 1);
  hipError_t e;
  if (epi == EPI_STORE) e = launch_epi<EPI_STORE>(g, mt, grid, st);
  else if (epi == EPI_ADD) e = launch_epi<EPI_ADD>(g, mt, grid, st);
  else e = launch_epi<EPI_SWIGLU>(g, mt, grid, st);
  if (e != hipSuccess || g.ksplit <= 1) return e;
  const int64_t total = (int64_t)g.M * g.N;
  int blocks = (int)std::min<int64_t>((total + 255) / 256, 4096);
  if (epi == EPI_STORE) hipLaunchKernelGGL(gemm_reduce_kernel<EPI_STORE>, dim3(blocks), dim3(256), 0, st, g);
  else if (epi == EPI_ADD) hipLaunchKernelGGL(gemm_reduce_kernel<EPI_ADD>, dim3(blocks), dim3(256), 0, st, g);
  else hipLaunchKernelGGL(gemm_reduce_kernel<EPI_SWIGLU>, dim3(blocks), dim3(256), 0, st, g);
  return hipGetLastError();
}
