// Projection kernel: C[m][n] = sum_k A[m][k] W[n][k] for the QKV, o_proj,
// gate/up, down, router, expert and lm-head products (engine.zig: every
// projection is a 1x1 conv y = W x per token column; decoder.rs AttnWeights:
// weights are row-major [out][in]).
//
// Design for gfx950 (weights are read exactly once per call, so the kernel
// is bound by HBM bandwidth for decode and small chunks):
//  * One block = NW wavefronts = one 16-row tile of W (two tiles for the
//    paired epilogues: SwiGLU gate rows n and up rows n + N; QKV rows i and
//    i + d/2 of a head, the two halves RoPE rotates together).  The waves
//    split the K loop by interleaved 32-wide steps, so at every step the
//    block reads NW * 64 contiguous bytes of each weight row.
//  * Weight fragments go straight from HBM into MFMA B-operand registers
//    with 16-byte loads (lane l reads row l % 16 at k offset
//    8 (l / 16)); activations are the A operand, MT tiles of 16 rows, so one
//    weight fragment feeds MT MFMAs (v_mfma_f32_16x16x32_bf16, fp32 acc).
//  * A comes from global memory (L2-resident), or, for decode, is built once
//    per block in LDS by the fused RMSNorm prologue (engine.zig rmsnormColumn:
//    x / sqrt(mean(x^2) + eps) * g, in fp32, then stored as split bf16: a hi
//    plane bf16(v) and a lo plane bf16(v - hi), each multiplied by the
//    weight fragment, so the MFMA input keeps about 16 mantissa bits).
//  * The NW partial tiles are summed in LDS in fixed wave order
//    (deterministic); the epilogue (store / residual add / SwiGLU / bias +
//    RoPE + KV append / logits with per-tile argmax candidates) runs on 256
//    threads.
//  * Optional split-K across blocks (blockIdx.z) writes fp32 partials that
//    gemm_reduce sums in fixed split order and then applies the epilogue.
//  * Grouped mode (MoE experts): blockIdx.y selects a group (one expert and
//    a contiguous run of rows); the weight base moves to that expert.
#include "common.h"
#include "launch.h"
#include "epilogue.h"

namespace {

// Accumulate this wave's share of the block tile.  AMODE 0: A from global;
// AMODE 2: A from the normalised copy in LDS (row m at a_lds + m * K, lo
// plane at a_lo).  SPLIT: A carries a lo plane, multiplied as well.
// int8 weights: 8 codes (8 bytes) -> 8 bf16 values, exactly (|q| <= 127
// has 7 significant bits, so the fp32 conversion's top half is the bf16).
__device__ __forceinline__ u32x4 i8x8_to_bf16(u32x2 w) {
  u32x4 o;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t v = w[h];
    const uint32_t f0 = __float_as_uint((float)(int8_t)(v & 0xFFu));
    const uint32_t f1 = __float_as_uint((float)(int8_t)((v >> 8) & 0xFFu));
    const uint32_t f2 = __float_as_uint((float)(int8_t)((v >> 16) & 0xFFu));
    const uint32_t f3 = __float_as_uint((float)(int8_t)(v >> 24));
    o[2 * h] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
    o[2 * h + 1] = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
  }
  return o;
}

template <int MT, int NP, int U, int NW, int AMODE, bool SPLIT, bool QW>
__device__ __forceinline__ void gemm_tile(const GemmArgs &g, const void *Wv, const uint16_t *a_lds,
                                          int64_t a_lo, int row0, int rows, int mp, int n0, bool nvalid,
                                          int s0, int s1, f32x4 (&acc)[MT][NP]) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  const int c = lane & 15, quad = lane >> 4;
  const int K = g.K;
  const uint16_t *wrow[NP];
  const int8_t *qrow[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    wrow[p] = static_cast<const uint16_t *>(Wv) + (int64_t)(n0 + c + p * g.np_off) * K + quad * 8;
    qrow[p] = static_cast<const int8_t *>(Wv) + (int64_t)(n0 + c + p * g.np_off) * K + quad * 8;
  }
  const uint16_t *arow[MT];
  bool mvalid[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = mp + t * 16 + c;
    mvalid[t] = m < rows;
    if (AMODE == 2) {
      arow[t] = a_lds + (int64_t)(mvalid[t] ? m : 0) * K + quad * 8;
    } else {
      int64_t src = 0;
      if (mvalid[t]) src = g.a_rows ? g.a_rows[row0 + m] : (row0 + m);
      arow[t] = g.A + src * g.lda + quad * 8;
    }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int p = 0; p < NP; ++p) acc[t][p] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int NS = SPLIT ? 2 : 1;
  if constexpr (QW) {
    // int8 codes: a 64-wide step is two MFMA k groups whose k are permuted
    // so that lane l's 16 codes of a row are contiguous (k = 64 s + 16 q +
    // 0..15, group 0 taking the first 8, group 1 the last 8); the
    // activation fragments follow the same permutation, and a dot product
    // does not depend on the order of its terms.  Each load instruction of a
    // wave then reads 16 rows x 64 contiguous bytes, as the bf16 path does.
    constexpr int UQ = U >= 2 ? U / 2 : 1;
    for (int st = s0 + wave; st < s1; st += NW * UQ) {
      u32x4 wf[UQ][2][NP];
      u32x4 af[UQ][2][MT][NS];
#pragma unroll
      for (int u = 0; u < UQ; ++u) {
        const int step = st + u * NW;
        const int k = step * 64 + quad * 8;  // + the row pointers' quad * 8: 64 s + 16 q
        const bool kv = (step < s1) && (step * 64 + quad * 16 < K);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const u32x4 raw = (kv && nvalid) ? load16_nt(qrow[p] + k) : u32x4{0u, 0u, 0u, 0u};
          wf[u][0][p] = i8x8_to_bf16(u32x2{raw[0], raw[1]});
          wf[u][1][p] = i8x8_to_bf16(u32x2{raw[2], raw[3]});
        }
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int sp = 0; sp < NS; ++sp) {
            af[u][0][t][sp] = (kv && mvalid[t]) ? load16(arow[t] + sp * a_lo + k) : u32x4{0u, 0u, 0u, 0u};
            af[u][1][t][sp] = (kv && mvalid[t]) ? load16(arow[t] + sp * a_lo + k + 8) : u32x4{0u, 0u, 0u, 0u};
          }
      }
#pragma unroll
      for (int u = 0; u < UQ; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int p = 0; p < NP; ++p)
#pragma unroll
              for (int sp = 0; sp < NS; ++sp)
                acc[t][p] = mfma16x16x32(as_bf16x8(af[u][h][t][sp]), as_bf16x8(wf[u][h][p]), acc[t][p]);
    }
    return;
  }
  for (int st = s0 + wave; st < s1; st += NW * U) {
    u32x4 wf[U][NP];
    u32x4 af[U][MT][NS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int step = st + u * NW;
      const int k = step * 32;
      const bool kv = (step < s1) && (k + quad * 8 < K);
#pragma unroll
      for (int p = 0; p < NP; ++p) wf[u][p] = (kv && nvalid) ? load16_nt(wrow[p] + k) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int sp = 0; sp < NS; ++sp)
          af[u][t][sp] = (kv && mvalid[t]) ? load16(arow[t] + sp * a_lo + k) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
          for (int sp = 0; sp < NS; ++sp)
            acc[t][p] = mfma16x16x32(as_bf16x8(af[u][t][sp]), as_bf16x8(wf[u][p]), acc[t][p]);
  }
}

template <int MT, int EPI, int U, int NW, int AMODE, bool SPLIT, bool QW>
__global__ __launch_bounds__(NW * WAVE) void gemm_kernel(GemmArgs g) {
  constexpr int NP = paired<EPI>();
  __shared__ f32x4 red[NW][NP][WAVE];
  __shared__ float inv_s[16];
  __shared__ float sred[NW];
  extern __shared__ uint4 dyn_lds[];
  uint16_t *a_lds = reinterpret_cast<uint16_t *>(dyn_lds);

  // bf16 weights, or int8 codes with their row scales (QW)
  const void *W = QW ? static_cast<const void *>(g.Wq) : static_cast<const void *>(g.W);
  const float *wscale = g.wscale;
  int row0 = 0, rows = g.M;
  if (g.n_groups) {
    const int gi = blockIdx.y;
    if (gi >= *g.n_groups) return;
    const int64_t ex = g.group_expert[gi];
    if (QW) {
      W = static_cast<const int8_t *>(W) + ex * g.w_group_stride;
      wscale += ex * (g.w_group_stride / g.K);
    } else {
      W = static_cast<const uint16_t *>(W) + ex * g.w_group_stride;
    }
    row0 = g.group_start[gi];
    rows = g.group_count[gi];
  }
  const int n0 = tile_n0<EPI>(g, blockIdx.x);
  const bool nvalid = (EPI == EPI_QKV) || (n0 + (threadIdx.x & 15)) < g.N;
  // k steps: 32 wide (one MFMA k group), 64 wide for int8 codes (two groups)
  const int steps = QW ? (g.K + 63) / 64 : (g.K + 31) / 32;
  int s0 = 0, s1 = steps;
  if (g.ksplit > 1) {
    const int per = (steps + g.ksplit - 1) / g.ksplit;
    s0 = blockIdx.z * per;
    s1 = min(steps, s0 + per);
  }
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;

  if (AMODE == 2) {
    // fused RMSNorm prologue (rows <= 16): per-row 1/rms in fixed order, then
    // the normalised rows into LDS as split bf16 (hi plane, then lo plane)
    const int K = g.K;
    for (int m = 0; m < rows; ++m) {
      const float *xr = g.x + (int64_t)m * g.lda;
      float ss = 0.f;
      for (int k = threadIdx.x * 4; k < K; k += NW * WAVE * 4) {
        const f32x4 v = loadf4(xr + k);
        ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
      }
      ss = block_sum<NW>(ss, sred);
      if (threadIdx.x == 0) inv_s[m] = 1.0f / sqrtf(ss / (float)K + g.eps);
    }
    __syncthreads();
    const int k8 = K / 8;
    for (int e = threadIdx.x; e < rows * k8; e += NW * WAVE) {
      const int m = e / k8, k = (e - m * k8) * 8;
      const float *xr = g.x + (int64_t)m * g.lda + k;
      const f32x4 x0 = loadf4(xr), x1 = loadf4(xr + 4);
      const f32x4 g0 = loadf4(g.gamma + k), g1 = loadf4(g.gamma + k + 4);
      const float iv = inv_s[m];
      u32x4 oh, ol;
      { const u32pair t_ = pack_split2(x0[0] * iv * g0[0], x0[1] * iv * g0[1]); oh[0] = t_.hi; ol[0] = t_.lo; }
      { const u32pair t_ = pack_split2(x0[2] * iv * g0[2], x0[3] * iv * g0[3]); oh[1] = t_.hi; ol[1] = t_.lo; }
      { const u32pair t_ = pack_split2(x1[0] * iv * g1[0], x1[1] * iv * g1[1]); oh[2] = t_.hi; ol[2] = t_.lo; }
      { const u32pair t_ = pack_split2(x1[2] * iv * g1[2], x1[3] * iv * g1[3]); oh[3] = t_.hi; ol[3] = t_.lo; }
      *reinterpret_cast<u32x4 *>(a_lds + (int64_t)m * K + k) = oh;
      *reinterpret_cast<u32x4 *>(a_lds + (int64_t)(rows + m) * K + k) = ol;
    }
    __syncthreads();
  }

  for (int mp = 0; mp < rows; mp += 16 * MT) {
    f32x4 acc[MT][NP];
    const int64_t a_lo = AMODE == 2 ? (int64_t)rows * g.K : g.a_lo;
    gemm_tile<MT, NP, U, NW, AMODE, SPLIT, QW>(g, W, a_lds, a_lo, row0, rows, mp, n0, nvalid, s0, s1, acc);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
      for (int p = 0; p < NP; ++p) red[wave][p][lane] = acc[t][p];
      __syncthreads();
      if (threadIdx.x < 256) {
        // thread -> (lane', i): output row 4 (lane' / 16) + i of the m-tile, column lane' % 16
        const int ol = threadIdx.x >> 2, oi = threadIdx.x & 3;
        const int c = ol & 15;
        const int n = n0 + c;
        const int m = mp + t * 16 + (ol >> 4) * 4 + oi;
        float v[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          float s = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) s += red[w][p][ol][oi];
          v[p] = s;
        }
        const bool ok = m < rows && (EPI == EPI_QKV || n < g.N);
        if (QW) {
          // the row scales (powers of two: exact); a column past N scales by 1
#pragma unroll
          for (int p = 0; p < NP; ++p) v[p] *= (EPI == EPI_QKV || n < g.N) ? wscale[n + p * g.np_off] : 1.0f;
        }
        if (ok) {
          const int64_t orow = row0 + m;
          if (g.ksplit > 1) {
            const int64_t np_cols = (int64_t)gridDim.x * 16;
            float *dst = g.Cpart + ((int64_t)blockIdx.z * g.M + orow) * NP * np_cols;
#pragma unroll
            for (int p = 0; p < NP; ++p) dst[p * np_cols + blockIdx.x * 16 + c] = v[p];
          } else {
            epi_apply<EPI>(g, orow, n, v[0], v[NP - 1]);
          }
        }
        if (EPI == EPI_LOGITS) {
          // best (value, index) of this tile's 16 columns for row m: the 16
          // columns of a row sit in lanes that differ in bits 2..5
          float bv = ok ? v[0] : -INFINITY;
          int bi = ok ? n : 0x7fffffff;
#pragma unroll
          for (int o = 4; o <= 32; o <<= 1) {
            const float ov = __shfl_xor(bv, o, WAVE);
            const int oi2 = __shfl_xor(bi, o, WAVE);
            if (better(ov, oi2, bv, bi)) {
              bv = ov;
              bi = oi2;
            }
          }
          if (c == 0 && m < rows) {
            g.am.part_val[(int64_t)m * gridDim.x + blockIdx.x] = bv;
            g.am.part_idx[(int64_t)m * gridDim.x + blockIdx.x] = bi;
          }
        }
      }
      __syncthreads();
    }
  }

}

template <int EPI>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmArgs g, int ntiles) {
  constexpr int NP = paired<EPI>();
  const int64_t np_cols = (int64_t)ntiles * 16;
  const int64_t total = (int64_t)g.M * np_cols;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = e / np_cols;
    const int pc = (int)(e - m * np_cols);
    const int n = tile_n0<EPI>(g, pc / 16) + (pc & 15);
    if (EPI != EPI_QKV && n >= g.N) continue;
    float v[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      float s = 0.f;
      for (int z = 0; z < g.ksplit; ++z) s += g.Cpart[((int64_t)z * g.M + m) * NP * np_cols + p * np_cols + pc];
      v[p] = s;
    }
    epi_apply<EPI>(g, m, n, v[0], v[NP - 1]);
  }
}

// Split-K reduce of a residual projection fused with the RMSNorm that reads
// the new residual (engine.zig Engine.forward: x += W o, then the next
// sub-block's rmsnormColumn): one block per row; the partials are summed in
// fixed split order, added to x, and x / sqrt(mean(x^2) + eps) * gamma is
// written as the next projection's split-bf16 activation.
__global__ __launch_bounds__(1024) void gemm_reduce_norm_kernel(GemmArgs g, int ntiles) {
  __shared__ float lds[16];
  const int64_t np_cols = (int64_t)ntiles * 16;
  const int m = blockIdx.x, N = g.N;
  float *xr = g.C + (int64_t)m * g.ldc;
  const float *pr = g.Cpart + (int64_t)m * np_cols;
  const int64_t zstride = (int64_t)g.M * np_cols;
  float ss = 0.f;
  for (int n = threadIdx.x * 4; n < N; n += 1024 * 4) {
    // x + (p_0 + p_1 + ...), the order of the element-wise reduce; the
    // partials of up to 8 splits are loaded together
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int z0 = 0; z0 < g.ksplit; z0 += 8) {
      f32x4 p[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) p[u] = *reinterpret_cast<const f32x4 *>(pr + min(z0 + u, g.ksplit - 1) * zstride + n);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (z0 + u < g.ksplit) {
          acc[0] += p[u][0];
          acc[1] += p[u][1];
          acc[2] += p[u][2];
          acc[3] += p[u][3];
        }
    }
    f32x4 v = *reinterpret_cast<const f32x4 *>(xr + n);
    v[0] += acc[0];
    v[1] += acc[1];
    v[2] += acc[2];
    v[3] += acc[3];
    *reinterpret_cast<f32x4 *>(xr + n) = v;
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = block_sum<16>(ss, lds);
  const float inv = 1.0f / sqrtf(ss / (float)N + g.norm_eps);
  uint16_t *orow = g.norm_out + (int64_t)m * N;
  for (int n = threadIdx.x * 4; n < N; n += 1024 * 4) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(xr + n);
    const f32x4 w = *reinterpret_cast<const f32x4 *>(g.norm_gamma + n);
    u32x2 oh, ol;
    { const u32pair t_ = pack_split2(v[0] * inv * w[0], v[1] * inv * w[1]); oh[0] = t_.hi; ol[0] = t_.lo; }
    { const u32pair t_ = pack_split2(v[2] * inv * w[2], v[3] * inv * w[3]); oh[1] = t_.hi; ol[1] = t_.lo; }
    *reinterpret_cast<u32x2 *>(orow + n) = oh;
    *reinterpret_cast<u32x2 *>(orow + g.norm_lo + n) = ol;
  }
}

// U: weight steps per load batch, so that a batch holds about 16 fragments
template <int MT, int EPI, int NW, int AMODE, bool SPLIT, bool QW = false>
hipError_t launch_cfg(const GemmArgs &g, dim3 grid, size_t dyn, hipStream_t st) {
  constexpr int NP = paired<EPI>();
  constexpr int F = MT * (SPLIT ? 2 : 1) + NP;
  constexpr int U = F <= 4 ? 4 : (F <= 8 ? 2 : 1);
  hipLaunchKernelGGL((gemm_kernel<MT, EPI, U, NW, AMODE, SPLIT, QW>), grid, dim3(NW * WAVE), dyn, st, g);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const GemmArgs &g, int mt, bool norm, dim3 grid, size_t dyn, hipStream_t st) {
  if (g.Wq) {
    // int8 codes: decode batches and verify passes (one 16-row tile of rows)
    if (mt != 1 || !g.wscale) return hipErrorInvalidValue;
    if (norm) return launch_cfg<1, EPI, 8, 2, true, true>(g, grid, dyn, st);
    if (g.a_lo) return launch_cfg<1, EPI, 8, 0, true, true>(g, grid, 0, st);
    return launch_cfg<1, EPI, 8, 0, false, true>(g, grid, 0, st);
  }
  if (norm) return launch_cfg<1, EPI, 8, 2, true>(g, grid, dyn, st);
  if (!g.a_lo) {
    switch (mt) {
      case 1: return launch_cfg<1, EPI, 8, 0, false>(g, grid, 0, st);
      case 2: return launch_cfg<2, EPI, 4, 0, false>(g, grid, 0, st);
      case 4: return launch_cfg<4, EPI, 4, 0, false>(g, grid, 0, st);
      default: return launch_cfg<8, EPI, 4, 0, false>(g, grid, 0, st);
    }
  }
  switch (mt) {
    case 1: return launch_cfg<1, EPI, 8, 0, true>(g, grid, 0, st);
    case 2: return launch_cfg<2, EPI, 4, 0, true>(g, grid, 0, st);
    case 4: return launch_cfg<4, EPI, 4, 0, true>(g, grid, 0, st);
    default: return launch_cfg<8, EPI, 4, 0, true>(g, grid, 0, st);
  }
}

}  // namespace

int gemm_mtiles(int rows) {
  if (rows <= 16) return 1;
  if (rows <= 32) return 2;
  if (rows <= 64) return 4;
  return 8;
}

int gemm_ntiles(const GemmArgs &g, int epi) {
  if (epi == EPI_QKV) return (g.qkv.Hq + 2 * g.qkv.Hkv) * (g.qkv.d / 32);
  return (g.N + 15) / 16;
}

bool gemm_norm_fits(int rows, int K) { return rows <= GEMM_NORM_MAX_ROWS && (size_t)rows * K * 4 <= GEMM_NORM_MAX_LDS; }

hipError_t launch_gemm(const GemmArgs &g, int epi, int max_rows, int n_group_slots, hipStream_t st) {
  const int ntiles = gemm_ntiles(g, epi);
  const bool norm = g.x != nullptr;
  const int mt = gemm_mtiles(max_rows);
  const size_t dyn = norm ? (size_t)g.M * g.K * 4 : 0;  // hi and lo planes
  dim3 grid(ntiles, g.n_groups ? n_group_slots : 1, g.ksplit > 1 ? g.ksplit : 1);
  hipError_t e;
  switch (epi) {
    case EPI_STORE: e = launch_epi<EPI_STORE>(g, mt, norm, grid, dyn, st); break;
    case EPI_ADD: e = launch_epi<EPI_ADD>(g, mt, norm, grid, dyn, st); break;
    case EPI_SWIGLU: e = launch_epi<EPI_SWIGLU>(g, mt, norm, grid, dyn, st); break;
    case EPI_QKV: e = launch_epi<EPI_QKV>(g, mt, norm, grid, dyn, st); break;
    default: e = launch_epi<EPI_LOGITS>(g, mt, norm, grid, dyn, st); break;
  }
  if (e != hipSuccess || g.ksplit <= 1) return e;
  return launch_gemm_reduce(g, epi, ntiles, st);
}

hipError_t launch_gemm_reduce(const GemmArgs &g, int epi, int ntiles, hipStream_t st) {
  if (epi == EPI_ADD && g.norm_out) {
    if (g.N % 4 || ntiles * 16 != g.N) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gemm_reduce_norm_kernel, dim3(g.M), dim3(1024), 0, st, g, ntiles);
    return hipGetLastError();
  }
  const int64_t total = (int64_t)g.M * ntiles * 16;
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 4096);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL(gemm_reduce_kernel<EPI_STORE>, dim3(blocks), dim3(256), 0, st, g, ntiles); break;
    case EPI_ADD: hipLaunchKernelGGL(gemm_reduce_kernel<EPI_ADD>, dim3(blocks), dim3(256), 0, st, g, ntiles); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(gemm_reduce_kernel<EPI_SWIGLU>, dim3(blocks), dim3(256), 0, st, g, ntiles); break;
    case EPI_QKV: hipLaunchKernelGGL(gemm_reduce_kernel<EPI_QKV>, dim3(blocks), dim3(256), 0, st, g, ntiles); break;
    default: return hipErrorInvalidValue;  // logits are never split
  }
  return hipGetLastError();
}
