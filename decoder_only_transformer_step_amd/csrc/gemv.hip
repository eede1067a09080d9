// Single-token projection (batch-1 decode): y[n] = sum_k W[n][k] a[k]
// (engine.zig: a projection at activation width 1 reads the whole weight
// matrix for one column; pipeline.rs lm_head_forward: the row-parallel
// matvec that dominates a decode step).
//
// gfx950 design: the step is a pure weight stream (2 bytes per
// multiply-add), so the kernel is built around the HBM access shape.
//  * Each wave owns one item (a weight row, or a row pair for the paired
//    epilogues: SwiGLU gate/up rows n and n + N, QKV rows i and i + d/2 of
//    a head) and walks it in 1 KB steps: lane l loads 16 contiguous bytes at
//    k = 8 l + 512 s, so every load instruction of the wave is one
//    contiguous kilobyte.  Long contiguous bursts sustain measurably more
//    HBM bandwidth than 16-rows-by-64-bytes MFMA fragments.
//  * The activation is kept in fp32 in LDS (the fused RMSNorm prologue
//    writes it there once per block), so the only rounding on the path is
//    the weights' own bf16 storage.  Each lane does 8 fp32 FMAs per 16-byte
//    load, then a 64-lane butterfly sum gives the dot product.
//  * Software pipeline: the first batch of weight loads is issued before the
//    activation prologue, and each later batch while the previous one is
//    consumed, so every wave keeps several kilobytes in flight at all times.
//  * Persistent grid (about two blocks per compute unit): the activation
//    prologue runs once per block, and each wave streams its items back to
//    back, the next item's first loads overlapping the current reduction.
//  * Grouped mode (MoE experts): blockIdx.y = routing slot; the weight base
//    moves to the chosen expert.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace {

constexpr int GV_MAX_WAVES = 8;

template <int EPI>
constexpr int gv_rows() {
  return (EPI == EPI_SWIGLU || EPI == EPI_QKV) ? 2 : 1;
}

// weight rows of item `it`
template <int EPI>
__device__ __forceinline__ void item_rows(const GemvArgs &g, int it, int &r0, int &r1) {
  if (EPI == EPI_QKV) {
    const int half = g.qkv.d / 2;
    const int hh = it / half, i = it - hh * half;
    r0 = hh * g.qkv.d + i;
    r1 = r0 + half;
  } else if (EPI == EPI_SWIGLU) {
    r0 = it;
    r1 = it + g.N;
  } else {
    r0 = r1 = it;
  }
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// Loads of UNR 1 KB steps for every row the wave owns.
template <int R, int UNR>
__device__ __forceinline__ void load_batch(u32x4 (&v)[UNR][R], const uint16_t *const (&wp)[R],
                                           const bool (&rv)[R], int s0, int steps, int K, int lane) {
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int st = s0 + u;
    const bool ok = st < steps && st * 512 + lane * 8 < K;
#pragma unroll
    for (int r = 0; r < R; ++r) v[u][r] = (ok && rv[r]) ? load16(wp[r] + st * 512) : u32x4{0u, 0u, 0u, 0u};
  }
}

// acc[r] += dot(weights of batch, activation) over UNR steps.
template <int R, int UNR>
__device__ __forceinline__ void fma_batch(float (&acc)[R], const u32x4 (&v)[UNR][R], const float *xs, int s0,
                                          int steps, int K, int lane) {
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int k = (s0 + u) * 512 + lane * 8;
    if ((s0 + u) < steps && k < K) {
      const f32x4 xa = *reinterpret_cast<const f32x4 *>(xs + k);
      const f32x4 xb = *reinterpret_cast<const f32x4 *>(xs + k + 4);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const u32x4 w = v[u][r];
        float a = acc[r];
        a = fmaf(bf16_lo(w[0]), xa[0], a);
        a = fmaf(bf16_hi(w[0]), xa[1], a);
        a = fmaf(bf16_lo(w[1]), xa[2], a);
        a = fmaf(bf16_hi(w[1]), xa[3], a);
        a = fmaf(bf16_lo(w[2]), xb[0], a);
        a = fmaf(bf16_hi(w[2]), xb[1], a);
        a = fmaf(bf16_lo(w[3]), xb[2], a);
        a = fmaf(bf16_hi(w[3]), xb[3], a);
        acc[r] = a;
      }
    }
  }
}

// Rows of item `it` and their weight pointers (lane offset included).
template <int EPI, int NR>
__device__ __forceinline__ void item_ptrs(const GemvArgs &g, const uint16_t *W, int it, int lane,
                                          int (&rows)[NR], const uint16_t *(&wp)[NR], bool (&rv)[NR]) {
  int r0 = 0, r1 = 0;
  const bool ok = it < g.n_items;
  if (ok) item_rows<EPI>(g, it, r0, r1);
  rows[0] = r0;
  rows[NR - 1] = r1;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    rv[r] = ok;
    wp[r] = W + (int64_t)rows[r] * g.K + lane * 8;
  }
}

// Epilogue of one item (lane 0 writes).
template <int EPI>
__device__ __forceinline__ void item_epilogue(const GemvArgs &g, int out_row, int r0, int r1, float v0, float v1) {
  if (EPI == EPI_STORE) {
    g.C[(int64_t)out_row * g.ldc + r0] = v0 + (g.bias ? g.bias[r0] : 0.f);
  } else if (EPI == EPI_ADD) {
    g.C[r0] += v0;
  } else if (EPI == EPI_SWIGLU) {
    g.C[(int64_t)out_row * g.ldc + r0] = silu_f(v0) * v1;
  } else if (EPI == EPI_LOGITS) {
    g.C[r0] = v0;
  } else if (EPI == EPI_QKV) {
    // bias, then RoPE on q and k rows, then the KV-cache append
    // (engine.zig ropeAndCache, "rope" pairing u_i with u_{i+d/2};
    // decoder.rs AttnWeights: bias before RoPE)
    const QkvEpi &q = g.qkv;
    const int d = q.d, half = d / 2;
    const int hh = r0 / d, i = r0 - hh * d;
    float u0 = v0, u1 = v1;
    if (q.bias) {
      u0 += q.bias[r0];
      u1 += q.bias[r1];
    }
    const int pos = q.row_pos[0], seq = q.row_seq[0];
    const int64_t base = (int64_t)seq * q.seq_stride + q.layer_off;
    if (hh < q.Hq + q.Hkv) {
      const float2 t = q.cs[(int64_t)pos * half + i];
      const float a0 = u0 * t.x - u1 * t.y, a1 = u0 * t.y + u1 * t.x;
      if (hh < q.Hq) {
        uint16_t *dst = q.q + (int64_t)hh * d;
        uint32_t h0, l0, h1, l1;
        split_bf16(a0, h0, l0);
        split_bf16(a1, h1, l1);
        dst[i] = (uint16_t)h0;
        dst[i + half] = (uint16_t)h1;
        dst[q.q_lo + i] = (uint16_t)l0;
        dst[q.q_lo + i + half] = (uint16_t)l1;
      } else {
        uint16_t *dst = q.kcache + base + ((int64_t)(hh - q.Hq) * q.S + pos) * d;
        dst[i] = (uint16_t)f32_to_bf16_bits(a0);
        dst[i + half] = (uint16_t)f32_to_bf16_bits(a1);
      }
    } else {
      uint16_t *vt = q.vcache + base + (int64_t)(hh - q.Hq - q.Hkv) * d * q.S;
      vt[(int64_t)i * q.S + pos] = (uint16_t)f32_to_bf16_bits(u0);
      vt[(int64_t)(i + half) * q.S + pos] = (uint16_t)f32_to_bf16_bits(u1);
    }
  }
}

// Persistent grid: each wave walks the items it, it + stride, ... as one
// sequence of UNR-step load batches, ping-ponging between two register
// buffers, so the first batch of the next item is already in flight while
// the current item is reduced and written.
template <int EPI, int UNR, int GV_WAVES>
__global__ __launch_bounds__(GV_WAVES * WAVE) void gemv_kernel(GemvArgs g) {
  constexpr int NR = gv_rows<EPI>();
  extern __shared__ float xs[];
  __shared__ float sred[GV_MAX_WAVES];
  __shared__ float bv_s[GV_MAX_WAVES];
  __shared__ int bi_s[GV_MAX_WAVES];

  const uint16_t *W = g.W;
  const float *xin = g.a_f32;
  int out_row = 0;
  if (g.slot_expert) {
    const int slot = blockIdx.y;
    W += (int64_t)g.slot_expert[slot] * g.w_group_stride;
    if (xin) xin += (int64_t)slot * g.a_slot_stride;
    out_row = slot;
  }
  const int K = g.K;
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int stride = gridDim.x * GV_WAVES;
  const int steps = (K + 511) / 512;
  const int nb = (steps + UNR - 1) / UNR;  // batches per item

  // batch sequence position of the next load: item `li`, batch `lb`
  int li = blockIdx.x * GV_WAVES + wave, lb = 0;
  int lrows[NR];
  const uint16_t *lwp[NR];
  bool lrv[NR];
  item_ptrs<EPI, NR>(g, W, li, lane, lrows, lwp, lrv);

  u32x4 buf0[UNR][NR], buf1[UNR][NR];
  // the first weight loads go out before the activation prologue
  load_batch<NR, UNR>(buf0, lwp, lrv, 0, steps, K, lane);

  // activation -> LDS (fp32), with the RMSNorm prologue when gamma is set
  if (g.gamma) {
    float ss = 0.f;
    for (int k = threadIdx.x * 4; k < K; k += GV_WAVES * WAVE * 4) {
      const f32x4 v = loadf4(xin + k);
      ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
    ss = block_sum<GV_WAVES>(ss, sred);
    const float inv = 1.0f / sqrtf(ss / (float)K + g.eps);
    for (int k = threadIdx.x * 4; k < K; k += GV_WAVES * WAVE * 4) {
      const f32x4 v = loadf4(xin + k), w = loadf4(g.gamma + k);
      *reinterpret_cast<f32x4 *>(xs + k) = f32x4{v[0] * inv * w[0], v[1] * inv * w[1], v[2] * inv * w[2], v[3] * inv * w[3]};
    }
  } else if (xin) {
    for (int k = threadIdx.x * 4; k < K; k += GV_WAVES * WAVE * 4)
      *reinterpret_cast<f32x4 *>(xs + k) = loadf4(xin + k);
  } else {
    for (int k = threadIdx.x * 8; k < K; k += GV_WAVES * WAVE * 8) {
      const u32x4 w = load16(g.a_bf16 + k);
      *reinterpret_cast<f32x4 *>(xs + k) = f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
      *reinterpret_cast<f32x4 *>(xs + k + 4) = f32x4{bf16_lo(w[2]), bf16_hi(w[2]), bf16_lo(w[3]), bf16_hi(w[3])};
    }
  }
  __syncthreads();

  // consumption state: item `ci` (rows crows), batch `cb`
  int ci = li, cb = 0;
  int crows[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) crows[r] = lrows[r];
  float acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.f;
  float bv = -INFINITY;
  int bi = 0x7fffffff;

  // advance the load position by one batch and issue it into `dst`
  auto issue_next = [&](u32x4 (&dst)[UNR][NR]) {
    if (++lb == nb) {
      lb = 0;
      li += stride;
      item_ptrs<EPI, NR>(g, W, li, lane, lrows, lwp, lrv);
    }
    if (li < g.n_items) load_batch<NR, UNR>(dst, lwp, lrv, lb * UNR, steps, K, lane);
  };
  // consume `src` as batch cb of item ci; finish the item on its last batch
  auto consume = [&](const u32x4 (&src)[UNR][NR]) {
    fma_batch<NR, UNR>(acc, src, xs, cb * UNR, steps, K, lane);
    if (++cb == nb) {
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] = wave_sum(acc[r]);
      if (EPI == EPI_LOGITS && better(acc[0], crows[0], bv, bi)) {
        bv = acc[0];
        bi = crows[0];
      }
      if (lane == 0) item_epilogue<EPI>(g, out_row, crows[0], crows[NR - 1], acc[0], acc[NR - 1]);
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] = 0.f;
      cb = 0;
      ci += stride;
#pragma unroll
      for (int r = 0; r < NR; ++r) crows[r] = lrows[r];  // the load position is already on item ci
    }
  };

  while (ci < g.n_items) {
    issue_next(buf1);
    consume(buf0);
    if (ci >= g.n_items) break;
    issue_next(buf0);
    consume(buf1);
  }

  if (EPI == EPI_LOGITS) {
    // this block's best (value, index), for the argmax finalize pass
    if (lane == 0) {
      bv_s[wave] = bv;
      bi_s[wave] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < GV_WAVES; ++w)
        if (better(bv_s[w], bi_s[w], bv, bi)) {
          bv = bv_s[w];
          bi = bi_s[w];
        }
      g.part_val[blockIdx.x] = bv;
      g.part_idx[blockIdx.x] = bi;
    }
  }
}

// A load batch holds DEC_GEMV_LOADS kilobytes (twice that when deep) across
// the item's rows.
template <int EPI, int W, bool DEEP>
constexpr auto gv_kernel() {
  constexpr int NR = gv_rows<EPI>();
  return gemv_kernel<EPI, (DEEP ? 2 : 1) * DEC_GEMV_LOADS / NR, W>;
}

template <int EPI>
hipError_t launch_e(const GemvArgs &g, const GemvShape &sh, dim3 grid, size_t lds, hipStream_t st) {
  if (sh.waves == 4) {
    if (sh.deep) hipLaunchKernelGGL((gv_kernel<EPI, 4, true>()), grid, dim3(4 * WAVE), lds, st, g);
    else hipLaunchKernelGGL((gv_kernel<EPI, 4, false>()), grid, dim3(4 * WAVE), lds, st, g);
  } else {
    if (sh.deep) hipLaunchKernelGGL((gv_kernel<EPI, 8, true>()), grid, dim3(8 * WAVE), lds, st, g);
    else hipLaunchKernelGGL((gv_kernel<EPI, 8, false>()), grid, dim3(8 * WAVE), lds, st, g);
  }
  return hipGetLastError();
}

// Blocks of one kernel instance resident per compute unit (registers and
// the block's LDS), or 1 if the runtime cannot say.
template <int EPI, int W, bool DEEP>
int resident_e(size_t lds) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(gv_kernel<EPI, W, DEEP>()),
                                                   W * WAVE, lds) != hipSuccess || n < 1)
    n = 1;
  return n;
}

template <int W, bool DEEP>
int resident(int epi, size_t lds) {
  switch (epi) {
    case EPI_STORE: return resident_e<EPI_STORE, W, DEEP>(lds);
    case EPI_ADD: return resident_e<EPI_ADD, W, DEEP>(lds);
    case EPI_SWIGLU: return resident_e<EPI_SWIGLU, W, DEEP>(lds);
    case EPI_QKV: return resident_e<EPI_QKV, W, DEEP>(lds);
    default: return resident_e<EPI_LOGITS, W, DEEP>(lds);
  }
}

int device_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    hipDeviceProp_t p;
    cus = (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&p, dev) == hipSuccess) ? p.multiProcessorCount : 256;
  }
  return cus;
}

}  // namespace

// Persistent grid shape: blocks of 4 or 8 waves, m blocks per compute unit
// (m at most DEC_GEMV_BLOCKS_PER_CU and at most what fits in registers and
// LDS at once), chosen so that the busiest compute unit has as few items as
// possible (items spread evenly over the waves of evenly loaded CUs, no tail
// round with idle waves), then for the most waves in flight.  Deep batches
// when a wave owns a single item (nothing to pipeline across items) or there
// are few waves per compute unit, if they fit.
GemvShape gemv_shape(int n_items, int K, int epi) {
  const int cus = device_cus();
  const size_t lds = (size_t)K * 4;
  GemvShape best{8, 1, 1, false};
  long best_load = -1;
  int best_waves = 0, best_m = 1;
  for (int w : {8, 4}) {
    const int fit = std::min(DEC_GEMV_BLOCKS_PER_CU, w == 8 ? resident<8, false>(epi, lds) : resident<4, false>(epi, lds));
    for (int m = 1; m <= fit; ++m) {
      const long waves = (long)cus * m * w;
      const int per = (int)((n_items + waves - 1) / waves);
      const int blocks = (n_items + w * per - 1) / (w * per);
      // items on the busiest compute unit (blocks spread evenly over the CUs)
      const long load = (long)((blocks + cus - 1) / cus) * w * per;
      const int wpc = (int)((long)blocks * w / cus);
      if (best_load < 0 || load < best_load || (load == best_load && wpc > best_waves)) {
        best_load = load;
        best_waves = wpc;
        best_m = (blocks + cus - 1) / cus;
        best = GemvShape{w, blocks, per, false};
      }
    }
  }
  if (best.per_wave == 1 || (long)best.blocks * best.waves <= 8L * cus) {
    const int fit = best.waves == 8 ? resident<8, true>(epi, lds) : resident<4, true>(epi, lds);
    best.deep = best_m <= fit;
  }
  return best;
}

hipError_t launch_gemv(const GemvArgs &g, int epi, hipStream_t st, int *blocks) {
  const GemvShape sh = gemv_shape(g.n_items, g.K, epi);
  if (blocks) *blocks = sh.blocks;
  dim3 grid(sh.blocks, g.slot_expert ? g.n_slots : 1);
  const size_t lds = (size_t)g.K * 4;
  switch (epi) {
    case EPI_STORE: return launch_e<EPI_STORE>(g, sh, grid, lds, st);
    case EPI_ADD: return launch_e<EPI_ADD>(g, sh, grid, lds, st);
    case EPI_SWIGLU: return launch_e<EPI_SWIGLU>(g, sh, grid, lds, st);
    case EPI_QKV: return launch_e<EPI_QKV>(g, sh, grid, lds, st);
    default: return launch_e<EPI_LOGITS>(g, sh, grid, lds, st);
  }
}
