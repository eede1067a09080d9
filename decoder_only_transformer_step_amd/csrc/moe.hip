// MoE routing and combine (pipeline.rs MoeFfn; engine.zig Engine.forward and
// Engine.prefill; decoder.rs MoeWeights).
//
//  route:   P = softmax over ALL expert logits of the normed FFN input; the
//           k largest (distinct experts, lower index first on ties) with
//           weight P_e, or P_e / sum over the chosen when renormalising;
//           the shared-expert scale sigmoid(w_sg . b) (1 without a gate).
//  group:   pairs (row, slot) sorted by expert, then by row: every chosen
//           expert becomes one group whose weights are streamed once for
//           all rows that chose it (engine.zig Engine.prefill batching);
//           optionally the shared expert's slices as further groups that
//           every row joins.
//  combine: x += sum_j w_j y_pair(j) + gate * y_shared, slots in router
//           order (y_shared summed over its slices first).
#include "common.h"
#include "launch.h"

namespace {

constexpr int ROUTE_THREADS = 256;
constexpr int GROUP_MAX_PAIRS = 4096;  // rows x k (rows <= 512, k <= 8)

// One block per row.  All threads take the shared-gate dot product; the
// first wave then routes (moe_topk: the softmax max and sum are wave
// reductions, and each of the k picks is a wave arg-max over the experts not
// yet taken).
__global__ __launch_bounds__(ROUTE_THREADS) void moe_route_kernel(MoeRouteArgs a) {
  __shared__ float red[ROUTE_THREADS / WAVE];
  const int r = blockIdx.x, E = a.E;
  // shared-expert gate: sigmoid(w_sg . b), fp32 dot in fixed order
  float dot = 0.f;
  if (a.w_sh_gate) {
    if (a.act_f32 && a.gamma) {
      // b = RMSNorm(x) computed here: fp32 mean square, then the gain.  Eight
      // elements per thread per round, loads unconditional (clamped index,
      // masked in the sum) so that they are all in flight together.
      const float *x = a.act_f32 + (int64_t)r * a.H;
      const int H = a.H;
      float ss = 0.f;
      for (int j0 = threadIdx.x; j0 < H; j0 += 8 * ROUTE_THREADS) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = x[min(j0 + u * ROUTE_THREADS, H - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u) ss += j0 + u * ROUTE_THREADS < H ? v[u] * v[u] : 0.f;
      }
      ss = block_sum<ROUTE_THREADS / WAVE>(ss, red);
      const float inv = 1.0f / sqrtf(ss / (float)H + a.eps);
      for (int j0 = threadIdx.x; j0 < H; j0 += 8 * ROUTE_THREADS) {
        float v[8], gm[8], wg[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int j = min(j0 + u * ROUTE_THREADS, H - 1);
          v[u] = x[j];
          gm[u] = a.gamma[j];
          wg[u] = bf16_to_f32(a.w_sh_gate[j]);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) dot += j0 + u * ROUTE_THREADS < H ? (v[u] * inv * gm[u]) * wg[u] : 0.f;
      }
    } else if (a.act_f32) {
      const float *b = a.act_f32 + (int64_t)r * a.H;
      for (int j = threadIdx.x; j < a.H; j += blockDim.x) dot += b[j] * bf16_to_f32(a.w_sh_gate[j]);
    } else {
      const uint16_t *b = a.act + (int64_t)r * a.H;
      for (int j = threadIdx.x; j < a.H; j += blockDim.x)
        dot += (bf16_to_f32(b[j]) + bf16_to_f32(b[a.act_lo + j])) * bf16_to_f32(a.w_sh_gate[j]);
    }
  }
  dot = block_sum<ROUTE_THREADS / WAVE>(dot, red);
  if (threadIdx.x >= WAVE) return;
  const int lane = threadIdx.x;
  int32_t *ids = a.ids + (int64_t)r * a.k;
  float *w = a.wts + (int64_t)r * a.k;
  float wsel[8], sel;
  int isel[8];
  moe_topk(a.logits + (int64_t)r * E, E, a.k, lane, isel, wsel, sel);
  if (lane == 0) {
    for (int j = 0; j < a.k; ++j) {
      ids[j] = isel[j];
      w[j] = a.renorm ? wsel[j] / sel : wsel[j];
      if (a.ids_record) a.ids_record[(int64_t)r * a.k + j] = isel[j];
    }
    if (a.gate) a.gate[r] = a.w_sh_gate ? 1.0f / (1.0f + expf(-dot)) : 1.0f;
  }
}

// Group table over experts in increasing order, pairs by row, built by one
// block (any size).  The ids are staged in LDS; counts by LDS atomics; a
// pair's slot in its expert's group follows the number of earlier pairs with
// the same expert.  AT: the ids were written by other blocks of the same
// launch and are read with relaxed device-scope loads.
struct GroupLds {
  int ids[GROUP_MAX_PAIRS];
  int cnt[256];
  int start[256];
};

template <bool AT>
__device__ __forceinline__ void group_pairs(const MoeRouteArgs &a, GroupLds &s) {
  const int E = a.E, P = a.rows * a.k;
  for (int e = threadIdx.x; e < E; e += blockDim.x) s.cnt[e] = 0;
  for (int p = threadIdx.x; p < P; p += blockDim.x)
    s.ids[p] = AT ? __hip_atomic_load(a.ids + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : a.ids[p];
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += blockDim.x) atomicAdd(&s.cnt[s.ids[p]], 1);
  __syncthreads();
  if (threadIdx.x == 0) {
    int st = 0, ng = 0;
    for (int e = 0; e < E; ++e) {
      s.start[e] = st;
      if (s.cnt[e]) {
        a.group_expert[ng] = e;
        a.group_start[ng] = st;
        a.group_count[ng] = s.cnt[e];
        ++ng;
      }
      st += s.cnt[e];
    }
    // the shared expert's pseudo-experts: every row, after the routed pairs
    for (int j = 0; j < a.extra_groups; ++j) {
      a.group_expert[ng + j] = E + j;
      a.group_start[ng + j] = P + j * a.rows;
      a.group_count[ng + j] = a.rows;
    }
    *a.n_groups = ng + a.extra_groups;
  }
  for (int q = threadIdx.x; q < a.extra_groups * a.rows; q += blockDim.x) a.pair_row[P + q] = q % a.rows;
  __syncthreads();
  // a pair's slot: its expert's start plus the number of earlier pairs of
  // that expert.  Wave w scans experts w, w + waves, ...: per 64-pair chunk
  // a ballot marks the expert's pairs, and each marked lane counts the marks
  // below it (P / 64 ballots per expert instead of P compares per pair)
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE, nw = blockDim.x / WAVE;
  for (int e = wave; e < E; e += nw) {
    if (!s.cnt[e]) continue;
    int base = s.start[e];
    for (int c = 0; c < P; c += WAVE) {
      const int p = c + lane;
      const bool hit = p < P && s.ids[p] == e;
      const unsigned long long m = __ballot(hit);
      if (hit) {
        const int o = base + __popcll(m & ((1ull << lane) - 1));
        a.pair_row[o] = p / a.k;
        a.pair_of[p] = o;
      }
      base += __popcll(m);
    }
  }
}

__global__ __launch_bounds__(256) void moe_group_kernel(MoeRouteArgs a) {
  __shared__ GroupLds s;
  group_pairs<false>(a, s);
}

// Router and route in one launch (pipeline.rs MoeFfn: router logits of the
// normed FFN input, softmax over all experts, top-k): one block of 16 waves
// per row.  b = RMSNorm(x; gamma) goes to LDS in fp32; wave w computes the
// logits of experts w, w + 16, ... (lane l takes 8 consecutive elements at
// 8 l + 512 s, one 16-byte weight load each; loads of a wave's experts are
// issued together), the shared-gate dot product joins them, and the first
// wave then routes exactly as moe_route_kernel does.  With a.arrive set the
// launch also groups the pairs: every block publishes its ids with relaxed
// device-scope stores, waits for them and counts its arrival; the last
// block to arrive builds the group table (group_pairs) and resets the
// counter, so no block waits on another and no grouping launch follows.
constexpr int RR_THREADS = 1024;
constexpr int RR_X = 2;  // f32x4 of x per thread: H <= 8192
constexpr int RR_S = 4;  // 512-element steps of router weights in flight per wave
static_assert(RR_X * 4 * RR_THREADS >= MOE_ROUTER_MAX_H, "router rows held in registers");

__global__ __launch_bounds__(RR_THREADS) void moe_router_route_kernel(MoeRouteArgs a) {
  extern __shared__ float bsh[];       // b [H], then the logits [E]
  __shared__ float red[RR_THREADS / WAVE];
  const int r = blockIdx.x, E = a.E, H = a.H;
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  float *lg = bsh + H;
  const float *x = a.act_f32 + (int64_t)r * H;
  // x, gamma and the shared-gate row are loaded together, up front (H <=
  // RR_X * 4 * RR_THREADS: each thread keeps its elements in registers)
  f32x4 xv[RR_X], gv[RR_X];
  float sg[4 * RR_X];
#pragma unroll
  for (int i = 0; i < RR_X; ++i) {
    const int j = min((int)(threadIdx.x + i * RR_THREADS) * 4, H - 4);
    xv[i] = loadf4(x + j);
    gv[i] = loadf4(a.gamma + j);
  }
#pragma unroll
  for (int i = 0; i < 4 * RR_X; ++i) {
    const int j = min((int)threadIdx.x + i * RR_THREADS, H - 1);
    sg[i] = a.w_sh_gate ? bf16_to_f32(a.w_sh_gate[j]) : 0.f;
  }
  // RMSNorm in fp32: mean square in fixed order, then the gain
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < RR_X; ++i)
    if ((int)(threadIdx.x + i * RR_THREADS) * 4 < H)
      ss += xv[i][0] * xv[i][0] + xv[i][1] * xv[i][1] + xv[i][2] * xv[i][2] + xv[i][3] * xv[i][3];
  ss = block_sum<RR_THREADS / WAVE>(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)H + a.eps);
#pragma unroll
  for (int i = 0; i < RR_X; ++i) {
    const int j = (threadIdx.x + i * RR_THREADS) * 4;
    if (j < H)
      *reinterpret_cast<f32x4 *>(bsh + j) = f32x4{xv[i][0] * inv * gv[i][0], xv[i][1] * inv * gv[i][1],
                                                  xv[i][2] * inv * gv[i][2], xv[i][3] * inv * gv[i][3]};
  }
  __syncthreads();
  // logits: wave w takes experts w + 16 i, four at a time; per expert, lane
  // l takes the elements 8 l + 512 s, and the loads of up to RR_S steps of
  // the four experts go out together (H % 8 == 0; lanes past H, and experts
  // past E, read a valid chunk and drop it)
  constexpr int NW = RR_THREADS / WAVE, EU = 4;
  const int steps = (H + 511) / 512;
  for (int e0 = wave; e0 < E; e0 += NW * EU) {
    float acc[EU];
#pragma unroll
    for (int u = 0; u < EU; ++u) acc[u] = 0.f;
    for (int s0 = 0; s0 < steps; s0 += RR_S) {
      u32x4 w[RR_S][EU];
#pragma unroll
      for (int t = 0; t < RR_S; ++t) {
        const int k = (s0 + t) * 512 + lane * 8;
        const int kk = k < H ? k : 0;
#pragma unroll
        for (int u = 0; u < EU; ++u) w[t][u] = load16(a.w_router + (int64_t)min(e0 + NW * u, E - 1) * H + kk);
      }
#pragma unroll
      for (int t = 0; t < RR_S; ++t) {
        const int k = (s0 + t) * 512 + lane * 8;
        const bool ok = k < H;
        const int kk = ok ? k : 0;
        const f32x4 b0 = *reinterpret_cast<const f32x4 *>(bsh + kk);
        const f32x4 b1 = *reinterpret_cast<const f32x4 *>(bsh + kk + 4);
#pragma unroll
        for (int u = 0; u < EU; ++u) {
          float d = bf16_lo(w[t][u][0]) * b0[0];
          d = fmaf(bf16_hi(w[t][u][0]), b0[1], d);
          d = fmaf(bf16_lo(w[t][u][1]), b0[2], d);
          d = fmaf(bf16_hi(w[t][u][1]), b0[3], d);
          d = fmaf(bf16_lo(w[t][u][2]), b1[0], d);
          d = fmaf(bf16_hi(w[t][u][2]), b1[1], d);
          d = fmaf(bf16_lo(w[t][u][3]), b1[2], d);
          d = fmaf(bf16_hi(w[t][u][3]), b1[3], d);
          acc[u] += ok ? d : 0.f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < EU; ++u) {
      const int e = e0 + NW * u;
      const float t = wave_sum(acc[u]);
      if (lane == 0 && e < E) {
        lg[e] = t;
        if (a.logits_out) a.logits_out[(int64_t)r * E + e] = t;
      }
    }
  }
  // shared-expert gate: sigmoid(w_sg . b), fp32 dot in fixed order
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < 4 * RR_X; ++i) {
    const int j = threadIdx.x + i * RR_THREADS;
    if (j < H) dot += bsh[j] * sg[i];
  }
  dot = block_sum<RR_THREADS / WAVE>(dot, red);   // (its barriers also publish the logits)
  if (threadIdx.x < WAVE) {
    int32_t *ids = a.ids + (int64_t)r * a.k;
    float *w = a.wts + (int64_t)r * a.k;
    float wsel[8], sel;
    int isel[8];
    moe_topk(lg, E, a.k, lane, isel, wsel, sel);
    if (lane == 0) {
      for (int j = 0; j < a.k; ++j) {
        if (a.arrive) __hip_atomic_store(ids + j, isel[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else ids[j] = isel[j];
        w[j] = a.renorm ? wsel[j] / sel : wsel[j];
        if (a.ids_record) a.ids_record[(int64_t)r * a.k + j] = isel[j];
      }
      if (a.gate) a.gate[r] = a.w_sh_gate ? 1.0f / (1.0f + expf(-dot)) : 1.0f;
    }
  }
  if (!a.arrive) return;
  // the ids are complete, then one arrival for the block; the last block
  // to arrive (counter rows - 1) groups every row's pairs
  __shared__ int last_s;
  __shared__ GroupLds gs;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    last_s = __hip_atomic_fetch_add(a.arrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.rows - 1;
  __syncthreads();
  if (!last_s) return;
  if (threadIdx.x == 0) __hip_atomic_store(a.arrive, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  group_pairs<true>(a, gs);
}

// x[r][c] += sum_j w_j y[pair(r, j)][c] + gate_r ysh[r][c]; grid (columns / 256, rows)
__global__ __launch_bounds__(256) void moe_combine_kernel(float *x, const float *y, const float *ysh,
                                                         const float *wts, const float *gate,
                                                         const int32_t *pair_of, int k, int H, int sh_parts,
                                                         int64_t sh_stride) {
  const int r = blockIdx.y, c = blockIdx.x * blockDim.x + threadIdx.x;
  float w[8];
  int64_t pr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int jj = min(j, k - 1);
    w[j] = wts[r * k + jj];
    pr[j] = pair_of ? pair_of[r * k + jj] : r * k + jj;
  }
  const float gs = ysh ? gate[r] : 0.f;
  if (c >= H) return;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < k) acc += w[j] * y[pr[j] * H + c];
  if (ysh) {
    float s = 0.f;
    for (int i = 0; i < sh_parts; ++i) s += ysh[i * sh_stride + (int64_t)r * H + c];
    acc += gs * s;
  }
  x[(int64_t)r * H + c] += acc;
}

}  // namespace

hipError_t launch_moe_route(const MoeRouteArgs &a, bool group, hipStream_t st) {
  if (a.E > 256 || a.k > 8 || (group && a.rows * a.k > GROUP_MAX_PAIRS) || a.extra_groups < 0 ||
      a.extra_groups > 8)
    return hipErrorInvalidValue;
  MoeRouteArgs b = a;
  if (!group || !a.w_router) b.arrive = nullptr;  // only the one-launch router groups by itself
  if (b.w_router) {
    if (!b.act_f32 || !b.gamma || b.H % 8 || b.H > MOE_ROUTER_MAX_H) return hipErrorInvalidValue;
    hipLaunchKernelGGL(moe_router_route_kernel, dim3(b.rows), dim3(RR_THREADS), (size_t)(b.H + b.E) * 4, st, b);
  } else {
    hipLaunchKernelGGL(moe_route_kernel, dim3(b.rows), dim3(ROUTE_THREADS), 0, st, b);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !group || b.arrive) return e;
  hipLaunchKernelGGL(moe_group_kernel, dim3(1), dim3(256), 0, st, b);
  return hipGetLastError();
}

hipError_t launch_moe_combine(float *x, const float *y, const float *ysh, const float *wts,
                              const float *gate, const int32_t *pair_of, int rows, int k, int H,
                              hipStream_t st, int sh_parts, int64_t sh_stride) {
  if (k < 1 || k > 8 || sh_parts < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_combine_kernel, dim3((H + 255) / 256, rows), dim3(256), 0, st, x, y, ysh, wts, gate,
                     pair_of, k, H, sh_parts, sh_stride);
  return hipGetLastError();
}
