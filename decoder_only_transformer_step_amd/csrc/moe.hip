// MoE routing and combine (pipeline.rs MoeFfn; engine.zig Engine.forward and
// Engine.prefill; decoder.rs MoeWeights).
//
//  route:   P = softmax over ALL expert logits of the normed FFN input; the
//           k largest (distinct experts, lower index first on ties) with
//           weight P_e, or P_e / sum over the chosen when renormalising;
//           the shared-expert scale sigmoid(w_sg . b) (1 without a gate).
//  group:   pairs (row, slot) sorted by expert, then by row: every chosen
//           expert becomes one group whose weights are streamed once for
//           all rows that chose it (engine.zig Engine.prefill batching).
//  combine: x += sum_j w_j y_pair(j) + gate * y_shared, slots in router order.
#include "common.h"
#include "launch.h"

namespace {

constexpr int ROUTE_THREADS = 256;

// One block per row: softmax, top-k, shared gate.
__global__ __launch_bounds__(ROUTE_THREADS) void moe_route_kernel(MoeRouteArgs a) {
  __shared__ float lg[256];
  __shared__ float red[4];
  __shared__ int taken[256];
  const int r = blockIdx.x, E = a.E;
  const float *row = a.logits + (int64_t)r * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    lg[e] = row[e];
    taken[e] = 0;
  }
  __syncthreads();
  // shared-expert gate: sigmoid(w_sg . b), fp32 dot in fixed order
  float dot = 0.f;
  if (a.w_sh_gate) {
    if (a.act_f32) {
      const float *b = a.act_f32 + (int64_t)r * a.H;
      for (int j = threadIdx.x; j < a.H; j += blockDim.x) dot += b[j] * bf16_to_f32(a.w_sh_gate[j]);
    } else {
      const uint16_t *b = a.act + (int64_t)r * a.H;
      for (int j = threadIdx.x; j < a.H; j += blockDim.x)
        dot += (bf16_to_f32(b[j]) + bf16_to_f32(b[a.act_lo + j])) * bf16_to_f32(a.w_sh_gate[j]);
    }
  }
  dot = block_sum<ROUTE_THREADS / WAVE>(dot, red);
  if (threadIdx.x == 0) {
    float m = -INFINITY;
    for (int e = 0; e < E; ++e) m = fmaxf(m, lg[e]);
    float z = 0.f;
    for (int e = 0; e < E; ++e) z += expf(lg[e] - m);
    float sel = 0.f;
    int32_t *ids = a.ids + (int64_t)r * a.k;
    float *w = a.wts + (int64_t)r * a.k;
    for (int j = 0; j < a.k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || lg[e] > lg[best])) best = e;
      taken[best] = 1;
      ids[j] = best;
      w[j] = expf(lg[best] - m) / z;
      sel += w[j];
    }
    if (a.renorm)
      for (int j = 0; j < a.k; ++j) w[j] /= sel;
    if (a.ids_record)
      for (int j = 0; j < a.k; ++j) a.ids_record[(int64_t)r * a.k + j] = ids[j];
    if (a.gate) a.gate[r] = a.w_sh_gate ? 1.0f / (1.0f + expf(-dot)) : 1.0f;
  }
}

// One block: group table over experts in increasing order, pairs by row.
__global__ __launch_bounds__(256) void moe_group_kernel(MoeRouteArgs a) {
  __shared__ int cnt[256];
  __shared__ int start[256];
  const int E = a.E, P = a.rows * a.k;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int c = 0;
    for (int p = 0; p < P; ++p) c += (a.ids[p] == e);
    cnt[e] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0, ng = 0;
    for (int e = 0; e < E; ++e) {
      start[e] = s;
      if (cnt[e]) {
        a.group_expert[ng] = e;
        a.group_start[ng] = s;
        a.group_count[ng] = cnt[e];
        ++ng;
      }
      s += cnt[e];
    }
    *a.n_groups = ng;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int o = start[e];
    for (int p = 0; p < P; ++p)
      if (a.ids[p] == e) {
        a.pair_row[o] = p / a.k;
        a.pair_of[p] = o;
        ++o;
      }
  }
}

__global__ __launch_bounds__(256) void moe_combine_kernel(float *x, const float *y, const float *ysh,
                                                         const float *wts, const float *gate,
                                                         const int32_t *pair_of, int k, int H) {
  const int r = blockIdx.x;
  float *xr = x + (int64_t)r * H;
  for (int c = threadIdx.x; c < H; c += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) acc += wts[r * k + j] * y[(int64_t)(pair_of ? pair_of[r * k + j] : r * k + j) * H + c];
    if (ysh) acc += gate[r] * ysh[(int64_t)r * H + c];
    xr[c] += acc;
  }
}

}  // namespace

hipError_t launch_moe_route(const MoeRouteArgs &a, bool group, hipStream_t st) {
  hipLaunchKernelGGL(moe_route_kernel, dim3(a.rows), dim3(ROUTE_THREADS), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !group) return e;
  hipLaunchKernelGGL(moe_group_kernel, dim3(1), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_moe_combine(float *x, const float *y, const float *ysh, const float *wts,
                              const float *gate, const int32_t *pair_of, int rows, int k, int H,
                              hipStream_t st) {
  hipLaunchKernelGGL(moe_combine_kernel, dim3(rows), dim3(256), 0, st, x, y, ysh, wts, gate,
                     pair_of, k, H);
  return hipGetLastError();
}
