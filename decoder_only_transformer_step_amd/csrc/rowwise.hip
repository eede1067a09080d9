// Row-wise kernels of the step: embedding gather, RMSNorm (with the bf16
// cast of the projection input fused in), bias + RoPE + KV-cache append,
// and the greedy argmax over the vocabulary.  All are HBM/latency bound and
// move each element once; reductions run in a fixed order.
#include "common.h"
#include "launch.h"

namespace {

// x[r] = E[token] widened to fp32, scale 1 (pipeline.rs embed_single;
// engine.zig Engine.forward with embed_scale 1).  Token ids were validated
// on the host; next_token values come from argmax and are in range.
__global__ __launch_bounds__(256) void embed_kernel(const uint16_t *E, const int32_t *ids,
                                                    const int32_t *next_token,
                                                    const int32_t *row_seq, int use_next, int H,
                                                    float *x) {
  const int r = blockIdx.x;
  const int tok = use_next ? next_token[row_seq[r]] : ids[r];
  const uint16_t *src = E + (int64_t)tok * H;
  float *dst = x + (int64_t)r * H;
  for (int j = threadIdx.x * 8; j < H; j += blockDim.x * 8) {
    const u32x4 w = load16(src + j);
    f32x4 lo = {bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
    f32x4 hi = {bf16_lo(w[2]), bf16_hi(w[2]), bf16_lo(w[3]), bf16_hi(w[3])};
    *reinterpret_cast<f32x4 *>(dst + j) = lo;
    *reinterpret_cast<f32x4 *>(dst + j + 4) = hi;
  }
}

// out = bf16(x / sqrt(mean(x^2) + eps) * g): engine.zig rmsnormColumn (eps
// inside the root, gain after), accumulated in fp32.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float *x, int64_t ldx, const float *g,
                                                      int H, float eps, uint16_t *out,
                                                      int64_t ldo) {
  __shared__ float lds[4];
  const float *xr = x + (int64_t)blockIdx.x * ldx;
  float ss = 0.f;
  for (int j = threadIdx.x * 4; j < H; j += blockDim.x * 4) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(xr + j);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = block_sum<4>(ss, lds);
  const float inv = 1.0f / sqrtf(ss / (float)H + eps);
  uint16_t *orow = out + (int64_t)blockIdx.x * ldo;
  for (int j = threadIdx.x * 4; j < H; j += blockDim.x * 4) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(xr + j);
    const f32x4 w = *reinterpret_cast<const f32x4 *>(g + j);
    u32x2 o;
    o[0] = pack_bf16x2(v[0] * inv * w[0], v[1] * inv * w[1]);
    o[1] = pack_bf16x2(v[2] * inv * w[2], v[3] * inv * w[3]);
    *reinterpret_cast<u32x2 *>(orow + j) = o;
  }
}

// Bias, then RoPE on q and k, then the cache append (engine.zig
// ropeAndCache with the half-split pairing; decoder.rs AttnWeights: bias is
// added before RoPE).  Pair i of a head is (u_i, u_{i+d/2}), rotated by the
// angle pos * base^(-2i/d) whose cos/sin come from the fp64-built table.
// K goes to row pos of the [S][d] cache, V to column pos of the transposed
// [d][S] cache.
__global__ __launch_bounds__(256) void rope_append_kernel(RopeArgs a) {
  const int r = blockIdx.x;
  const int d = a.d, half = d / 2;
  const int qkvr = (a.Hq + 2 * a.Hkv) * d;
  const float *src = a.qkv + (int64_t)r * qkvr;
  const int pos = a.row_pos[r], seq = a.row_seq[r];
  const float2 *cs = a.cs + (int64_t)pos * half;
  uint16_t *kb = a.kcache + (int64_t)seq * a.seq_stride + a.layer_off;
  uint16_t *vb = a.vcache + (int64_t)seq * a.seq_stride + a.layer_off;
  const int nq = a.Hq * half, nk = a.Hkv * half, nv = a.Hkv * d;
  for (int it = threadIdx.x; it < nq + nk + nv; it += blockDim.x) {
    if (it < nq + nk) {
      const bool isq = it < nq;
      const int j = isq ? it : it - nq;
      const int h = j / half, i = j - h * half;
      const int e0 = (isq ? 0 : a.Hq * d) + h * d + i;
      float u0 = src[e0], u1 = src[e0 + half];
      if (a.bias) {
        u0 += a.bias[e0];
        u1 += a.bias[e0 + half];
      }
      const float2 t = cs[i];
      const float r0 = u0 * t.x - u1 * t.y;
      const float r1 = u0 * t.y + u1 * t.x;
      if (isq) {
        uint16_t *qo = a.q + ((int64_t)r * a.Hq + h) * d;
        qo[i] = (uint16_t)f32_to_bf16_bits(r0);
        qo[i + half] = (uint16_t)f32_to_bf16_bits(r1);
      } else {
        uint16_t *ko = kb + ((int64_t)h * a.S + pos) * d;
        ko[i] = (uint16_t)f32_to_bf16_bits(r0);
        ko[i + half] = (uint16_t)f32_to_bf16_bits(r1);
      }
    } else {
      const int j = it - nq - nk;
      const int h = j / d, i = j - h * d;
      const int e0 = (a.Hq + a.Hkv) * d + h * d + i;
      float v = src[e0];
      if (a.bias) v += a.bias[e0];
      vb[((int64_t)h * d + i) * a.S + pos] = (uint16_t)f32_to_bf16_bits(v);
    }
  }
}

// Greedy argmax over one row of logits, lowest index on ties (the strict '>'
// scans of engine.zig's MoE prefill test and pipeline.rs ppl_ids).
__global__ __launch_bounds__(1024) void argmax_kernel(const float *logits, int64_t ld, int V,
                                                      int32_t *idx, int32_t *next_token,
                                                      const int32_t *row_seq) {
  __shared__ float sv[16];
  __shared__ int si[16];
  const float *row = logits + (int64_t)blockIdx.x * ld;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int v = threadIdx.x; v < V; v += blockDim.x) {
    const float x = row[v];
    if (x > bv) {
      bv = x;
      bi = v;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(bv, o, WAVE);
    const int oi = __shfl_xor(bi, o, WAVE);
    if (ov > bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  }
  const int w = threadIdx.x / WAVE;
  if ((threadIdx.x & (WAVE - 1)) == 0) {
    sv[w] = bv;
    si[w] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int nw = blockDim.x / WAVE;
    for (int i = 1; i < nw; ++i)
      if (sv[i] > bv || (sv[i] == bv && si[i] < bi)) {
        bv = sv[i];
        bi = si[i];
      }
    if (bi == 0x7fffffff) bi = 0;
    if (idx) idx[blockIdx.x] = bi;
    if (next_token) next_token[row_seq[blockIdx.x]] = bi;
  }
}

}  // namespace

hipError_t launch_embed(const uint16_t *E, const int32_t *ids, const int32_t *next_token,
                        const int32_t *row_seq, int use_next, int rows, int H, float *x,
                        hipStream_t st) {
  hipLaunchKernelGGL(embed_kernel, dim3(rows), dim3(256), 0, st, E, ids, next_token, row_seq,
                     use_next, H, x);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float *x, int64_t ldx, const float *g, int rows, int H, float eps,
                          uint16_t *out, int64_t ldo, hipStream_t st) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(256), 0, st, x, ldx, g, H, eps, out, ldo);
  return hipGetLastError();
}

hipError_t launch_rope_append(const RopeArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(rope_append_kernel, dim3(a.rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_argmax(const float *logits, int64_t ld, int rows, int V, int32_t *idx,
                         int32_t *next_token, const int32_t *row_seq, hipStream_t st) {
  hipLaunchKernelGGL(argmax_kernel, dim3(rows), dim3(1024), 0, st, logits, ld, V, idx, next_token,
                     row_seq);
  return hipGetLastError();
}

// KV-prefix import for V: [Hkv][len][d] (position-major, as handed in) to the
// transposed cache [Hkv][d][S].  64x64 tiles through LDS so both the read and
// the write are coalesced.
namespace {
__global__ __launch_bounds__(256) void kv_load_v_kernel(const uint16_t *src, uint16_t *dst, int len,
                                                        int d, int S) {
  __shared__ uint16_t tile[64][65];
  const int t0 = blockIdx.x * 64, j0 = blockIdx.y * 64, g = blockIdx.z;
  const uint16_t *s = src + (int64_t)g * len * d;
  uint16_t *o = dst + (int64_t)g * d * S;
  for (int e = threadIdx.x; e < 64 * 64; e += blockDim.x) {
    const int tt = e / 64, jj = e % 64;
    const int t = t0 + tt, j = j0 + jj;
    tile[tt][jj] = (t < len && j < d) ? s[(int64_t)t * d + j] : 0;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += blockDim.x) {
    const int jj = e / 64, tt = e % 64;
    const int t = t0 + tt, j = j0 + jj;
    if (t < len && j < d) o[(int64_t)j * S + t] = tile[tt][jj];
  }
}
}  // namespace

hipError_t launch_kv_load_v(const uint16_t *src, uint16_t *dst, int Hkv, int len, int d, int S,
                            hipStream_t st) {
  dim3 grid((len + 63) / 64, (d + 63) / 64, Hkv);
  hipLaunchKernelGGL(kv_load_v_kernel, grid, dim3(256), 0, st, src, dst, len, d, S);
  return hipGetLastError();
}
