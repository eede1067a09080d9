// Row-wise kernels of the step: embedding gather, RMSNorm (with the bf16
// cast of the projection input fused in) for the chunk-sized row counts,
// and the transposing import of a V-cache prefix.  All are HBM/latency bound
// and move each element once; reductions run in a fixed order.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace {

// x[r] = E[token] widened to fp32, scale 1 (pipeline.rs embed_single;
// engine.zig Engine.forward with embed_scale 1).  Token ids were validated
// on the host; next_token values come from argmax and are in range.
__global__ __launch_bounds__(256) void embed_kernel(const uint16_t *E, const int32_t *ids,
                                                    const int32_t *next_token,
                                                    const int32_t *row_seq, int use_next, int H,
                                                    float *x, const uint32_t *o_cnt, uint32_t *o_base,
                                                    int n_o, int o_stride) {
  const int r = blockIdx.x;
  if (r == 0)
    for (int i = threadIdx.x; i < n_o; i += blockDim.x)
      o_base[i] = __hip_atomic_load(const_cast<uint32_t *>(o_cnt + (int64_t)i * o_stride), __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
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

// out = x / sqrt(mean(x^2) + eps) * g: engine.zig rmsnormColumn (eps inside
// the root, gain after), accumulated in fp32, stored as split bf16 (or as
// plain bf16 when out_lo is 0, or as fp32).
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float *x, int64_t ldx, const float *g,
                                                      int H, float eps, uint16_t *out,
                                                      int64_t ldo, int64_t out_lo, float *out_f32) {
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
    if (out_f32) {
      *reinterpret_cast<f32x4 *>(out_f32 + (int64_t)blockIdx.x * ldo + j) =
          f32x4{v[0] * inv * w[0], v[1] * inv * w[1], v[2] * inv * w[2], v[3] * inv * w[3]};
      continue;
    }
    u32x2 oh, ol;
    { const u32pair t_ = pack_split2(v[0] * inv * w[0], v[1] * inv * w[1]); oh[0] = t_.hi; ol[0] = t_.lo; }
    { const u32pair t_ = pack_split2(v[2] * inv * w[2], v[3] * inv * w[3]); oh[1] = t_.hi; ol[1] = t_.lo; }
    *reinterpret_cast<u32x2 *>(orow + j) = oh;
    if (out_lo) *reinterpret_cast<u32x2 *>(orow + out_lo + j) = ol;
  }
}

// Per-head QK-norm (engine.zig applyHeadNorm: RMSNorm of each q and k head
// with gains [d] and the model's eps, before RoPE), then RoPE ("rope"
// pairing u_i with u_{i+d/2}), the q store and the KV append, as the fused
// QKV epilogue does them when there is no per-head norm.  One 64-lane block
// per (row, head of q, k or v); lane i owns the pair (i, i + d/2).
__global__ __launch_bounds__(64) void qk_norm_rope_kernel(QkNormArgs a) {
  const int nh = a.Hq + 2 * a.Hkv;
  const int r = blockIdx.x / nh, hh = blockIdx.x - r * nh;
  const int d = a.d, half = d / 2, i = threadIdx.x;
  const bool on = i < half;
  const float *src = a.qkv + (int64_t)r * a.ld + (int64_t)hh * d;
  float u0 = on ? src[i] : 0.f, u1 = on ? src[i + half] : 0.f;
  const int pos = a.row_pos[r], seq = a.row_seq[r];
  int prow;
  const int64_t base = kv_loc(a.pt, a.mp, a.S, a.seq_stride, seq, pos, prow) + a.layer_off;
  if (hh < a.Hq + a.Hkv) {
    const float ss = wave_sum(u0 * u0 + u1 * u1);
    const float inv = 1.0f / sqrtf(ss / (float)d + a.eps);
    if (!on) return;
    const float *g = hh < a.Hq ? a.q_norm : a.k_norm;
    u0 = u0 * inv * g[i];
    u1 = u1 * inv * g[i + half];
    const float2 t = a.cs[(int64_t)pos * half + i];
    const float r0 = u0 * t.x - u1 * t.y;
    const float r1 = u0 * t.y + u1 * t.x;
    if (hh < a.Hq) {
      uint16_t *dst = a.q + ((int64_t)r * a.Hq + hh) * d;
      uint32_t h0, l0, h1, l1;
      split_bf16(r0, h0, l0);
      split_bf16(r1, h1, l1);
      dst[i] = (uint16_t)h0;
      dst[i + half] = (uint16_t)h1;
      dst[a.q_lo + i] = (uint16_t)l0;
      dst[a.q_lo + i + half] = (uint16_t)l1;
    } else {
      uint16_t *dst = a.kcache + base + ((int64_t)(hh - a.Hq) * a.S + prow) * d;
      dst[i] = (uint16_t)f32_to_bf16_bits(r0);
      dst[i + half] = (uint16_t)f32_to_bf16_bits(r1);
    }
  } else if (on) {
    uint16_t *vt = a.vcache + base + (int64_t)(hh - a.Hq - a.Hkv) * d * a.S;
    vt[(int64_t)i * a.S + prow] = (uint16_t)f32_to_bf16_bits(u0);
    vt[(int64_t)(i + half) * a.S + prow] = (uint16_t)f32_to_bf16_bits(u1);
  }
}

// Per-row int8 quantisation: e is the smallest integer with 127 * 2^e >= a
// (a = the row's largest magnitude; a = m 2^p with m in [0.5, 1) gives
// e = p - 7 when m <= 127/128, else p - 6), q = rint(w / 2^e) (ties to
// even; the division by a power of two is exact).  The dequantised q 2^e
// has at most 7 significant bits and is stored exactly as bf16.  One block
// per row.
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t *W, int K, int8_t *q, float *scale,
                                                            uint16_t *deq) {
  __shared__ float red[4];
  const int64_t r = blockIdx.x;
  const uint16_t *w = W + r * K;
  float a = 0.f;
  for (int k = threadIdx.x; k < K; k += 256) a = fmaxf(a, fabsf(bf16_to_f32(w[k])));
  a = wave_max(a);
  if ((threadIdx.x & (WAVE - 1)) == 0) red[threadIdx.x / WAVE] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  int e = 0;
  if (a > 0.f) {
    int p;
    const float m = frexpf(a, &p);
    e = (m <= 0.9921875f) ? p - 7 : p - 6;
  }
  const float inv = ldexpf(1.0f, -e), s = ldexpf(1.0f, e);
  for (int k = threadIdx.x; k < K; k += 256) {
    const float c = rintf(bf16_to_f32(w[k]) * inv);
    q[r * K + k] = (int8_t)c;
    deq[r * K + k] = (uint16_t)f32_to_bf16_bits(c * s);
  }
  if (threadIdx.x == 0) scale[r] = s;
}

// 4-bit quantisation, one thread per group of 32 consecutive weights of a
// row: e is the smallest integer with 7 * 2^e >= a (a = the group's largest
// magnitude; a < 2^p from frexp, so e starts at p - 2 and steps down while
// 7 * 2^(e-1) still covers a), q = rint(w / 2^e) (ties to even), |q| <= 7.
// Codes are stored offset by 8 as nibbles (element 2j in the low nibble of
// byte j, 2j + 1 in the high one), the exponent as one int8, and the
// dequantised q 2^e (3 significant bits) exactly as bf16.
__global__ __launch_bounds__(256) void quantize_q4_kernel(const uint16_t *W, int64_t groups, int K, uint8_t *codes,
                                                          int8_t *exps, uint16_t *deq) {
  const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gi >= groups) return;
  const int gpr = K / 32;
  const int64_t r = gi / gpr;
  const int64_t k0 = r * K + (gi - r * gpr) * 32;
  float w[32];
#pragma unroll
  for (int j = 0; j < 32; j += 8) {
    const u32x4 v = load16(W + k0 + j);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      w[j + 2 * h] = bf16_lo(v[h]);
      w[j + 2 * h + 1] = bf16_hi(v[h]);
    }
  }
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) a = fmaxf(a, fabsf(w[j]));
  int e = 0;
  if (a > 0.f) {
    int p;
    (void)frexpf(a, &p);
    e = p - 2;
    while (7.0f * ldexpf(1.0f, e - 1) >= a) --e;
  }
  const float inv = ldexpf(1.0f, -e), s = ldexpf(1.0f, e);
  uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float c = rintf(w[j] * inv);
    packed[j >> 3] |= (uint32_t)((int)c + 8) << (4 * (j & 7));
    deq[k0 + j] = (uint16_t)f32_to_bf16_bits(c * s);
  }
  *reinterpret_cast<u32x4 *>(codes + k0 / 2) = u32x4{packed[0], packed[1], packed[2], packed[3]};
  exps[gi] = (int8_t)e;
}

// The last node of a captured decode step: record the step's greedy token
// and move the row to the next position (the next replay reads it there).
__global__ __launch_bounds__(64) void decode_advance_kernel(int32_t *row_pos, const int32_t *next_token, int seq,
                                                            int32_t *out) {
  if (threadIdx.x != 0) return;
  const int i = out[0];
  out[1 + i] = next_token[seq];
  out[0] = i + 1;
  row_pos[0] += 1;
}

}  // namespace

hipError_t launch_decode_advance(int32_t *row_pos, const int32_t *next_token, int seq, int32_t *out,
                                 hipStream_t st) {
  hipLaunchKernelGGL(decode_advance_kernel, dim3(1), dim3(64), 0, st, row_pos, next_token, seq, out);
  return hipGetLastError();
}

hipError_t launch_quantize_rows(const uint16_t *W, int64_t rows, int K, int8_t *q, float *scale, uint16_t *deq,
                                hipStream_t st) {
  if (rows <= 0 || rows > 0x7fffffff || K <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)rows), dim3(256), 0, st, W, K, q, scale, deq);
  return hipGetLastError();
}

hipError_t launch_quantize_q4(const uint16_t *W, int64_t rows, int K, uint8_t *codes, int8_t *exps, uint16_t *deq,
                              hipStream_t st) {
  if (rows <= 0 || K <= 0 || K % 32) return hipErrorInvalidValue;
  const int64_t groups = rows * (K / 32);
  const int64_t blocks = (groups + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_q4_kernel, dim3((unsigned)blocks), dim3(256), 0, st, W, groups, K, codes, exps, deq);
  return hipGetLastError();
}

hipError_t launch_qk_norm_rope(const QkNormArgs &a, hipStream_t st) {
  if (a.d / 2 > 64 || a.rows <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(qk_norm_rope_kernel, dim3(a.rows * (a.Hq + 2 * a.Hkv)), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_embed(const uint16_t *E, const int32_t *ids, const int32_t *next_token,
                        const int32_t *row_seq, int use_next, int rows, int H, float *x,
                        const uint32_t *o_cnt, uint32_t *o_base, int n_o, int o_stride, hipStream_t st) {
  hipLaunchKernelGGL(embed_kernel, dim3(rows), dim3(256), 0, st, E, ids, next_token, row_seq,
                     use_next, H, x, o_cnt, o_base, n_o, o_stride);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float *x, int64_t ldx, const float *g, int rows, int H, float eps,
                          uint16_t *out, int64_t ldo, int64_t out_lo, hipStream_t st, float *out_f32) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(256), 0, st, x, ldx, g, H, eps, out, ldo, out_lo, out_f32);
  return hipGetLastError();
}


// Greedy argmax over per-tile candidates (value, index) of one row, lowest
// index on ties (the strict '>' scans of engine.zig's MoE prefill test and
// pipeline.rs ppl_ids).  Rows of one sequence are consecutive (a prefill
// chunk, or one row per sequence in a decode batch); blocks reduce rows in
// parallel, so only the last row of each run of equal sequences writes that
// sequence's next token.
namespace {
constexpr int FIN_BATCH = 16;

__global__ __launch_bounds__(1024) void argmax_finalize_kernel(const float *pv, const int32_t *pi, int nparts,
                                                               int rows, int32_t *idx, int32_t *next_token,
                                                               const int32_t *row_seq) {
  __shared__ float sv[16];
  __shared__ int si[16];
  for (int r = blockIdx.x; r < rows; r += gridDim.x) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    // FIN_BATCH candidates per thread in flight at a time (clamped indices,
    // so the loads are unconditional; the order of the comparisons does not
    // matter, `better` being a total order on distinct indices)
    for (int p0 = 0; p0 < nparts; p0 += FIN_BATCH * (int)blockDim.x) {
      float v[FIN_BATCH];
      int ix[FIN_BATCH];
#pragma unroll
      for (int u = 0; u < FIN_BATCH; ++u) {
        const int p = min(p0 + u * (int)blockDim.x + (int)threadIdx.x, nparts - 1);
        v[u] = pv[(int64_t)r * nparts + p];
        ix[u] = pi[(int64_t)r * nparts + p];
      }
#pragma unroll
      for (int u = 0; u < FIN_BATCH; ++u)
        if (better(v[u], ix[u], bv, bi)) {
          bv = v[u];
          bi = ix[u];
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, WAVE);
      const int oi = __shfl_xor(bi, o, WAVE);
      if (better(ov, oi, bv, bi)) {
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
      for (int i = 1; i < (int)(blockDim.x / WAVE); ++i)
        if (better(sv[i], si[i], bv, bi)) {
          bv = sv[i];
          bi = si[i];
        }
      if (bi == 0x7fffffff) bi = 0;
      if (idx) idx[r] = bi;
      if (next_token && (r == rows - 1 || row_seq[r + 1] != row_seq[r])) next_token[row_seq[r]] = bi;
    }
    __syncthreads();
  }
}
}  // namespace

hipError_t launch_argmax_finalize(const float *part_val, const int32_t *part_idx, int nparts, int rows,
                                  int32_t *idx, int32_t *next_token, const int32_t *row_seq,
                                  hipStream_t st) {
  if (nparts < 1 || rows < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(argmax_finalize_kernel, dim3(std::min(rows, 1024)), dim3(1024), 0, st, part_val, part_idx,
                     nparts, rows, idx, next_token, row_seq);
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

namespace {
// KV-prefix import into a paged cache: position t of the sequence lives in
// page pt[t / P] at row t % P; K rows [P][d] and V^T rows [d][P] per kv head
// inside a page's layer.  K and V both come as [Hkv][len][d]; each block
// moves a 64-position x 64-dim tile of one head (V through LDS, so both the
// read and the transposed write are coalesced).
__global__ __launch_bounds__(256) void kv_load_paged_kernel(const uint16_t *src_k, const uint16_t *src_v,
                                                            uint16_t *kpool, uint16_t *vpool, const int32_t *pt,
                                                            int64_t unit, int64_t layer_off, int len, int d, int P) {
  __shared__ uint16_t tile[64][65];
  const int t0 = blockIdx.x * 64, j0 = blockIdx.y * 64, g = blockIdx.z;
  const uint16_t *sk = src_k + (int64_t)g * len * d, *sv = src_v + (int64_t)g * len * d;
  for (int e = threadIdx.x; e < 64 * 64; e += blockDim.x) {
    const int tt = e / 64, jj = e % 64;
    const int t = t0 + tt, j = j0 + jj;
    if (t < len && j < d) {
      const int64_t base = (int64_t)pt[t / P] * unit + layer_off;
      kpool[base + ((int64_t)g * P + t % P) * d + j] = sk[(int64_t)t * d + j];
    }
    tile[tt][jj] = (t < len && j < d) ? sv[(int64_t)t * d + j] : 0;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += blockDim.x) {
    const int jj = e / 64, tt = e % 64;
    const int t = t0 + tt, j = j0 + jj;
    if (t < len && j < d) {
      const int64_t base = (int64_t)pt[t / P] * unit + layer_off;
      vpool[base + ((int64_t)g * d + j) * P + t % P] = tile[tt][jj];
    }
  }
}
}  // namespace

hipError_t launch_kv_load_paged(const uint16_t *src_k, const uint16_t *src_v, uint16_t *kpool, uint16_t *vpool,
                                const int32_t *pt, int64_t unit, int64_t layer_off, int Hkv, int len, int d, int P,
                                hipStream_t st) {
  if (len <= 0 || P <= 0 || d <= 0) return hipErrorInvalidValue;
  dim3 grid((len + 63) / 64, (d + 63) / 64, Hkv);
  hipLaunchKernelGGL(kv_load_paged_kernel, grid, dim3(256), 0, st, src_k, src_v, kpool, vpool, pt, unit, layer_off,
                     len, d, P);
  return hipGetLastError();
}

hipError_t launch_kv_load_v(const uint16_t *src, uint16_t *dst, int Hkv, int len, int d, int S,
                            hipStream_t st) {
  dim3 grid((len + 63) / 64, (d + 63) / 64, Hkv);
  hipLaunchKernelGGL(kv_load_v_kernel, grid, dim3(256), 0, st, src, dst, len, d, S);
  return hipGetLastError();
}
