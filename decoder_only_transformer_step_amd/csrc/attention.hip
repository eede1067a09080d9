// Causal GQA attention over the bf16 KV cache, for decode (one query row per
// sequence) and chunked prefill (many query rows of one sequence).
//
// Math (engine.zig Engine.forward / attentionDecode; pipeline.rs
// Pipeline::new): for query head h at position p, kv head
// g = floor(h Hkv / Hq), s_t = q . k_t / sqrt(d) for t <= p, w = softmax(s),
// o = sum_t w_t v_t.
//
// gfx950 design (flash-decoding with split KV):
//  * A "column group" is up to 16 query columns that share one kv head and
//    one sequence: G heads of one decode row, or 16/G rows x G heads of a
//    prefill chunk.  The kv head's K and V are read once for all of them.
//  * A task (one wavefront) takes one column group and one contiguous key
//    range (split).  Per 32-key tile: S^T = K Q^T with 8 MFMA 16x16x32
//    (K rows straight from HBM as the A operand, Q^T in registers as B),
//    an online softmax per column in fp32 (exp2 with log2(e)/sqrt(d)
//    folded into the scale), and O^T += V^T P^T with d/16 MFMAs.
//  * V is stored transposed in the cache ([dim][position]), so the A operand
//    of the PV product is two 8-byte loads per lane, and the B operand
//    (P^T) is exactly the lane's own scores: the MFMA k index is mapped to
//    keys {4 (l/16) + j, 16 + 4 (l/16) + j}, the layout the QK product
//    leaves them in.  No LDS round trip, no cross-lane shuffles for P.
//  * Each task writes (m, l, O) partials; attn_merge combines the splits of
//    a column group in fixed order (log-sum-exp), so results do not depend
//    on scheduling.  With a single split the task normalises and writes the
//    output itself.
#include "common.h"
#include "launch.h"

namespace {

constexpr float NEG_SENTINEL = -1.0e30f;

__device__ __forceinline__ int group_keys(const AttnArgs &a, int rg, int c, bool &valid, int &row,
                                          int &head, int g) {
  const int G = a.G;
  row = rg * a.rows_per_group + c / G;
  head = g * G + c % G;
  valid = (c < a.rows_per_group * G) && (row < a.rows);
  return valid ? a.row_pos[row] : -1;
}

template <int D>
__global__ __launch_bounds__(256) void attn_partial_kernel(AttnArgs a) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int task = blockIdx.x * 4 + threadIdx.x / WAVE;
  if (task >= a.n_groups * a.n_splits) return;
  const int gi = task / a.n_splits, split = task - gi * a.n_splits;
  const int g = gi % a.Hkv, rg = gi / a.Hkv;
  const int c = lane & 15, quad = lane >> 4;

  bool valid;
  int row, head;
  const int pos = group_keys(a, rg, c, valid, row, head, g);
  // keys of the group: 0 .. max position of its rows (wave-wide max over columns)
  int kmax = pos;
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) kmax = max(kmax, __shfl_xor(kmax, o, WAVE));
  const int keys = kmax + 1;
  const int k0 = split * a.kc;
  if (k0 >= keys) return;
  const int k1 = min(k0 + a.kc, keys);

  const int seq = a.row_seq[rg * a.rows_per_group];
  const uint16_t *kb = a.kcache + (int64_t)seq * a.seq_stride + a.layer_off + (int64_t)g * a.S * D;
  const uint16_t *vb = a.vcache + (int64_t)seq * a.seq_stride + a.layer_off + (int64_t)g * D * a.S;

  u32x4 qf[D / 32];
  const uint16_t *qrow = a.q + ((int64_t)row * a.Hq + head) * D + quad * 8;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) qf[ks] = valid ? load16(qrow + ks * 32) : u32x4{0u, 0u, 0u, 0u};

  float m_run = NEG_SENTINEL, l_run = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int t0 = k0; t0 < k1; t0 += 32) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    const uint16_t *k_lo = kb + (int64_t)(t0 + c) * D + quad * 8;
    const uint16_t *k_hi = k_lo + 16 * D;
    u32x4 ka[D / 32], kbv[D / 32];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      ka[ks] = load16(k_lo + ks * 32);
      kbv[ks] = load16(k_hi + ks * 32);
    }
    u32x2 va[D / 16], vv[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const uint16_t *vr = vb + (int64_t)(dt * 16 + c) * a.S + t0 + quad * 4;
      va[dt] = load8(vr);
      vv[dt] = load8(vr + 16);
    }
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      s0 = mfma16x16x32(as_bf16x8(ka[ks]), as_bf16x8(qf[ks]), s0);
      s1 = mfma16x16x32(as_bf16x8(kbv[ks]), as_bf16x8(qf[ks]), s1);
    }
    // lane holds S[key = t0 + 4 quad + i][col c] in s0, key + 16 in s1
    float sv[8];
    float tmax = NEG_SENTINEL;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key0 = t0 + quad * 4 + i, key1 = key0 + 16;
      sv[i] = (key0 <= pos && key0 < k1) ? s0[i] * a.scale_log2 : -INFINITY;
      sv[4 + i] = (key1 <= pos && key1 < k1) ? s1[i] * a.scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, fmaxf(sv[i], sv[4 + i]));
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, WAVE));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, WAVE));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);
    float psum = 0.f;
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = exp2f(sv[i] - m_new);
      psum += p[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    u32x4 pb;
    pb[0] = pack_bf16x2(p[0], p[1]);
    pb[1] = pack_bf16x2(p[2], p[3]);
    pb[2] = pack_bf16x2(p[4], p[5]);
    pb[3] = pack_bf16x2(p[6], p[7]);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      acc[dt] *= alpha;
      u32x4 av;
      av[0] = va[dt][0];
      av[1] = va[dt][1];
      av[2] = vv[dt][0];
      av[3] = vv[dt][1];
      acc[dt] = mfma16x16x32(as_bf16x8(av), as_bf16x8(pb), acc[dt]);
    }
  }
  // acc[dt][i] = O^T[dim = dt*16 + 4 quad + i][col c]
  float l_tot = l_run + __shfl_xor(l_run, 16, WAVE);
  l_tot += __shfl_xor(l_tot, 32, WAVE);
  if (a.n_splits == 1) {
    if (!valid) return;
    const float inv = 1.0f / l_tot;
    uint16_t *orow = a.out + ((int64_t)row * a.Hq + head) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      u32x2 w;
      w[0] = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
      w[1] = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
      *reinterpret_cast<u32x2 *>(orow + dt * 16 + quad * 4) = w;
    }
    return;
  }
  float *po = a.part_o + ((int64_t)task * 16 + c) * D;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4 *>(po + dt * 16 + quad * 4) = acc[dt];
  if (quad == 0) {
    a.part_ml[((int64_t)task * 16 + c) * 2 + 0] = m_run;
    a.part_ml[((int64_t)task * 16 + c) * 2 + 1] = l_tot;
  }
}

// One block per column group: thread (c, j) combines column c's splits for
// dims j, j + 16, ... in split order.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  const int gi = blockIdx.x;
  const int g = gi % a.Hkv, rg = gi / a.Hkv;
  const int c = threadIdx.x >> 4, j = threadIdx.x & 15;
  bool valid;
  int row, head;
  const int pos = group_keys(a, rg, c, valid, row, head, g);
  // the group's key count, from its last valid row (positions grow with the row)
  int kmax = -1;
  for (int cc = 0; cc < 16; ++cc) {
    bool v2;
    int r2, h2;
    kmax = max(kmax, group_keys(a, rg, cc, v2, r2, h2, g));
  }
  (void)pos;
  if (!valid) return;
  const int nsp = min(a.n_splits, (kmax + 1 + a.kc - 1) / a.kc);
  const int64_t base = (int64_t)gi * a.n_splits;
  float M = NEG_SENTINEL;
  for (int s = 0; s < nsp; ++s) M = fmaxf(M, a.part_ml[((base + s) * 16 + c) * 2]);
  float L = 0.f;
  float o[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) o[t] = 0.f;
  for (int s = 0; s < nsp; ++s) {
    const float m = a.part_ml[((base + s) * 16 + c) * 2], l = a.part_ml[((base + s) * 16 + c) * 2 + 1];
    const float w = exp2f(m - M);
    L += w * l;
    const float *po = a.part_o + ((base + s) * 16 + c) * D;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) o[t] += w * po[t * 16 + j];
  }
  const float inv = 1.0f / L;
  uint16_t *orow = a.out + ((int64_t)row * a.Hq + head) * D;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) orow[t * 16 + j] = (uint16_t)f32_to_bf16_bits(o[t] * inv);
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, int head_dim, hipStream_t st) {
  const int tasks = a.n_groups * a.n_splits;
  dim3 grid((tasks + 3) / 4);
  if (head_dim == 128) hipLaunchKernelGGL(attn_partial_kernel<128>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(attn_partial_kernel<64>, grid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_splits == 1) return e;
  if (head_dim == 128) hipLaunchKernelGGL(attn_merge_kernel<128>, dim3(a.n_groups), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(attn_merge_kernel<64>, dim3(a.n_groups), dim3(256), 0, st, a);
  return hipGetLastError();
}
