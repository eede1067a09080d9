// Projection epilogues shared by the multi-row projection kernels: the
// weight row of a 16-row tile, and what happens to one output element
// (store, residual add, SwiGLU, bias + RoPE + KV append, logits).
#pragma once
#include "common.h"
#include "launch.h"

namespace {

template <int EPI>
constexpr int paired() {
  return (EPI == EPI_SWIGLU || EPI == EPI_QKV) ? 2 : 1;
}

// First weight row of tile b.
template <int EPI>
__device__ __forceinline__ int tile_n0(const GemmArgs &g, int b) {
  if (EPI == EPI_QKV) {
    const int per_head = g.qkv.d / 32;  // tile pairs per head
    const int hh = b / per_head, j = b - hh * per_head;
    return hh * g.qkv.d + 16 * j;
  }
  return b * 16;
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// Epilogue of one output element: row orow, weight row n = n0 + c (and its
// partner row n + np_off for the paired epilogues).
template <int EPI>
__device__ __forceinline__ void epi_apply(const GemmArgs &g, int64_t orow, int n, float v0, float v1) {
  if (EPI == EPI_STORE) {
    g.C[orow * g.ldc + n] = v0 + (g.bias ? g.bias[n] : 0.f);
  } else if (EPI == EPI_ADD) {
    g.C[orow * g.ldc + n] += v0;
  } else if (EPI == EPI_SWIGLU) {
    uint32_t hi, lo;
    split_bf16(silu_f(v0) * v1, hi, lo);
    g.Hout[orow * g.ldc + n] = (uint16_t)hi;
    g.Hout[g.h_lo + orow * g.ldc + n] = (uint16_t)lo;
  } else if (EPI == EPI_LOGITS) {
    g.C[orow * g.ldc + n] = v0;
  } else if (EPI == EPI_QKV) {
    // bias, then RoPE on q and k rows, then the KV-cache append (engine.zig
    // ropeAndCache, "rope" pairing u_i with u_{i+d/2}; decoder.rs AttnWeights:
    // bias before RoPE).  K goes to row pos of the [S][d] cache, V to
    // column pos of the transposed [d][S] cache.
    const QkvEpi &q = g.qkv;
    const int d = q.d, half = d / 2;
    const int hh = n / d, i = n - hh * d;  // i < d/2
    float u0 = v0, u1 = v1;
    if (q.bias) {
      u0 += q.bias[n];
      u1 += q.bias[n + half];
    }
    const int pos = q.row_pos[orow], seq = q.row_seq[orow];
    int prow;
    const int64_t base = kv_loc(q.pt, q.mp, q.P, q.seq_stride, seq, pos, prow) + q.layer_off;
    if (hh < q.Hq + q.Hkv) {
      const float2 t = q.cs[(int64_t)pos * half + i];
      const float r0 = u0 * t.x - u1 * t.y;
      const float r1 = u0 * t.y + u1 * t.x;
      if (hh < q.Hq) {
        uint16_t *dst = q.q + (orow * q.Hq + hh) * d;
        uint32_t h0, l0, h1, l1;
        split_bf16(r0, h0, l0);
        split_bf16(r1, h1, l1);
        dst[i] = (uint16_t)h0;
        dst[i + half] = (uint16_t)h1;
        dst[q.q_lo + i] = (uint16_t)l0;
        dst[q.q_lo + i + half] = (uint16_t)l1;
      } else {
        uint16_t *dst = q.kcache + base + ((int64_t)(hh - q.Hq) * q.S + prow) * d;
        dst[i] = (uint16_t)f32_to_bf16_bits(r0);
        dst[i + half] = (uint16_t)f32_to_bf16_bits(r1);
      }
    } else {
      uint16_t *vt = q.vcache + base + (int64_t)(hh - q.Hq - q.Hkv) * d * q.S;
      vt[(int64_t)i * q.S + prow] = (uint16_t)f32_to_bf16_bits(u0);
      vt[(int64_t)(i + half) * q.S + prow] = (uint16_t)f32_to_bf16_bits(u1);
    }
  }
}

}  // namespace
