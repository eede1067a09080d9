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
//    load; the LDS layout makes each wave's 16-byte reads contiguous across
//    lanes.  A DPP reduction gives the dot product.
//  * Pipeline: two register buffers per wave (8 KB each for bf16 weights,
//    4 KB for int8 codes); the activation loads
//    go out first, then the first two weight chunks, so the prologue waits
//    only for the activation while the weights stream in.  Every load is
//    unconditional, so the compiler's memory wait counts stay exact.
//  * One item per wave, 8 waves per block; blocks beyond the resident set
//    queue up behind the running ones.
//  * Grouped mode (MoE experts): blockIdx.y = routing slot; the weight base
//    moves to the chosen expert.  For batch-1 decode the kernel routes by
//    itself: each wave takes the top-k of the router logits (moe_topk, the
//    same selection as the route kernels) and moves to its slot's pick, so
//    no separate route launch sits between the router and the experts.
//  * Quantised weights (Q = 1): int8 codes with one scale per row.  The same
//    1 KB loads then carry 16 weights per lane (k = 16 l + 1024 s), the
//    activation slots hold 16 elements per lane and step, and the row's
//    scale multiplies the finished dot product: half the bytes per weight.
//  * 4-bit weights (Q = 2): one 16-byte lane load is 32 codes, exactly one
//    group with its own power-of-two scale (k = 32 l + 2048 s).  Codes are
//    stored offset by 8 (nibble n = q + 8), so a code converts with one
//    unsigned byte-to-float instruction after the nibbles are split into
//    bytes; the offset comes back as 8 times the group's activation sum,
//    computed once per block in LDS.  The group's dot product is then scaled
//    by its 2^e: a quarter of the bf16 bytes per weight, plus one exponent
//    byte per 32 weights.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace {


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

// Zero page for the lanes of a ragged last step (k >= K): their loads are
// redirected here by a pointer select, so every load is unconditional and
// the compiler's wait counts stay exact (a per-lane branch around a load, or
// a select on its value, makes it wait for everything in flight).
__device__ u32x4 gv_zero[1];

// Elements per lane and per 1 KB step: 8 bf16, 16 int8 or 32 4-bit weights.
template <int Q>
constexpr int gv_epl() {
  return Q == 2 ? 32 : Q ? 16 : 8;
}
// Bytes of a row of K weights.
template <int Q>
__device__ __forceinline__ int64_t gv_row_bytes(int K) {
  return Q == 2 ? K / 2 : Q ? K : 2 * (int64_t)K;
}
// 1 KB steps per register buffer (all rows of the item together): 8 KB for
// bf16; 4 KB for int8, so that a row of a K = 14336 projection still takes
// more than two chunks and its loads overlap the (heavier) int8 arithmetic.
template <int Q>
constexpr int gv_ch() {
  return Q ? 4 : 8;
}

// Loads of UNR 1 KB steps for every row the wave owns (wp: byte pointers
// with the lane's offset included).
template <int R, int UNR, int Q>
__device__ __forceinline__ void load_batch(u32x4 (&v)[UNR][R], const char *const (&wp)[R], int s0, int K,
                                           int lane) {
  constexpr int EPL = gv_epl<Q>();
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int st = s0 + u;
    const bool ok = st * 64 * EPL + lane * EPL < K;  // false for every lane past the last step
#pragma unroll
    for (int r = 0; r < R; ++r)
      v[u][r] = load16_nt(ok ? static_cast<const void *>(wp[r] + st * 1024) : static_cast<const void *>(gv_zero));
  }
}

// Activation layout in LDS: fp32, padded with zeros to whole 512-element
// steps, with lane l's 8 elements of step s as two 16-byte slots
// (s * 2 + h) * 64 + l, so that each 16-byte read of a wave is contiguous
// across the lanes (no bank conflicts).
__device__ __forceinline__ int xs_slot(int k) {  // k: element index, a multiple of 4
  return ((k >> 9) * 2 + ((k >> 2) & 1)) * 64 + ((k & 511) >> 3);
}
// int8 weights: lane l's 16 elements of step s in four slots (4 s + h) 64 + l.
__device__ __forceinline__ int xs_slot_q(int k) {
  return ((k >> 10) * 4 + ((k >> 2) & 3)) * 64 + ((k & 1023) >> 4);
}
// 4-bit weights: lane l's 32 elements of step s in eight slots (8 s + h) 64 + l.
__device__ __forceinline__ int xs_slot_q4(int k) {
  return ((k >> 11) * 8 + ((k >> 2) & 7)) * 64 + ((k & 2047) >> 5);
}
template <int Q>
__device__ __forceinline__ int xs_slot_t(int k) {
  return Q == 2 ? xs_slot_q4(k) : Q ? xs_slot_q(k) : xs_slot(k);
}

// 4-bit weights: the group exponents of UNR steps for every row (one byte per
// lane and step; lanes past the row read the zero page: exponent 0, and
// their codes and activations are zero).
template <int R, int UNR>
__device__ __forceinline__ void load_exps(int (&ev)[UNR][R], const int8_t *const (&ep)[R], int s0, int K,
                                          int lane) {
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int st = s0 + u;
    const bool ok = st * 2048 + lane * 32 < K;
#pragma unroll
    for (int r = 0; r < R; ++r)
      ev[u][r] = *(ok ? ep[r] + st * 64 : reinterpret_cast<const int8_t *>(gv_zero));
  }
}

// 4-bit dot product of one lane's group: nibbles n = q + 8, split into the
// bytes of lo (even elements) and hi (odd elements) of each 32-bit word;
// returns sum n_j x_j.  The empty asm statements only pin lo and hi as
// values: without them the compiler extracts every nibble with its own
// bit-field instruction instead of converting each byte of the two masked
// words directly (v_cvt_f32_ubyte0..3), one VALU instruction more per code.
__device__ __forceinline__ float q4_dot(const u32x4 &w, const f32x4 (&x)[8]) {
  float d = 0.f;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    uint32_t lo = w[h] & 0x0F0F0F0Fu, hi = (w[h] >> 4) & 0x0F0F0F0Fu;
    asm("" : "+v"(lo));
    asm("" : "+v"(hi));
    const f32x4 xa = x[2 * h], xb = x[2 * h + 1];
    d = fmaf((float)(lo & 0xFFu), xa[0], d);
    d = fmaf((float)(hi & 0xFFu), xa[1], d);
    d = fmaf((float)((lo >> 8) & 0xFFu), xa[2], d);
    d = fmaf((float)((hi >> 8) & 0xFFu), xa[3], d);
    d = fmaf((float)((lo >> 16) & 0xFFu), xb[0], d);
    d = fmaf((float)((hi >> 16) & 0xFFu), xb[1], d);
    d = fmaf((float)(lo >> 24), xb[2], d);
    d = fmaf((float)(hi >> 24), xb[3], d);
  }
  return d;
}

__device__ __forceinline__ float i8f(uint32_t w, int j) { return (float)(int8_t)(w >> (8 * j)); }

// acc[r] += dot(weights of batch, activation) over UNR steps.
template <int R, int UNR, int Q, int EU>
__device__ __forceinline__ void fma_batch(float (&acc)[R], const u32x4 (&v)[UNR][R], const int (&ev)[EU][R],
                                          const f32x4 *xs, const float *gsum, int s0, int steps, int lane) {
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int st = s0 + u;
    if (Q == 2 && st < steps) {
      f32x4 x[8];
#pragma unroll
      for (int h = 0; h < 8; ++h) x[h] = xs[(st * 8 + h) * 64 + lane];
      const float off = 8.0f * gsum[st * 64 + lane];
#pragma unroll
      for (int r = 0; r < R; ++r)
        acc[r] = fmaf(q4_dot(v[u][r], x) - off, __builtin_amdgcn_ldexpf(1.0f, ev[EU == UNR ? u : 0][r]), acc[r]);
    } else if (Q == 1 && st < steps) {
      f32x4 x[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) x[h] = xs[(st * 4 + h) * 64 + lane];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const u32x4 w = v[u][r];
        float a = acc[r];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          a = fmaf(i8f(w[h], 0), x[h][0], a);
          a = fmaf(i8f(w[h], 1), x[h][1], a);
          a = fmaf(i8f(w[h], 2), x[h][2], a);
          a = fmaf(i8f(w[h], 3), x[h][3], a);
        }
        acc[r] = a;
      }
    } else if (!Q && st < steps) {
      const f32x4 xa = xs[(st * 2) * 64 + lane];
      const f32x4 xb = xs[(st * 2 + 1) * 64 + lane];
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

// Epilogue inputs of one item that do not depend on the dot product (bias,
// RoPE angle, the residual value), loaded when the item's first weights are
// issued so that the epilogue itself waits on nothing.
struct ItemPre {
  float a, b, c, e;
  float mw[8], my[8];  // EPI_MOE_ADD: routed weights and outputs of the item's row
};

template <int EPI>
__device__ __forceinline__ ItemPre item_prefetch(const GemvArgs &g, int out_row, int r0, int r1) {
  // loads through pointer selects (a missing bias reads the zero page): a
  // branch around a load would make the merge wait for it
  const float *zf = reinterpret_cast<const float *>(gv_zero);
  ItemPre p{};
  if (EPI == EPI_MOE_ADD) {
    p.a = g.C[r0];
    p.b = *g.moe_gate;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int jj = min(j, g.moe_k - 1);
      p.mw[j] = g.moe_w[jj];
      p.my[j] = g.moe_y[(int64_t)jj * g.N + r0];
    }
  } else if (EPI == EPI_STORE) {
    p.a = *(g.bias ? g.bias + r0 : zf);
  } else if (EPI == EPI_ADD) {
    p.a = g.C[r0];
  } else if (EPI == EPI_QKV) {
    const QkvEpi &q = g.qkv;
    const int half = q.d / 2, i = r0 % q.d;
    p.c = *(q.bias ? q.bias + r0 : zf);
    p.e = *(q.bias ? q.bias + r1 : zf);
    const int pos = q.row_pos ? q.row_pos[0] : q.pos_arg;
    const float2 t = q.cs[(int64_t)pos * half + i];  // unused for v rows
    p.a = t.x;
    p.b = t.y;
  }
  return p;
}

// Rows of item `it` (a valid item), their weight pointers (lane offset
// included) and the item's epilogue inputs.
template <int EPI, int NR, int Q>
__device__ __forceinline__ void item_ptrs(const GemvArgs &g, const char *W, int it, int lane, int out_row,
                                          int (&rows)[NR], const char *(&wp)[NR], ItemPre &pre) {
  int r0, r1;
  item_rows<EPI>(g, it, r0, r1);
  rows[0] = r0;
  rows[NR - 1] = r1;
#pragma unroll
  for (int r = 0; r < NR; ++r) wp[r] = W + (int64_t)rows[r] * gv_row_bytes<Q>(g.K) + lane * 16;
  pre = item_prefetch<EPI>(g, out_row, r0, r1);
}

// Epilogue of one item (lane 0 writes).
// AT: the SwiGLU output goes out with a relaxed device-scope store (read
// inside the same launch by the down projection's blocks).
template <int EPI, bool AT = false>
__device__ __forceinline__ void item_epilogue(const GemvArgs &g, int out_row, int r0, int r1, float v0, float v1,
                                              const ItemPre &pre) {
  if (EPI == EPI_STORE) {
    g.C[(int64_t)out_row * g.ldc + r0] = v0 + pre.a;
  } else if (EPI == EPI_ADD) {
    g.C[r0] = pre.a + v0;
  } else if (EPI == EPI_MOE_ADD) {
    // the combine's order: routed slots in router order, then the shared expert
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < g.moe_k) acc += pre.mw[j] * pre.my[j];
    acc += pre.b * v0;
    g.C[r0] = pre.a + acc;
  } else if (EPI == EPI_SWIGLU) {
    if (AT)
      __hip_atomic_store(g.C + (int64_t)out_row * g.ldc + r0, silu_f(v0) * v1, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    else
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
    const float u0 = v0 + pre.c, u1 = v1 + pre.e;
    const int pos = q.row_pos ? q.row_pos[0] : q.pos_arg;
    const int seq = q.row_seq ? q.row_seq[0] : q.seq_arg;
    int prow;
    const int64_t base = kv_loc(q.pt, q.mp, q.P, q.seq_stride, seq, pos, prow) + q.layer_off;
    if (hh < q.Hq + q.Hkv) {
      const float a0 = u0 * pre.a - u1 * pre.b, a1 = u0 * pre.b + u1 * pre.a;
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
        uint16_t *dst = q.kcache + base + ((int64_t)(hh - q.Hq) * q.S + prow) * d;
        dst[i] = (uint16_t)f32_to_bf16_bits(a0);
        dst[i + half] = (uint16_t)f32_to_bf16_bits(a1);
      }
    } else {
      uint16_t *vt = q.vcache + base + (int64_t)(hh - q.Hq - q.Hkv) * d * q.S;
      vt[(int64_t)i * q.S + prow] = (uint16_t)f32_to_bf16_bits(u0);
      vt[(int64_t)(i + half) * q.S + prow] = (uint16_t)f32_to_bf16_bits(u1);
    }
  }
}

// In-kernel routing (batch-1 MoE decode): one block publishes the route for
// the launches that follow.  Wave 0 writes the top-k ids and their weights;
// the block's threads take the shared-gate dot product w_sg . b from the
// normed activation in LDS (slot i of the layout holds elements k0 .. k0 + 3).
template <int Q, int WV>
__device__ __forceinline__ void publish_route(const GemvArgs &g, const f32x4 *xs, int steps, float *sred) {
  constexpr int EPL = gv_epl<Q>(), HPL = EPL / 4;
  float dot = 0.f;
  if (g.route_w_sg) {
    for (int i = threadIdx.x; i < steps * 64 * HPL; i += WV * WAVE) {
      const int s = i / (64 * HPL), h = (i / 64) % HPL, l = i % 64;
      const int k0 = s * 64 * EPL + l * EPL + 4 * h;
      if (k0 < g.K) {
        const f32x4 b = xs[i];
#pragma unroll
        for (int u = 0; u < 4; ++u) dot += b[u] * bf16_to_f32(g.route_w_sg[k0 + u]);
      }
    }
  }
  dot = block_sum<WV>(dot, sred);
  if (threadIdx.x >= WAVE) return;
  const int lane = threadIdx.x, k = g.n_slots;
  int isel[8];
  float wsel[8], sel;
  moe_topk(g.route_logits, g.route_E, k, lane, isel, wsel, sel);
  if (lane == 0) {
    for (int j = 0; j < k; ++j) {
      g.route_ids[j] = isel[j];
      g.route_wts[j] = g.route_renorm ? wsel[j] / sel : wsel[j];
      if (g.route_rec) g.route_rec[j] = isel[j];
    }
    *g.route_gate = g.route_w_sg ? 1.0f / (1.0f + expf(-dot)) : 1.0f;
  }
}

// One item per wave, WV (4 or 8) waves per block.  The wave's weight rows are
// streamed in chunks of CH 1 KB steps through two register buffers: the
// first two chunks go out before the activation prologue, and each buffer
// is refilled as soon as it has been consumed, so two chunks are always in
// flight.  Every load is unconditional (ragged steps read a zero page), and
// the activation is loaded ahead of the weights when it fits in registers,
// so the prologue waits only for it.  NCH: the row's chunk count when it is
// 1 or 2 (no refills), else 0 (the refill loop).
// IPW > 1 (4-bit weights, one chunk per item): each wave takes IPW items,
// wave w of block b items (b IPW + j) WV + w, and loads item j + 1 into the
// other register buffer while item j is summed, so the activation prologue
// of a block is paid once for IPW times the weights.
// A launch that runs two projections one after the other (the SwiGLU
// gate/up, then the down projection of its output): ROLE 1 blocks (the
// first) store their outputs with relaxed device-scope stores and count
// their arrival on one of GV_NCNT counters once every store is complete;
// ROLE 2 blocks issue their first weight chunks, wait (bounded spin) until
// the counters' sum reaches their snapshots' sum + nb1, then read the
// activation after their weights (mode 0).  No block
// waits on a later one: the first part's blocks precede the second's in
// the dispatch order.
struct GvSync {
  uint32_t *cnt;
  const uint32_t *base;
  int32_t nb1;
};
constexpr uint32_t GV_SPIN_LIMIT = 1u << 20;
constexpr int GV_AB = 8;               // activation loads in flight per thread
constexpr int GV_SC1 = 16;             // cache policy bits of a load: sc1
constexpr int GV_RSRC_W3 = 0x00020000;  // buffer descriptor word 3 (raw dword access)

// Wave 0 polls the GV_NCNT counters, one a lane, until their sum reaches
// the sum of the snapshots plus nb1 (modulo 2^32).
__device__ __forceinline__ uint32_t gv_lane_sum(uint32_t v) {
#pragma unroll
  for (int o = 1; o < GV_NCNT; o <<= 1) v += (uint32_t)__shfl_xor((int)v, o);
  return __builtin_amdgcn_readfirstlane(v);  // lane 0's: the same for every lane
}

__device__ __forceinline__ void gv_wait(const GvSync &sy) {
  if (threadIdx.x < WAVE) {
    const int l = threadIdx.x;
    const uint32_t target = gv_lane_sum(l < GV_NCNT ? sy.base[l] : 0u) + (uint32_t)sy.nb1;
    for (uint32_t n = 0; n < GV_SPIN_LIMIT; ++n) {
      const uint32_t seen =
          l < GV_NCNT ? __hip_atomic_load(sy.cnt + l * SYNC_STRIDE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
      if ((int32_t)(gv_lane_sum(seen) - target) >= 0) break;
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

template <int EPI, int NCH, int WV, int Q, int IPW, int ROLE>
__device__ __forceinline__ void gemv_body(const GemvArgs &ga, int bx0, int by, const GvSync &sy) {
  constexpr int NR = gv_rows<EPI>(), CH = gv_ch<Q>() / NR, NT = WV * WAVE, PRN = 32 / WV, PRH = PRN / 2;
  constexpr int SE = 64 * gv_epl<Q>();  // elements per 1 KB step
  extern __shared__ f32x4 xs[];  // activation, fp32 in the layout of xs_slot
  __shared__ float sred[WV];
  __shared__ float bv_s[WV];
  __shared__ int bi_s[WV];

  // A second part with its own weights, rows and output (same activation)
  // can follow the grouped slots in one grid: blocks past blocks1 x n_slots
  // run it.  Otherwise blockIdx.y is the slot.
  GemvArgs g = ga;
  int bx = bx0, slot = by;
  if (ga.W2) {
    const int nb1 = ga.blocks1 * ga.n_slots;
    if (bx >= nb1) {
      bx -= nb1;
      g.W = ga.W2;
      g.Wq = ga.W2q;
      g.wscale = ga.w2scale;
      g.wexp = ga.w2exp;
      g.N = ga.N2;
      g.n_items = ga.n_items2;
      g.C = ga.C2;
      g.slot_expert = nullptr;
      g.route_logits = nullptr;
    } else {
      slot = bx / ga.blocks1;
      bx -= slot * ga.blocks1;
    }
  }
  const char *W = Q ? reinterpret_cast<const char *>(g.Wq) : reinterpret_cast<const char *>(g.W);
  const float *xin = g.a_f32;
  int out_row = 0;
  if (g.slot_expert || g.route_logits) {
    int64_t ex;
    if (g.route_logits) {
      int isel[8];
      float wsel[8], sel;
      moe_topk(g.route_logits, g.route_E, slot + 1, threadIdx.x & (WAVE - 1), isel, wsel, sel);
      ex = __builtin_amdgcn_readfirstlane(isel[min(slot, 7)]);
    } else {
      ex = g.slot_expert[slot];
    }
    W += Q == 2 ? ex * g.w_group_stride / 2 : ex * g.w_group_stride * (Q ? 1 : 2);
    if (Q == 1) g.wscale += ex * (g.w_group_stride / g.K);  // the expert's row scales
    if (Q == 2) g.wexp += ex * (g.w_group_stride / 32);     // the expert's group exponents
    if (xin) xin += (int64_t)slot * g.a_slot_stride;
    out_row = slot;
  }
  const int K = g.K;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int steps = (K + SE - 1) / SE, nch = NCH ? NCH : (steps + CH - 1) / CH;
  static_assert(IPW == 1 || (NCH == 1 && Q == 2), "several items per wave: 4-bit weights, one chunk per item");
  const int it = bx * WV * IPW + wave;
  const bool valid = it < g.n_items;
  int rows[NR];
  const char *wp[NR];
  ItemPre pre;
  item_ptrs<EPI, NR, Q>(g, W, valid ? it : g.n_items - 1, lane, out_row, rows, wp, pre);
  // the rows' scales, loaded with the first weights (int8 weights only)
  float wsc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) wsc[r] = Q == 1 ? g.wscale[rows[r]] : 1.0f;
  // 4-bit weights: the rows' group exponents, lane l's at step s in byte 64 s + l
  constexpr int EU = Q == 2 ? CH : 1;
  const int8_t *ep[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) ep[r] = Q == 2 ? g.wexp + (int64_t)rows[r] * (K / 32) + lane : nullptr;

  // activation into registers first when it fits.  Mode 1: x and gamma
  // (RMSNorm); 2: fp32 x; 3: bf16 x; 0: read after the weights are issued.
  const int mode = ROLE == 2 ? 0
                 : g.gamma ? (K <= PRH * 4 * NT ? 1 : 0) : xin ? (K <= PRN * 4 * NT ? 2 : 0) : (K <= PRN * 8 * NT ? 3 : 0);
  // (addresses picked by pointer selects, loads unconditional: a branch
  // around them would make the merge wait for the data)
  u32x4 pr[PRN];
#pragma unroll
  for (int i = 0; i < PRN; ++i) {
    const int k1 = min((int)(threadIdx.x + (i % PRH) * NT) * 4, K - 4);
    const int k2 = min((int)(threadIdx.x + i * NT) * 4, K - 4);
    const int k3 = min((int)(threadIdx.x + i * NT) * 8, K - 8);
    const void *src = mode == 1 ? static_cast<const void *>((i < PRH ? xin : g.gamma) + k1)
                    : mode == 2 ? static_cast<const void *>(xin + k2)
                    : mode == 3 ? static_cast<const void *>(g.a_bf16 + k3)
                                : static_cast<const void *>(gv_zero);
    pr[i] = load16(src);
  }

  // (loads past the row read the zero page: no load sits under a branch)
  u32x4 buf0[CH][NR], buf1[CH][NR];
  int ex0[EU][NR], ex1[EU][NR];
  load_batch<NR, CH, Q>(buf0, wp, 0, K, lane);
  if (Q == 2) load_exps<NR, EU>(ex0, ep, 0, K, lane);
  if (NCH != 1) {
    load_batch<NR, CH, Q>(buf1, wp, CH, K, lane);
    if (Q == 2) load_exps<NR, EU>(ex1, ep, CH, K, lane);
  }
  if constexpr (ROLE == 2) gv_wait(sy);

  // activation -> LDS (fp32, with the RMSNorm when gamma is set)
  auto put4 = [&](int k, f32x4 v) { xs[xs_slot_t<Q>(k)] = v; };
  auto as_f4 = [](u32x4 v) { return __builtin_bit_cast(f32x4, v); };
  if (mode == 1) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < PRH; ++i) {
      const f32x4 v = as_f4(pr[i]);
      if ((int)(threadIdx.x + i * NT) * 4 < K) ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
    ss = block_sum<WV>(ss, sred);
    const float inv = 1.0f / sqrtf(ss / (float)K + g.eps);
#pragma unroll
    for (int i = 0; i < PRH; ++i) {
      const int k = (threadIdx.x + i * NT) * 4;
      const f32x4 v = as_f4(pr[i]), w = as_f4(pr[PRH + i]);
      if (k < K) put4(k, f32x4{v[0] * inv * w[0], v[1] * inv * w[1], v[2] * inv * w[2], v[3] * inv * w[3]});
    }
  } else if (mode == 2) {
#pragma unroll
    for (int i = 0; i < PRN; ++i) {
      const int k = (threadIdx.x + i * NT) * 4;
      if (k < K) put4(k, as_f4(pr[i]));
    }
  } else if (mode == 3) {
#pragma unroll
    for (int i = 0; i < PRN; ++i) {
      const int k = (threadIdx.x + i * NT) * 8;
      const u32x4 w = pr[i];
      if (k < K) {
        put4(k, f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])});
        put4(k + 4, f32x4{bf16_lo(w[2]), bf16_hi(w[2]), bf16_lo(w[3]), bf16_hi(w[3])});
      }
    }
  } else if (g.gamma) {
    float ss = 0.f;
    for (int k = threadIdx.x * 4; k < K; k += NT * 4) {
      const f32x4 v = loadf4(xin + k);
      ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
    ss = block_sum<WV>(ss, sred);
    const float inv = 1.0f / sqrtf(ss / (float)K + g.eps);
    for (int k = threadIdx.x * 4; k < K; k += NT * 4) {
      const f32x4 v = loadf4(xin + k), w = loadf4(g.gamma + k);
      put4(k, f32x4{v[0] * inv * w[0], v[1] * inv * w[1], v[2] * inv * w[2], v[3] * inv * w[3]});
    }
  } else if (ROLE == 2) {
    // the first part's outputs of this launch, read at device scope (the
    // sc1 policy of a device-scope atomic load, 16 bytes a lane; reads past
    // K return zero), GV_AB loads in flight per thread
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(xin), 0, K * 4, GV_RSRC_W3);
    for (int k0 = 0; k0 < K; k0 += GV_AB * NT * 4) {
      u32x4 v[GV_AB];
#pragma unroll
      for (int i = 0; i < GV_AB; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (k0 + (threadIdx.x + i * NT) * 4) * 4, 0, GV_SC1);
#pragma unroll
      for (int i = 0; i < GV_AB; ++i) {
        const int k = k0 + (threadIdx.x + i * NT) * 4;
        if (k < K) put4(k, as_f4(v[i]));
      }
    }
  } else if (xin) {
    for (int k = threadIdx.x * 4; k < K; k += NT * 4) put4(k, loadf4(xin + k));
  } else {
    for (int k = threadIdx.x * 8; k < K; k += NT * 8) {
      const u32x4 w = load16(g.a_bf16 + k);
      put4(k, f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])});
      put4(k + 4, f32x4{bf16_lo(w[2]), bf16_hi(w[2]), bf16_lo(w[3]), bf16_hi(w[3])});
    }
  }
  // zero padding up to whole steps
  for (int k = K + threadIdx.x * 4; k < steps * SE; k += NT * 4) put4(k, f32x4{0.f, 0.f, 0.f, 0.f});
  __syncthreads();
  // 4-bit weights: each lane's group sum of the activation, for the code offset
  float *gsum = reinterpret_cast<float *>(xs + (int64_t)steps * SE / 4);
  if (Q == 2) {
    for (int i = threadIdx.x; i < steps * 64; i += NT) {
      const int s = i >> 6, l = i & 63;
      float t = 0.f;
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const f32x4 v = xs[(s * 8 + h) * 64 + l];
        t += (v[0] + v[1]) + (v[2] + v[3]);
      }
      gsum[i] = t;
    }
    __syncthreads();
  }

  if constexpr (IPW > 1) {
    // item j from one buffer while item j + 1 streams into the other
    int rows_n[NR];
    const char *wp_n[NR];
    const int8_t *ep_n[NR];
    ItemPre pre_n;
    float bvw = -INFINITY;
    int biw = 0x7fffffff;
    auto one = [&](u32x4 (&cur)[CH][NR], int (&cex)[EU][NR], u32x4 (&nxt)[CH][NR], int (&nex)[EU][NR], int j) {
      const int itj = it + j * WV;
      if (j + 1 < IPW) {
        const int itn = min(itj + WV, g.n_items - 1);
        item_ptrs<EPI, NR, Q>(g, W, itn, lane, out_row, rows_n, wp_n, pre_n);
#pragma unroll
        for (int r = 0; r < NR; ++r) ep_n[r] = g.wexp + (int64_t)rows_n[r] * (K / 32) + lane;
        load_batch<NR, CH, Q>(nxt, wp_n, 0, K, lane);
        load_exps<NR, EU>(nex, ep_n, 0, K, lane);
      }
      float a[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) a[r] = 0.f;
      fma_batch<NR, CH, Q, EU>(a, cur, cex, xs, gsum, 0, steps, lane);
#pragma unroll
      for (int r = 0; r < NR; ++r) a[r] = wave_sum(a[r]);
      const bool vj = itj < g.n_items;
      if (vj && lane == 0) item_epilogue<EPI>(g, out_row, rows[0], rows[NR - 1], a[0], a[NR - 1], pre);
      if (EPI == EPI_LOGITS && vj && better(a[0], rows[0], bvw, biw)) {
        bvw = a[0];
        biw = rows[0];
      }
      if (j + 1 < IPW) {
#pragma unroll
        for (int r = 0; r < NR; ++r) rows[r] = rows_n[r];
        pre = pre_n;
      }
    };
#pragma unroll
    for (int j = 0; j < IPW; j += 2) {
      one(buf0, ex0, buf1, ex1, j);
      if (j + 1 < IPW) one(buf1, ex1, buf0, ex0, j + 1);
    }
    if (EPI == EPI_LOGITS) {
      if (lane == 0) {
        bv_s[wave] = bvw;
        bi_s[wave] = biw;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        float bv = bv_s[0];
        int bi = bi_s[0];
        for (int w = 1; w < WV; ++w)
          if (better(bv_s[w], bi_s[w], bv, bi)) {
            bv = bv_s[w];
            bi = bi_s[w];
          }
        g.part_val[bx0] = bv;
        g.part_idx[bx0] = bi;
      }
    }
    return;
  }

  float acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.f;
  int c = 0;
  if (NCH == 0) {
    for (; c + 2 < nch; c += 2) {
      fma_batch<NR, CH, Q, EU>(acc, buf0, ex0, xs, gsum, c * CH, steps, lane);
      load_batch<NR, CH, Q>(buf0, wp, (c + 2) * CH, K, lane);
      if (Q == 2) load_exps<NR, EU>(ex0, ep, (c + 2) * CH, K, lane);
      fma_batch<NR, CH, Q, EU>(acc, buf1, ex1, xs, gsum, (c + 1) * CH, steps, lane);
      load_batch<NR, CH, Q>(buf1, wp, (c + 3) * CH, K, lane);
      if (Q == 2) load_exps<NR, EU>(ex1, ep, (c + 3) * CH, K, lane);
    }
  }
  fma_batch<NR, CH, Q, EU>(acc, buf0, ex0, xs, gsum, c * CH, steps, lane);
  if (NCH != 1) fma_batch<NR, CH, Q, EU>(acc, buf1, ex1, xs, gsum, (c + 1) * CH, steps, lane);
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = wave_sum(acc[r]) * wsc[r];
  if (valid && lane == 0) item_epilogue<EPI, ROLE == 1>(g, out_row, rows[0], rows[NR - 1], acc[0], acc[NR - 1], pre);

  if (g.route_logits && bx == 0 && slot == 0) publish_route<Q, WV>(g, xs, steps, sred);

  if (EPI == EPI_LOGITS) {
    // this block's best (value, index), for the argmax finalize pass
    if (lane == 0) {
      bv_s[wave] = valid ? acc[0] : -INFINITY;
      bi_s[wave] = valid ? rows[0] : 0x7fffffff;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float bv = bv_s[0];
      int bi = bi_s[0];
      for (int w = 1; w < WV; ++w)
        if (better(bv_s[w], bi_s[w], bv, bi)) {
          bv = bv_s[w];
          bi = bi_s[w];
        }
      g.part_val[bx0] = bv;
      g.part_idx[bx0] = bi;
    }
  }
  if constexpr (ROLE == 1) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(sy.cnt + (bx0 % GV_NCNT) * SYNC_STRIDE, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int EPI, int NCH, int WV, int Q, int IPW>
__global__ __launch_bounds__(WV * WAVE) void gemv_kernel(GemvArgs ga) {
  gemv_body<EPI, NCH, WV, Q, IPW, 0>(ga, blockIdx.x, blockIdx.y, GvSync{});
}

// The SwiGLU gate/up projection and the down projection of its output in
// one launch: blocks [0, nb1) the first, the rest the second (GvSync).
template <int NCH1, int NCH2, int WV>
__global__ __launch_bounds__(WV * WAVE) void gemv_ffn_kernel(GemvArgs gu, GemvArgs dn, GvSync sy) {
  if ((int)blockIdx.x < sy.nb1) gemv_body<EPI_SWIGLU, NCH1, WV, 0, 1, 1>(gu, blockIdx.x, 0, sy);
  else gemv_body<EPI_ADD, NCH2, WV, 0, 1, 2>(dn, blockIdx.x - sy.nb1, 0, sy);
}

template <int WV, int C1>
void launch_ffn_c2(int c2, dim3 grid, size_t lds, hipStream_t st, const GemvArgs &gu, const GemvArgs &dn,
                   const GvSync &sy) {
  if (c2 == 1) hipLaunchKernelGGL((gemv_ffn_kernel<C1, 1, WV>), grid, dim3(WV * WAVE), lds, st, gu, dn, sy);
  else if (c2 == 2) hipLaunchKernelGGL((gemv_ffn_kernel<C1, 2, WV>), grid, dim3(WV * WAVE), lds, st, gu, dn, sy);
  else hipLaunchKernelGGL((gemv_ffn_kernel<C1, 0, WV>), grid, dim3(WV * WAVE), lds, st, gu, dn, sy);
}

template <int WV>
void launch_ffn_w(int c1, int c2, dim3 grid, size_t lds, hipStream_t st, const GemvArgs &gu, const GemvArgs &dn,
                  const GvSync &sy) {
  if (c1 == 1) launch_ffn_c2<WV, 1>(c2, grid, lds, st, gu, dn, sy);
  else if (c1 == 2) launch_ffn_c2<WV, 2>(c2, grid, lds, st, gu, dn, sy);
  else launch_ffn_c2<WV, 0>(c2, grid, lds, st, gu, dn, sy);
}

int device_cus();

// Items per wave of a launch: 4-bit weights whose rows fit one chunk and
// plain (not grouped) launches take GV_IPW items per wave.
constexpr int GV_IPW = 4;
template <int EPI, int Q>
int gv_ipw(const GemvArgs &g) {
  constexpr int CH = gv_ch<Q>() / gv_rows<EPI>(), SE = 64 * gv_epl<Q>();
  const int nch = ((g.K + SE - 1) / SE + CH - 1) / CH;
  if (Q != 2 || nch != 1 || g.slot_expert || g.route_logits || g.W2) return 1;
  // only while the grid keeps at least two 8-wave blocks per compute unit
  return g.n_items >= 8 * GV_IPW * 2 * device_cus() ? GV_IPW : 1;
}

template <int EPI, int WV, int Q>
void launch_w(const GemvArgs &g, int nch, int ipw, size_t lds, hipStream_t st) {
  const int per_block = WV * ipw;
  const bool grouped = g.slot_expert || g.route_logits;
  dim3 grid((g.n_items + per_block - 1) / per_block, grouped ? g.n_slots : 1), block(WV * WAVE);
  if (g.W2) grid = dim3(g.blocks1 * g.n_slots + (g.n_items2 + WV - 1) / WV, 1);
  if (ipw > 1) {
    if constexpr (Q == 2) hipLaunchKernelGGL((gemv_kernel<EPI, 1, WV, Q, GV_IPW>), grid, block, lds, st, g);
  } else if (nch == 1) {
    hipLaunchKernelGGL((gemv_kernel<EPI, 1, WV, Q, 1>), grid, block, lds, st, g);
  } else if (nch == 2) {
    hipLaunchKernelGGL((gemv_kernel<EPI, 2, WV, Q, 1>), grid, block, lds, st, g);
  } else {
    hipLaunchKernelGGL((gemv_kernel<EPI, 0, WV, Q, 1>), grid, block, lds, st, g);
  }
}

template <int EPI, int Q>
void launch_eq(const GemvArgs &g, int wv, int ipw, size_t lds, hipStream_t st) {
  constexpr int CH = gv_ch<Q>() / gv_rows<EPI>(), SE = 64 * gv_epl<Q>();
  const int nch = ((g.K + SE - 1) / SE + CH - 1) / CH;
  if (wv == 4) launch_w<EPI, 4, Q>(g, nch, ipw, lds, st);
  else launch_w<EPI, 8, Q>(g, nch, ipw, lds, st);
}

template <int EPI>
int ipw_of(const GemvArgs &g) {
  return g.qbits == 4 ? gv_ipw<EPI, 2>(g) : 1;
}

template <int EPI>
void launch_e(const GemvArgs &g, int wv, size_t lds, hipStream_t st) {
  if (g.qbits == 4) launch_eq<EPI, 2>(g, wv, ipw_of<EPI>(g), lds, st);
  else if (g.qbits == 8) launch_eq<EPI, 1>(g, wv, 1, lds, st);
  else launch_eq<EPI, 0>(g, wv, 1, lds, st);
}

int epi_ipw(const GemvArgs &g, int epi) {
  switch (epi) {
    case EPI_STORE: return ipw_of<EPI_STORE>(g);
    case EPI_ADD: return ipw_of<EPI_ADD>(g);
    case EPI_SWIGLU: return ipw_of<EPI_SWIGLU>(g);
    case EPI_QKV: return ipw_of<EPI_QKV>(g);
    case EPI_MOE_ADD: return ipw_of<EPI_MOE_ADD>(g);
    default: return ipw_of<EPI_LOGITS>(g);
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

// Waves per block: 8, unless 4-wave blocks spread the items more evenly over
// the compute units (fewer waves on the busiest one).
int gemv_waves(int n_items) {
  const int cus = device_cus();
  auto busiest = [&](int wv) { return (((n_items + wv - 1) / wv + cus - 1) / cus) * wv; };
  return busiest(4) < busiest(8) ? 4 : 8;
}

int gemv_blocks(int n_items) {
  const int wv = gemv_waves(n_items);
  return (n_items + wv - 1) / wv;
}

// Worth it once the gate/up part fills the chip at least twice over: the
// down blocks' first weights then stream under its last blocks (8B-class
// decode, 1792 + 512 blocks: 330 -> 336 tok/s).  A part that fits in one
// wave of blocks gains nothing to hide the arrival wait under (135M-class,
// 192 + 72 blocks: 1326 -> 1299 tok/s).
bool gemv_ffn_fits(const GemvArgs &gu, const GemvArgs &dn) {
  return gu.W && dn.W && !gu.qbits && !dn.qbits && !gu.Wq && !dn.Wq && !gu.W2 && !dn.W2 && !gu.slot_expert &&
         !dn.slot_expert && !gu.route_logits && !dn.route_logits && gu.C && dn.a_f32 == gu.C && !dn.gamma &&
         dn.K == gu.N && gu.n_items == gu.N && dn.C && gemv_blocks(gu.n_items) >= 2 * device_cus();
}

hipError_t launch_gemv_ffn(const GemvArgs &gu, const GemvArgs &dn, uint32_t *cnt, const uint32_t *base,
                           hipStream_t st) {
  if (!gemv_ffn_fits(gu, dn) || !cnt || !base) return hipErrorInvalidValue;
  // the gate/up part's block shape (its RMSNorm sums over the block's waves)
  const int wv = gemv_waves(gu.n_items);
  const GvSync sy{cnt, base, (gu.n_items + wv - 1) / wv};
  const dim3 grid(sy.nb1 + (dn.n_items + wv - 1) / wv);
  const size_t lds = std::max(gemv_lds(gu.K, 0), gemv_lds(dn.K, 0));
  // chunk counts of each part's rows (1 or 2: no refills; else the refill loop)
  auto nch = [](const GemvArgs &g, int nr) {
    const int ch = gv_ch<0>() / nr, steps = (g.K + 511) / 512, n = (steps + ch - 1) / ch;
    return n <= 2 ? n : 0;
  };
  const int c1 = nch(gu, 2), c2 = nch(dn, 1);
  if (wv == 4) launch_ffn_w<4>(c1, c2, grid, lds, st, gu, dn, sy);
  else launch_ffn_w<8>(c1, c2, grid, lds, st, gu, dn, sy);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvArgs &g0, int epi, hipStream_t st, int *blocks) {
  GemvArgs g = g0;
  const int ipw = epi_ipw(g, epi);
  int wv = gemv_waves((g.n_items + ipw - 1) / ipw);
  if (g.W2) {
    // second part: SwiGLU after grouped slots only, 8-wave blocks for both parts
    if (epi != EPI_SWIGLU || !(g.slot_expert || g.route_logits) || g.n_items2 < 1 || !g.C2) return hipErrorInvalidValue;
    wv = 8;
    g.blocks1 = (g.n_items + wv - 1) / wv;
  }
  if (blocks) *blocks = (g.n_items + wv * ipw - 1) / (wv * ipw);
  // quantised weights: codes in 16-byte lane loads, and a quantised second part
  if (g.qbits != 0 && g.qbits != 8 && g.qbits != 4) return hipErrorInvalidValue;
  // in-kernel routing: a grouped launch of k <= 8 slots over E <= 256 logits
  if (g.route_logits && (g.slot_expert || g.n_slots < 1 || g.n_slots > 8 || g.route_E < g.n_slots ||
                         g.route_E > 256 || !g.route_ids || !g.route_wts || !g.route_gate))
    return hipErrorInvalidValue;
  if ((g.qbits != 0) != (g.Wq != nullptr)) return hipErrorInvalidValue;
  if (g.qbits == 8 && (!g.wscale || g.K % 16 || (g.W2 && (!g.W2q || !g.w2scale)) ||
                       ((g.slot_expert || g.route_logits) && g.w_group_stride % g.K)))
    return hipErrorInvalidValue;
  if (g.qbits == 4 && (!g.wexp || g.K % 32 || (g.W2 && (!g.W2q || !g.w2exp)) ||
                       ((g.slot_expert || g.route_logits) && g.w_group_stride % g.K)))
    return hipErrorInvalidValue;
  const size_t lds = gemv_lds(g.K, g.qbits);
  switch (epi) {
    case EPI_STORE: launch_e<EPI_STORE>(g, wv, lds, st); break;
    case EPI_ADD: launch_e<EPI_ADD>(g, wv, lds, st); break;
    case EPI_SWIGLU: launch_e<EPI_SWIGLU>(g, wv, lds, st); break;
    case EPI_QKV: launch_e<EPI_QKV>(g, wv, lds, st); break;
    case EPI_MOE_ADD:
      if (!g.moe_y || !g.moe_w || !g.moe_gate || g.moe_k < 1 || g.moe_k > 8 || g.slot_expert || g.route_logits)
        return hipErrorInvalidValue;
      launch_e<EPI_MOE_ADD>(g, wv, lds, st);
      break;
    default: launch_e<EPI_LOGITS>(g, wv, lds, st); break;
  }
  return hipGetLastError();
}
