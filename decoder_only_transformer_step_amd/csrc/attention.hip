// Causal GQA attention over the bf16 KV cache, for decode (one query row per
// sequence) and chunked prefill (many query rows of one sequence).
//
// Math (engine.zig Engine.forward / attentionDecode; pipeline.rs
// Pipeline::new): for query head h at position p, kv head
// g = floor(h Hkv / Hq), s_t = q . k_t / sqrt(d) for t <= p, w = softmax(s),
// o = sum_t w_t v_t.
//
// gfx950 design (flash-decoding with split KV, one kernel):
//  * A "column group" is up to 16 query columns that share one kv head and
//    one sequence: G heads of one decode row, or 16/G rows x G heads of a
//    prefill chunk.  The kv head's K and V are read once for all of them.
//  * One block (4 wavefronts) takes one column group and one contiguous key
//    range (split); its waves take interleaved 32-key tiles.  Per tile:
//    S^T = K Q^T with 2 d/32 MFMA 16x16x32 (K rows straight from HBM as the
//    A operand, Q^T in registers as B), an online softmax per column in fp32
//    (exp2, with log2(e)/sqrt(d) folded into the scale), and O^T += V^T P^T
//    with d/16 MFMAs.  Q and P enter the MFMAs as split bf16 (hi and lo
//    products), so only the cache itself is bf16-limited.
//  * V is stored transposed in the cache ([dim][position]), so the A operand
//    of the PV product is one 16-byte load per lane (8 consecutive keys of
//    a dim row), and the B operand (P^T) is exactly the lane's own scores:
//    the K rows of the QK product are permuted so that it leaves each lane
//    the scores of the same 8 consecutive keys.  No LDS round trip, no
//    cross-lane shuffles for P.
//  * Variants: a sliding window masks keys at or below pos - W and moves
//    the group's first split to the window's start; a soft-cap maps each
//    scaled score s to c tanh(s / c); a head's sink logit joins the final
//    denominator (attn_sink_fold) and adds nothing to the output.
//  * The 4 waves merge through LDS (log-sum-exp); with one split the block
//    normalises and writes the output.  With several, each block writes its
//    (m, l, O) partial and the splits are combined in split order, so the
//    result does not depend on scheduling: by the group's last block to
//    finish (an arrival counter per group), or by attn_merge.  The partials
//    and the counter use relaxed device-scope accesses (stores and loads
//    that are coherent across the XCDs' L2 caches by themselves), so neither
//    side needs an L2 write-back or invalidate, and no block waits on
//    another.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace {

constexpr float NEG_SENTINEL = -1.0e30f;

struct Col {
  bool valid;
  int row, head, pos;
};

// Position of query row `row` of row group rg, by where the positions live
// (PM = AttnArgs::pos_mode; mode 1 has one row per group, so its lookup
// index is the block-uniform rg and the value comes from the kernel
// arguments, with no memory round trip before the cache reads).
template <int PM>
__device__ __forceinline__ int row_position(const AttnArgs &a, int rg, int row) {
  if (PM == 1) return a.pos_arg[rg];
  if (PM == 2) return a.pos0 + row;
  return a.row_pos[row];
}

template <int PM>
__device__ __forceinline__ int group_seq(const AttnArgs &a, int rg) {
  if (PM == 1) return a.seq_arg[rg];
  if (PM == 2) return a.seq0;
  return a.row_seq[rg * a.rows_per_group];
}

template <int PM>
__device__ __forceinline__ Col column(const AttnArgs &a, int rg, int g, int c) {
  Col k;
  const int G = a.G;
  k.row = rg * a.rows_per_group + c / G;
  k.head = g * G + c % G;
  k.valid = (c < a.rows_per_group * G) && (k.row < a.rows);
  k.pos = k.valid ? row_position<PM>(a, rg, k.row) : -1;
  return k;
}

__device__ __forceinline__ void store_out(const AttnArgs &a, int64_t i, float v) {
  if (a.out_f32) {
    // (read inside the same launch when the output projection is fused)
    if (a.wo) __hip_atomic_store(a.out_f32 + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else a.out_f32[i] = v;
  } else {
    uint32_t hi, lo;
    split_bf16(v, hi, lo);
    a.out[i] = (uint16_t)hi;
    a.out[a.out_lo + i] = (uint16_t)lo;
  }
}

// keys of the group: 0 .. max position of its valid columns
template <int PM>
__device__ __forceinline__ int group_keys(const AttnArgs &a, int rg, int g) {
  if (PM == 1) return a.pos_arg[rg] + 1;
  if (PM == 2) return a.pos0 + min(a.rows - 1, (rg + 1) * a.rows_per_group - 1) + 1;
  int kmax = -1;
  for (int c = 0; c < 16; ++c) kmax = max(kmax, column<0>(a, rg, g, c).pos);
  return kmax + 1;
}

// First key of the group's splits: with a window, the lowest query position
// of the group bounds it (mode 0 groups start at key 0 and rely on masking).
template <int PM>
__device__ __forceinline__ int group_key_start(const AttnArgs &a, int rg) {
  if (PM == 1) return attn_key_start(a.window, a.pos_arg[rg]);
  if (PM == 2) return attn_key_start(a.window, a.pos0 + rg * a.rows_per_group);
  return 0;
}

// Combine one (column, dim j) of a group's split partials in split order.
// Each chunk of MERGE_CHUNK splits is one batch of independent loads ((m, l)
// and the O value per split), folded into running sums rescaled to the
// chunk's new maximum, so a merge of up to MERGE_CHUNK splits is a single
// memory round trip.  AT: the partials are read with relaxed device-scope
// loads (the merge inside attn_kernel; attn_merge reads them after a kernel
// boundary with plain loads).
constexpr int MERGE_CHUNK = 32;

template <bool AT>
__device__ __forceinline__ float part_load(const float *p) {
  if (AT) return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}

template <int D, bool AT>
__device__ __forceinline__ float merge_splits(const AttnArgs &a, int gi, int cc, int j, int nact, int head) {
  const float *ml = a.part_ml + ((int64_t)gi * a.n_splits * 16 + cc) * 2;
  const float *po = a.part_o + ((int64_t)gi * a.n_splits * 16 + cc) * D + j;
  float M = NEG_SENTINEL, L = 0.f, o = 0.f;
  for (int s0 = 0; s0 < nact; s0 += MERGE_CHUNK) {
    float ms[MERGE_CHUNK], ls[MERGE_CHUNK], ov[MERGE_CHUNK];
#pragma unroll
    for (int u = 0; u < MERGE_CHUNK; ++u) {
      const int64_t s = min(s0 + u, nact - 1);
      ms[u] = part_load<AT>(ml + s * 32);
      ls[u] = part_load<AT>(ml + s * 32 + 1);
      ov[u] = part_load<AT>(po + s * 16 * D);
    }
    // splits past nact (clamped duplicates) get weight 0; every loaded
    // value is used unconditionally, so no load is sunk into a branch
#pragma unroll
    for (int u = 0; u < MERGE_CHUNK; ++u) ms[u] = s0 + u < nact ? ms[u] : -INFINITY;
    float cm = M;
#pragma unroll
    for (int u = 0; u < MERGE_CHUNK; ++u) cm = fmaxf(cm, ms[u]);
    const float r = exp2f(M - cm);
    L *= r;
    o *= r;
#pragma unroll
    for (int u = 0; u < MERGE_CHUNK; ++u) {
      const float sc = exp2f(ms[u] - cm);
      L += sc * ls[u];
      o += sc * ov[u];
    }
    M = cm;
  }
  const float r = attn_sink_fold(a, head, M, L);
  return o * r / L;
}

// The merge inside attn_kernel, run by the group's last block (256
// threads, up to two (column, dim) values each, at most ATTN_FUSED_MAX_SPLITS
// splits and 256 (split, column) pairs): one round of relaxed device-scope
// loads brings every split's O values of the thread into registers and the
// (m, l) of every (split, column) into LDS; the columns' maxima, rescale
// factors and denominators are then formed in LDS, and each value is summed
// in split order.  sc and sl alias LDS the block no longer needs.  FM:
// the loads per value (nact <= FM; the dispatch below picks 8, 16 or 32, so
// a merge of a few splits issues a few loads).
template <int D, int PM, int FM>
__device__ __forceinline__ void merge_fused(const AttnArgs &a, int gi, int rg, int g, int nact, int ncols,
                                            float (*sc)[16], float (*sl)[16], float *den) {
  const int t = threadIdx.x;
  const int p0 = t, p1 = t + 256;
  const int c0 = p0 / D, j0 = p0 - c0 * D, c1 = p1 / D, j1 = p1 - c1 * D;
  const bool v0 = c0 < ncols, v1 = c1 < ncols;
  const int64_t base = (int64_t)gi * a.n_splits * 16;
  // (a value past the group's columns reads column 0, dim 0, and is dropped)
  const float *po0 = a.part_o + (base + (v0 ? c0 : 0)) * D + (v0 ? j0 : 0);
  const float *po1 = a.part_o + (base + (v1 ? c1 : 0)) * D + (v1 ? j1 : 0);
  float x0[FM], x1[FM];
#pragma unroll
  for (int u = 0; u < FM; ++u) {
    const int64_t su = min(u, nact - 1);
    x0[u] = part_load<true>(po0 + su * 16 * D);
    x1[u] = part_load<true>(po1 + su * 16 * D);
  }
  const bool ml_own = t < nact * ncols;
  const int ms = ml_own ? t / ncols : 0, mc = ml_own ? t - ms * ncols : 0;
  const float *ml = a.part_ml + (base + ms * 16 + mc) * 2;
  const float mv = part_load<true>(ml), lv = part_load<true>(ml + 1);
  if (ml_own) {
    sc[ms][mc] = mv;
    sl[ms][mc] = lv;
  }
  __syncthreads();
  if (t < ncols) {
    float M = NEG_SENTINEL;
    for (int s = 0; s < nact; ++s) M = fmaxf(M, sc[s][t]);
    float L = 0.f;
    for (int s = 0; s < nact; ++s) {
      const float f = exp2f(sc[s][t] - M);
      sc[s][t] = f;
      L += f * sl[s][t];
    }
    const float r = attn_sink_fold(a, column<PM>(a, rg, g, t).head, M, L);
    den[t] = r / L;
  }
  __syncthreads();
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int u = 0; u < FM; ++u) {
    if (u < nact) {
      o0 += sc[u][v0 ? c0 : 0] * x0[u];
      o1 += sc[u][v1 ? c1 : 0] * x1[u];
    }
  }
  if (v0) {
    const Col col = column<PM>(a, rg, g, c0);
    if (col.valid) store_out(a, ((int64_t)col.row * a.Hq + col.head) * D + j0, o0 * den[c0]);
  }
  if (v1) {
    const Col col = column<PM>(a, rg, g, c1);
    if (col.valid) store_out(a, ((int64_t)col.row * a.Hq + col.head) * D + j1, o1 * den[c1]);
  }
}

// A column group's output is complete: with the output projection fused,
// every thread's stores complete, then one arrival for the group.
__device__ __forceinline__ void publish_group(const AttnArgs &a) {
  if (!a.wo) return;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(a.o_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Fused output projection (batch-1 decode), one block of 4 waves past the
// attention grid: wave w owns rows (4 b + w) ATTN_O_RPW + r of wo.  The
// rows' weights (lane l holds k = 8 l + 512 s, as the batch-1 GEMV) and
// residual values stream into registers while the attention runs; thread 0
// then waits (a bounded spin) until every column group has arrived, the
// block stages o (fp32, relaxed device-scope loads) in LDS in the GEMV's
// layout, and each wave sums its rows with the GEMV's arithmetic order:
// step by step, 8 FMAs per 16-byte weight load, then the wave reduction,
// then x + sum, so the result is the separate launch's, bit for bit.  Every
// block reaches its end: the attention blocks wait on nothing, and they
// precede the projection blocks in the dispatch order.
//
// Measured (8B decode, 136 attention blocks and 256 projection blocks,
// in-kernel clock): the attention publishes its last group at about 12.4
// us; the projection blocks see it 1.4 us later, have o in LDS 1.3 us
// after that and end about 1 us later, against 13 + 8.4 us for the
// attention and projection launches one after the other.  The weights
// wait AO_HOLD_TICKS of the 100 MHz clock (1.5 us) before they go out, so
// that the attention's cache loads, issued first, are not queued behind
// 33.5 MB of them (8B decode 326 -> 329 tok/s against no wait; 3 us was
// slower again).
constexpr int AO_STEPS = ATTN_O_MAX_K / 512;
constexpr uint32_t AO_SPIN_LIMIT = 1u << 20;
constexpr uint64_t AO_HOLD_TICKS = 150;
__device__ u32x4 ao_zero[1];

__device__ __forceinline__ int ao_slot(int k) {  // k: a multiple of 4
  return ((k >> 9) * 2 + ((k >> 2) & 1)) * 64 + ((k & 511) >> 3);
}

template <int D>
__device__ __forceinline__ void o_proj_block(const AttnArgs &a, int b, f32x4 *xs) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int K = a.Hq * D, steps = (K + 511) / 512;
  const int r0 = (b * 4 + wave) * ATTN_O_RPW;
  int row[ATTN_O_RPW];
  u32x4 w[ATTN_O_RPW][AO_STEPS];
  float xr[ATTN_O_RPW];
#pragma unroll
  for (int r = 0; r < ATTN_O_RPW; ++r) row[r] = min(r0 + r, a.o_rows - 1);
  {
    const uint64_t t_go = wall_clock64() + AO_HOLD_TICKS;
    while (wall_clock64() < t_go) __builtin_amdgcn_s_sleep(2);
  }
#pragma unroll
  for (int s = 0; s < AO_STEPS; ++s) {
    const bool ok = s * 512 + lane * 8 < K;
#pragma unroll
    for (int r = 0; r < ATTN_O_RPW; ++r)
      w[r][s] = load16_nt(ok ? static_cast<const void *>(a.wo + (int64_t)row[r] * K + s * 512 + lane * 8)
                             : static_cast<const void *>(ao_zero));
  }
#pragma unroll
  for (int r = 0; r < ATTN_O_RPW; ++r) xr[r] = a.o_x[row[r]];

  if (threadIdx.x == 0) {
    const uint32_t target = *a.o_base + (uint32_t)a.n_groups;
    for (uint32_t n = 0; n < AO_SPIN_LIMIT; ++n) {
      const uint32_t seen = __hip_atomic_load(a.o_done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((int32_t)(seen - target) >= 0) break;
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  // o -> LDS, zero past K (AO_STEPS * 512 elements, 4 per thread and slot)
  const float *zf = reinterpret_cast<const float *>(ao_zero);
  float v[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int k = (u * 256 + threadIdx.x) * 4;
    const float *src = k < K ? a.out_f32 + k : zf;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[u][e] = __hip_atomic_load(const_cast<float *>(src + e), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) xs[ao_slot((u * 256 + threadIdx.x) * 4)] = f32x4{v[u][0], v[u][1], v[u][2], v[u][3]};
  __syncthreads();
  float acc[ATTN_O_RPW];
#pragma unroll
  for (int r = 0; r < ATTN_O_RPW; ++r) acc[r] = 0.f;
#pragma unroll
  for (int s = 0; s < AO_STEPS; ++s) {
    if (s < steps) {
      const f32x4 xa = xs[(s * 2) * 64 + lane], xb = xs[(s * 2 + 1) * 64 + lane];
#pragma unroll
      for (int r = 0; r < ATTN_O_RPW; ++r) {
        const u32x4 q = w[r][s];
        float t = acc[r];
        t = fmaf(bf16_lo(q[0]), xa[0], t);
        t = fmaf(bf16_hi(q[0]), xa[1], t);
        t = fmaf(bf16_lo(q[1]), xa[2], t);
        t = fmaf(bf16_hi(q[1]), xa[3], t);
        t = fmaf(bf16_lo(q[2]), xb[0], t);
        t = fmaf(bf16_hi(q[2]), xb[1], t);
        t = fmaf(bf16_lo(q[3]), xb[2], t);
        t = fmaf(bf16_hi(q[3]), xb[3], t);
        acc[r] = t;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < ATTN_O_RPW; ++r) acc[r] = wave_sum(acc[r]);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < ATTN_O_RPW; ++r)
      if (r0 + r < a.o_rows) a.o_x[row[r]] = xr[r] + acc[r];
  }
}

// NTK: the K rows are loaded non-temporal (a split of at most one tile per
// wave reads each K row once, within one wave: 8B decode 314-319 -> 321-322
// tok/s; the MoE decode's attention, one head per group, 10.56 -> 10.9 us
// per layer, about 0.5% of its step); with several tiles per wave the hint
// cost more than it gave (16 x 32 768-key batch 976 -> 943 tok/s), and V,
// whose 128-byte lines two waves share, stays plain everywhere.
// OF: the output projection is fused (blocks past the attention grid).
template <int D, int PM, bool PG, bool NTK = false, bool OF = false>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  constexpr int NDT = D / 16;
  __shared__ float lo[4][16][D];
  __shared__ float lm[4][16], ll[4][16];
  __shared__ int last_s;
  if constexpr (OF) {
    static_assert(64 * D >= AO_STEPS * 512, "o staging fits in lo");
    if (blockIdx.x >= a.n_groups * a.n_splits) {
      o_proj_block<D>(a, blockIdx.x - a.n_groups * a.n_splits, reinterpret_cast<f32x4 *>(&lo[0][0][0]));
      return;
    }
  }

  const int gi = blockIdx.x / a.n_splits, split = blockIdx.x - gi * a.n_splits;
  const int g = gi % a.Hkv, rg = gi / a.Hkv;
  const int keys = group_keys<PM>(a, rg, g), kstart = group_key_start<PM>(a, rg);
  const int nact = (keys - kstart + a.kc - 1) / a.kc;
  if (split >= nact) return;
  const int k0 = kstart + split * a.kc, k1 = min(k0 + a.kc, keys);

  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int c = lane & 15, quad = lane >> 4;
  const Col col = column<PM>(a, rg, g, c);
  const int seq = group_seq<PM>(a, rg);
  const uint16_t *kb = a.kcache + (int64_t)seq * a.seq_stride + a.layer_off + (int64_t)g * a.S * D;
  const uint16_t *vb = a.vcache + (int64_t)seq * a.seq_stride + a.layer_off + (int64_t)g * D * a.S;

  // K / V tile loads of the 32 keys at t.  K rows go straight into MFMA A
  // operands, permuted so that the QK product leaves lane l the scores of
  // keys 8 (l / 16) + 0..3 (s0) and 8 (l / 16) + 4..7 (s1): MFMA row m of s0
  // is key 8 (m / 4) + m % 4, of s1 key 8 (m / 4) + 4 + m % 4.  The PV
  // product then takes P^T as the lane's own 8 consecutive keys, and V^T as
  // one contiguous 16-byte load per lane (64 bytes of a dim row per quad).
  u32x4 ka[D / 32], kh[D / 32];
  u32x4 va[NDT];
  // a paged cache: the page of the tile at t (a 32-key tile never straddles
  // one); the loop reads the next tile's page one tile ahead, so a tile's
  // cache loads never wait on its page-table entry
  auto page_of = [&](int t) { return PG ? a.pt[(int64_t)seq * a.mp + t / a.S] : 0; };
  auto load_tile = [&](int t, int page) {
    const uint16_t *kt = kb, *vt = vb;
    int tt = t;
    if (PG) {
      const int64_t pb = (int64_t)page * a.seq_stride + a.layer_off;
      kt = a.kcache + pb + (int64_t)g * a.S * D;
      vt = a.vcache + pb + (int64_t)g * D * a.S;
      tt = t % a.S;
    }
    const int kr = 8 * (c >> 2) + (c & 3);
    const uint16_t *k_lo = kt + (int64_t)(tt + kr) * D + quad * 8;
    const uint16_t *k_hi = k_lo + 4 * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      ka[ks] = (NTK ? load16_nt : load16)(k_lo + ks * 32);
      kh[ks] = (NTK ? load16_nt : load16)(k_hi + ks * 32);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) va[dt] = load16(vt + (int64_t)(dt * 16 + c) * a.S + tt + quad * 8);
  };
  // the first tile goes out before q (a wave without a tile of its own
  // reloads the split's first tile, which stays inside the cache rows)
  const int t_first = k0 + 32 * wave;
  const int t_load = t_first < k1 ? t_first : k0;
  load_tile(t_load, page_of(t_load));

  // q of the column (an invalid column reads row 0 / head 0 and is zeroed:
  // unconditional loads keep the wait counts exact)
  u32x4 qf[D / 32], ql[D / 32];
  const uint16_t *qrow = a.q + (col.valid ? ((int64_t)col.row * a.Hq + col.head) * D : 0) + quad * 8;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    qf[ks] = load16(qrow + ks * 32);
    ql[ks] = load16(qrow + a.q_lo + ks * 32);
    if (!col.valid) qf[ks] = ql[ks] = u32x4{0u, 0u, 0u, 0u};
  }

  float m_run = NEG_SENTINEL, l_run = 0.f;
  f32x4 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // (clamped to the split's last key, so the entry load is unconditional)
  int page_next = page_of(min(t_first + 128, k1 - 1));
  for (int t0 = t_first; t0 < k1; t0 += 128) {
    if (t0 != t_first) {
      const int page = page_next;
      page_next = page_of(min(t0 + 128, k1 - 1));
      load_tile(t0, page);
    }
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      s0 = mfma16x16x32(as_bf16x8(ka[ks]), as_bf16x8(qf[ks]), s0);
      s0 = mfma16x16x32(as_bf16x8(ka[ks]), as_bf16x8(ql[ks]), s0);
      s1 = mfma16x16x32(as_bf16x8(kh[ks]), as_bf16x8(qf[ks]), s1);
      s1 = mfma16x16x32(as_bf16x8(kh[ks]), as_bf16x8(ql[ks]), s1);
    }
    // lane holds S[key = t0 + 8 quad + i][col c] in s0, key + 4 in s1
    // (the soft-cap, a uniform kernel argument, has a loop of its own, so
    // the plain loop is selects with no branches)
    float sv[8];
    float tmax = NEG_SENTINEL;
    if (a.softcap > 0.f) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key0 = t0 + quad * 8 + i, key1 = key0 + 4;
        sv[i] = (attn_key_ok(a, key0, col.pos) && key0 < k1) ? attn_logit2(a, s0[i]) : -INFINITY;
        sv[4 + i] = (attn_key_ok(a, key1, col.pos) && key1 < k1) ? attn_logit2(a, s1[i]) : -INFINITY;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key0 = t0 + quad * 8 + i, key1 = key0 + 4;
        const float v0 = s0[i] * a.scale_log2, v1 = s1[i] * a.scale_log2;
        sv[i] = (attn_key_ok(a, key0, col.pos) && key0 < k1) ? v0 : -INFINITY;
        sv[4 + i] = (attn_key_ok(a, key1, col.pos) && key1 < k1) ? v1 : -INFINITY;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, fmaxf(sv[i], sv[4 + i]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, WAVE));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, WAVE));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);
    float p[8], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = exp2f(sv[i] - m_new);
      psum += p[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    u32x4 pb, pl;
    { const u32pair t_ = pack_split2(p[0], p[1]); pb[0] = t_.hi; pl[0] = t_.lo; }
    { const u32pair t_ = pack_split2(p[2], p[3]); pb[1] = t_.hi; pl[1] = t_.lo; }
    { const u32pair t_ = pack_split2(p[4], p[5]); pb[2] = t_.hi; pl[2] = t_.lo; }
    { const u32pair t_ = pack_split2(p[6], p[7]); pb[3] = t_.hi; pl[3] = t_.lo; }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      acc[dt] *= alpha;
      acc[dt] = mfma16x16x32(as_bf16x8(va[dt]), as_bf16x8(pb), acc[dt]);
      acc[dt] = mfma16x16x32(as_bf16x8(va[dt]), as_bf16x8(pl), acc[dt]);
    }
  }
  // acc[dt][i] = O^T[dim = dt*16 + 4 quad + i][col c]; merge the 4 waves
  float l_tot = l_run + __shfl_xor(l_run, 16, WAVE);
  l_tot += __shfl_xor(l_tot, 32, WAVE);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4 *>(&lo[wave][c][dt * 16 + quad * 4]) = acc[dt];
  if (quad == 0) {
    lm[wave][c] = m_run;
    ll[wave][c] = l_tot;
  }
  __syncthreads();
  // thread -> column cc, dims jj + 16 q
  const int cc = threadIdx.x >> 4, jj = threadIdx.x & 15;
  const Col oc = column<PM>(a, rg, g, cc);
  float M = NEG_SENTINEL;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, lm[w][cc]);
  float L = 0.f, o[NDT];
#pragma unroll
  for (int q = 0; q < NDT; ++q) o[q] = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float sc = exp2f(lm[w][cc] - M);
    L += sc * ll[w][cc];
#pragma unroll
    for (int q = 0; q < NDT; ++q) o[q] += sc * lo[w][cc][jj + 16 * q];
  }
  if (nact == 1) {
    if (oc.valid) {
      const float r = attn_sink_fold(a, oc.head, M, L);
      const float inv = r / L;
      const int64_t ob = ((int64_t)oc.row * a.Hq + oc.head) * D;
#pragma unroll
      for (int q = 0; q < NDT; ++q) store_out(a, ob + jj + 16 * q, o[q] * inv);
    }
    if (OF) publish_group(a);
    return;
  }
  // several splits: publish this block's partial
  const int64_t task = blockIdx.x;
  float *po = a.part_o + (task * 16 + cc) * D;
  if (!a.counters) {  // for attn_merge
#pragma unroll
    for (int q = 0; q < NDT; ++q) po[jj + 16 * q] = o[q];
    if (jj == 0) {
      a.part_ml[(task * 16 + cc) * 2 + 0] = M;
      a.part_ml[(task * 16 + cc) * 2 + 1] = L;
    }
    return;
  }
  if (oc.valid) {
#pragma unroll
    for (int q = 0; q < NDT; ++q) __hip_atomic_store(po + jj + 16 * q, o[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (jj == 0) {
      __hip_atomic_store(a.part_ml + (task * 16 + cc) * 2 + 0, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.part_ml + (task * 16 + cc) * 2 + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // every thread's partial stores complete, then one arrival for the block;
  // the group's last block to arrive (counter nact - 1) merges
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    last_s = __hip_atomic_fetch_add(a.counters + gi, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nact - 1;
  __syncthreads();
  if (!last_s) return;
  if (threadIdx.x == 0) __hip_atomic_store(a.counters + gi, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // (the launcher sets counters only when a group has at most 512 values,
  // ATTN_FUSED_MAX_SPLITS splits and 256 (split, column) pairs); the
  // block's own merge is done with lo, which now holds the scale table
  float(*sc)[16] = reinterpret_cast<float(*)[16]>(&lo[0][0][0]);
  float(*sl)[16] = sc + ATTN_FUSED_MAX_SPLITS;
  const int ncols = min(16, a.rows_per_group * a.G);
  static_assert(ATTN_FUSED_MAX_SPLITS == 32, "merge_fused dispatch");
  if (nact <= 8) merge_fused<D, PM, 8>(a, gi, rg, g, nact, ncols, sc, sl, &lm[0][0]);
  else if (nact <= 16) merge_fused<D, PM, 16>(a, gi, rg, g, nact, ncols, sc, sl, &lm[0][0]);
  else merge_fused<D, PM, 32>(a, gi, rg, g, nact, ncols, sc, sl, &lm[0][0]);
  if (OF) publish_group(a);
}

// One block per (group, valid column), one thread per dim: combine the
// group's splits in split order (merge_splits).
template <int D, int PM>
__global__ __launch_bounds__(D) void attn_merge_kernel(AttnArgs a, int ncols) {
  const int gi = blockIdx.x / ncols, cc = blockIdx.x - gi * ncols;
  const int g = gi % a.Hkv, rg = gi / a.Hkv;
  const Col oc = column<PM>(a, rg, g, cc);
  if (!oc.valid) return;
  const int nact = (group_keys<PM>(a, rg, g) - group_key_start<PM>(a, rg) + a.kc - 1) / a.kc;
  if (nact <= 1) return;                       // written directly by attn_kernel
  const int j = threadIdx.x;
  store_out(a, ((int64_t)oc.row * a.Hq + oc.head) * D + j, merge_splits<D, false>(a, gi, cc, j, nact, oc.head));
}

}  // namespace

namespace {

template <int D, int PM>
hipError_t launch_pm(const AttnArgs &a, hipStream_t st) {
  const int nb = a.n_groups * a.n_splits;
  if (PM != 2 && a.wo) {  // batch-1 decode with the output projection
    if (!a.counters || !a.out_f32 || a.rows != 1 || (int64_t)a.Hq * D > ATTN_O_MAX_K) return hipErrorInvalidValue;
    if (a.pt)
      hipLaunchKernelGGL((attn_kernel<D, PM, true, false, PM != 2>), dim3(nb + a.o_blocks), dim3(256), 0, st, a);
    else if (PM == 1 && a.kc <= 128)
      hipLaunchKernelGGL((attn_kernel<D, PM, false, PM == 1, PM != 2>), dim3(nb + a.o_blocks), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((attn_kernel<D, PM, false, false, PM != 2>), dim3(nb + a.o_blocks), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  if (a.wo) return hipErrorInvalidValue;
  if (a.pt) hipLaunchKernelGGL((attn_kernel<D, PM, true>), dim3(nb), dim3(256), 0, st, a);
  else if (PM == 1 && a.kc <= 128)  // decode, one 32-key tile per wave
    hipLaunchKernelGGL((attn_kernel<D, PM, false, PM == 1>), dim3(nb), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((attn_kernel<D, PM, false>), dim3(nb), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_splits == 1 || a.counters) return e;
  const int ncols = std::min(16, a.rows_per_group * a.G);  // valid columns of a group
  hipLaunchKernelGGL((attn_merge_kernel<D, PM>), dim3(a.n_groups * ncols), dim3(D), 0, st, a, ncols);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs &a, hipStream_t st) {
  switch (a.pos_mode) {
    case 1: return launch_pm<D, 1>(a, st);
    case 2: return launch_pm<D, 2>(a, st);
    default: return launch_pm<D, 0>(a, st);
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, int head_dim, hipStream_t st) {
  return head_dim == 128 ? launch_d<128>(a, st) : launch_d<64>(a, st);
}
