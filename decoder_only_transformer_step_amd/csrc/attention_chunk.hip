// Causal GQA attention for a prefill chunk (one sequence, rows at
// consecutive positions): for query head h at position p, kv head
// g = floor(h Hkv / Hq), s_t = q . k_t / sqrt(d) for t <= p, softmax,
// o = sum_t w_t v_t (engine.zig Engine.forward / Engine.prefill;
// pipeline.rs Pipeline::new: scale 1/sqrt(head_dim)).
//
// gfx950 design (flash attention over the bf16 cache, 32x32x16 MFMA):
//  * A block = 4 waves = 128 query columns of one kv head: 128 / G rows x
//    the G heads that share the head.  Each wave owns 32 columns, with q^T
//    (split bf16) in registers as the B operand.
//  * The block walks 32-key tiles of its key range; each tile (K rows and
//    the V^T columns, 16 KB) is loaded once with coalesced loads into a
//    padded LDS stage and used by all 4 waves (128 columns).  Two stages:
//    the next tile's loads are in flight while the current one is used.
//  * Per tile a wave computes S^T = K Q^T (d/16 MFMAs x 2 for the q lo
//    plane), an online softmax per column in fp32 (exp2, folded scale,
//    causal mask), and O^T += V^T P^T (d/32 output tiles x 2 k groups x 2
//    for the P lo plane).  The PV k index maps to keys the way the QK
//    product leaves them in the lanes, so P needs no shuffle.
//  * Long key ranges split over blocks; each block writes (m, l, O) per
//    column and attn_chunk_merge combines the splits in order.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace {

constexpr int AC_WAVES = 4;
constexpr int AC_COLS = 32 * AC_WAVES;  // query columns per block
constexpr float AC_NEG = -1.0e30f;
constexpr int AC_MAX_TASKS = 1024;      // blocks x splits whose partials fit the buffers

template <int D>
struct AcLay {
  static constexpr int KS = D + 8;   // K tile row stride in elements (16 bytes of padding)
  static constexpr int VS = 32 + 8;  // V^T tile row stride in elements (16 bytes of padding)
  static constexpr int K_ELEMS = 32 * KS;
  static constexpr int STAGE = K_ELEMS + D * VS;
  static constexpr int KP = 32 * D / 8 / 256;  // 16-byte K pieces per thread
  static constexpr int VP = D * 4 / 256;       // 16-byte V^T pieces per thread
};

__device__ __forceinline__ void ac_store_out(const AttnArgs &a, int64_t i, float v) {
  uint32_t hi, lo;
  split_bf16(v, hi, lo);
  a.out[i] = (uint16_t)hi;
  a.out[a.out_lo + i] = (uint16_t)lo;
}

template <int D, bool PG>
__global__ __launch_bounds__(256, 2) void attn_chunk_kernel(AttnArgs a, int rpb) {
  using L = AcLay<D>;
  constexpr int NJ = D / 16, NDT = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * L::STAGE];

  const int gi = blockIdx.x / a.n_splits, split = blockIdx.x - gi * a.n_splits;
  const int g = gi % a.Hkv, rb = gi / a.Hkv;
  const int row_lo = rb * rpb, row_hi = min(a.rows, row_lo + rpb);
  const int keys = a.pos0 + row_hi;  // last position of the block + 1
  const int kstart = attn_key_start(a.window, a.pos0 + row_lo);
  const int nact = (keys - kstart + a.kc - 1) / a.kc;
  if (split >= nact) return;
  const int k0 = kstart + split * a.kc, k1 = min(k0 + a.kc, keys);

  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE, h = lane >> 5;
  const int G = a.G;
  const int col = 32 * wave + (lane & 31);
  const int row = row_lo + col / G, head = g * G + col % G;
  const bool valid = col < rpb * G && row < row_hi;
  const int pos = valid ? a.pos0 + row : -1;
  const int64_t cbase = (int64_t)a.seq0 * a.seq_stride + a.layer_off;
  const uint16_t *kb = a.kcache + cbase + (int64_t)g * a.S * D;
  const uint16_t *vb = a.vcache + cbase + (int64_t)g * D * a.S;

  // tile loads: thread -> 16-byte pieces of the K rows and the V^T columns
  u32x4 kr[L::KP], vr[L::VP];
  auto load_tile = [&](int t0) {
    // a paged cache: the tile's page (a 32-key tile never straddles one)
    const uint16_t *kt = kb, *vt = vb;
    int tt = t0;
    if (PG) {
      const int64_t pb = (int64_t)a.pt[(int64_t)a.seq0 * a.mp + t0 / a.S] * a.seq_stride + a.layer_off;
      kt = a.kcache + pb + (int64_t)g * a.S * D;
      vt = a.vcache + pb + (int64_t)g * D * a.S;
      tt = t0 % a.S;
    }
#pragma unroll
    for (int i = 0; i < L::KP; ++i) {
      const int p = threadIdx.x + 256 * i, key = p / (D / 8), ch = p % (D / 8);
      kr[i] = load16(kt + (int64_t)(tt + key) * D + ch * 8);
    }
#pragma unroll
    for (int i = 0; i < L::VP; ++i) {
      const int p = threadIdx.x + 256 * i, dim = p >> 2, pc = p & 3;
      vr[i] = load16(vt + (int64_t)dim * a.S + tt + pc * 8);
    }
  };
  auto store_tile = [&](uint16_t *st) {
#pragma unroll
    for (int i = 0; i < L::KP; ++i) {
      const int p = threadIdx.x + 256 * i, key = p / (D / 8), ch = p % (D / 8);
      *reinterpret_cast<u32x4 *>(st + key * L::KS + ch * 8) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < L::VP; ++i) {
      const int p = threadIdx.x + 256 * i, dim = p >> 2, pc = p & 3;
      *reinterpret_cast<u32x4 *>(st + L::K_ELEMS + dim * L::VS + pc * 8) = vr[i];
    }
  };

  const int ntiles = (k1 - k0 + 31) / 32;
  load_tile(k0);

  // q^T as the B operand: lane l holds column l % 32 at d = 16 j + 8 h + e
  // (an invalid column reads row 0 / head 0 and is zeroed)
  u32x4 qh[NJ], ql[NJ];
  const uint16_t *qrow = a.q + (valid ? ((int64_t)row * a.Hq + head) * D : 0) + 8 * h;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    qh[j] = load16(qrow + 16 * j);
    ql[j] = load16(qrow + a.q_lo + 16 * j);
    if (!valid) qh[j] = ql[j] = u32x4{0u, 0u, 0u, 0u};
  }

  store_tile(lds);
  __syncthreads();

  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  float m_run = AC_NEG, l_run = 0.f;

  for (int it = 0; it < ntiles; ++it) {
    const int t0 = k0 + 32 * it;
    const uint16_t *cur = lds + (it & 1) * L::STAGE;
    // the next tile (or the current one again at the end: harmless, in range)
    load_tile(it + 1 < ntiles ? t0 + 32 : t0);

    // S^T[key][col] = sum_d K[key][d] q[col][d]; lane: col l % 32, keys
    // t0 + 8 (i / 4) + 4 h + i % 4
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
    // the tile's K fragments first, so the LDS reads overlap each other
    u32x4 ka[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) ka[j] = *reinterpret_cast<const u32x4 *>(cur + (lane & 31) * L::KS + 16 * j + 8 * h);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      s = mfma32x32x16(as_bf16x8(ka[j]), as_bf16x8(qh[j]), s);
      s = mfma32x32x16(as_bf16x8(ka[j]), as_bf16x8(ql[j]), s);
    }
    // scores in log2 units; the soft-cap (a uniform kernel argument) gets a
    // loop of its own, so the plain loop is selects with no branches
    float p[16], tmax = AC_NEG;
    if (a.softcap > 0.f) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = t0 + 8 * (i >> 2) + 4 * h + (i & 3);
        p[i] = (attn_key_ok(a, key, pos) && key < k1) ? attn_logit2(a, s[i]) : -INFINITY;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = t0 + 8 * (i >> 2) + 4 * h + (i & 3);
        const float v = s[i] * a.scale_log2;
        p[i] = (attn_key_ok(a, key, pos) && key < k1) ? v : -INFINITY;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, p[i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, WAVE));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = exp2f(p[i] - m_new);
      psum += p[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
    // O^T[dim][col] += V^T[dim][key] P^T[key][col]: k group kg maps MFMA k
    // index 8 h + e to key 16 kg + 4 h + e (e < 4) and 16 kg + 8 + 4 h + e - 4,
    // exactly the lane's own p[8 kg .. 8 kg + 7]
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
      u32x4 ph, pl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const u32pair t_ = pack_split2(p[8 * kg + 2 * e], p[8 * kg + 2 * e + 1]);
        ph[e] = t_.hi;
        pl[e] = t_.lo;
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint16_t *vrow = cur + L::K_ELEMS + (32 * dt + (lane & 31)) * L::VS + 16 * kg + 4 * h;
        const u32x2 v0 = *reinterpret_cast<const u32x2 *>(vrow), v1 = *reinterpret_cast<const u32x2 *>(vrow + 8);
        const u32x4 va = {v0[0], v0[1], v1[0], v1[1]};
        acc[dt] = mfma32x32x16(as_bf16x8(va), as_bf16x8(ph), acc[dt]);
        acc[dt] = mfma32x32x16(as_bf16x8(va), as_bf16x8(pl), acc[dt]);
      }
    }
    if (it + 1 < ntiles) store_tile(lds + ((it + 1) & 1) * L::STAGE);
    __syncthreads();
  }

  // lane halves hold partial sums over their own keys (same m and alpha)
  const float l_tot = l_run + __shfl_xor(l_run, 32, WAVE);
  // lane: column l % 32, dims 32 dt + 8 (i / 4) + 4 h + i % 4
  if (nact == 1) {
    if (!valid) return;
    float Mv = m_run, Lv = l_tot;
    const float r = attn_sink_fold(a, head, Mv, Lv);
    const float inv = r / Lv;
    const int64_t ob = ((int64_t)row * a.Hq + head) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) ac_store_out(a, ob + 32 * dt + 8 * (i >> 2) + 4 * h + (i & 3), acc[dt][i] * inv);
    return;
  }
  float *po = a.part_o + ((int64_t)blockIdx.x * AC_COLS + col) * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) po[32 * dt + 8 * (i >> 2) + 4 * h + (i & 3)] = acc[dt][i];
  if (h == 0) {
    a.part_ml[((int64_t)blockIdx.x * AC_COLS + col) * 2 + 0] = m_run;
    a.part_ml[((int64_t)blockIdx.x * AC_COLS + col) * 2 + 1] = l_tot;
  }
}

// One block per (group, column), one thread per dim: the group's splits in
// split order (their (m, l) staged in LDS).
template <int D>
__global__ __launch_bounds__(D) void attn_chunk_merge_kernel(AttnArgs a, int rpb) {
  __shared__ float sm[AC_MAX_TASKS], sl[AC_MAX_TASKS];
  __shared__ float red[D / WAVE];
  const int gi = blockIdx.x / AC_COLS, col = blockIdx.x - gi * AC_COLS;
  const int g = gi % a.Hkv, rb = gi / a.Hkv;
  const int row_lo = rb * rpb, row_hi = min(a.rows, row_lo + rpb);
  const int G = a.G;
  const int row = row_lo + col / G, head = g * G + col % G;
  if (!(col < rpb * G && row < row_hi)) return;
  const int kstart = attn_key_start(a.window, a.pos0 + row_lo);
  const int nact = min((a.pos0 + row_hi - kstart + a.kc - 1) / a.kc, AC_MAX_TASKS);
  if (nact <= 1) return;  // written by attn_chunk_kernel
  const int j = threadIdx.x;
  const int64_t t0 = (int64_t)gi * a.n_splits;
  float mx = AC_NEG;
  for (int s = j; s < nact; s += D) {
    const float m = a.part_ml[((t0 + s) * AC_COLS + col) * 2], l = a.part_ml[((t0 + s) * AC_COLS + col) * 2 + 1];
    sm[s] = m;
    sl[s] = l;
    mx = fmaxf(mx, m);
  }
  mx = wave_max(mx);
  if ((j & (WAVE - 1)) == 0) red[j / WAVE] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < D / WAVE; ++w) M = fmaxf(M, red[w]);
  float Ls = 0.f, o = 0.f;
#pragma unroll 8
  for (int s = 0; s < nact; ++s) {
    const float sc = exp2f(sm[s] - M);
    Ls += sc * sl[s];
    o += sc * a.part_o[((t0 + s) * AC_COLS + col) * D + j];
  }
  const float r = attn_sink_fold(a, head, M, Ls);
  ac_store_out(a, ((int64_t)row * a.Hq + head) * D + j, o * r / Ls);
}

template <int D>
hipError_t launch_d(AttnArgs a, hipStream_t st) {
  const int rpb = AC_COLS / a.G;
  const int rblocks = (a.rows + rpb - 1) / rpb;
  a.n_groups = rblocks * a.Hkv;
  // split the keys so that about one block per compute unit runs, each at
  // least two 32-key tiles (every split writes 64 KB of partials per 128
  // columns, which the merge reads back; with at least four tiles, the MoE
  // prefill's 16 column groups ran 64 blocks: its attention 21.0 us per
  // layer against 16.3 with two, and the 8B chunks are unchanged)
  // with a window, a block's keys span at most its rows, the window and
  // the 32-key alignment of its first split
  const int keys = a.window > 0 ? std::min(a.pos0 + a.rows, a.window + rpb + 31) : a.pos0 + a.rows;
  int ns = std::max(1, 256 / a.n_groups);
  int kc = std::max(64, (int)(((keys + ns - 1) / ns + 31) / 32 * 32));
  ns = (keys + kc - 1) / kc;
  while ((int64_t)a.n_groups * ns > AC_MAX_TASKS && ns > 1) {
    kc *= 2;
    ns = (keys + kc - 1) / kc;
  }
  if ((int64_t)a.n_groups * ns > AC_MAX_TASKS) return hipErrorInvalidValue;
  a.kc = kc;
  a.n_splits = ns;
  if (a.pt) hipLaunchKernelGGL((attn_chunk_kernel<D, true>), dim3(a.n_groups * ns), dim3(256), 0, st, a, rpb);
  else hipLaunchKernelGGL((attn_chunk_kernel<D, false>), dim3(a.n_groups * ns), dim3(256), 0, st, a, rpb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ns == 1) return e;
  hipLaunchKernelGGL(attn_chunk_merge_kernel<D>, dim3(a.n_groups * AC_COLS), dim3(D), 0, st, a, rpb);
  return hipGetLastError();
}

}  // namespace

bool attention_chunk_fits(const AttnArgs &a, int head_dim) {
  // (the block count with one split must fit the partial buffers; larger
  // work lists take the general attention kernel)
  return a.pos_mode == 2 && a.out != nullptr && a.out_f32 == nullptr && (head_dim == 64 || head_dim == 128) &&
         a.G >= 1 && a.G <= AC_COLS && a.S % 32 == 0 &&
         (int64_t)((a.rows + AC_COLS / a.G - 1) / (AC_COLS / a.G)) * a.Hkv <= AC_MAX_TASKS;
}

hipError_t launch_attention_chunk(const AttnArgs &a, int head_dim, hipStream_t st) {
  if (!attention_chunk_fits(a, head_dim)) return hipErrorInvalidValue;
  return head_dim == 128 ? launch_d<128>(a, st) : launch_d<64>(a, st);
}
