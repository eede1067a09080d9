// Shared device helpers for the gfx950 kernels: bf16 packing, MFMA fragment
// types, wave reductions, and the launch-parameter structs the host side
// fills in.  CDNA4 wavefronts are 64 lanes; every kernel here is written for
// that width.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define WAVE 64

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

// ----------------------------------------------------------------- bf16 --

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7fffu + ((b >> 16) & 1u);
  return b >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Split-bf16 activations: v ~ hi + lo with hi = bf16(v), lo = bf16(v - hi),
// about 16 significant bits.  Activations that feed an MFMA are stored as a
// hi plane and a lo plane (same layout, lo at a fixed element offset) and
// multiplied twice against the exact bf16 weights; a single bf16 rounding
// of an activation costs more accuracy than a deep random-weight model can
// absorb within the logits tolerance.
__device__ __forceinline__ void split_bf16(float v, uint32_t &hi, uint32_t &lo) {
  hi = f32_to_bf16_bits(v);
  lo = f32_to_bf16_bits(v - __uint_as_float(hi << 16));
}
struct u32pair {
  uint32_t hi, lo;
};
// two values -> packed hi pair and packed lo pair
__device__ __forceinline__ u32pair pack_split2(float a, float b) {
  uint32_t ha, la, hb, lb;
  split_bf16(a, ha, la);
  split_bf16(b, hb, lb);
  return u32pair{ha | (hb << 16), la | (lb << 16)};
}

__device__ __forceinline__ u32x4 load16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
// A 16-byte load marked non-temporal (streamed once: weights of a batch-1
// projection).  On this part a 352 MB sweep read this way ran at 6.0-6.2
// TB/s against 5.1-5.2 TB/s with plain loads.
__device__ __forceinline__ u32x4 load16_nt(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x2 load8(const void *p) {
  return *reinterpret_cast<const u32x2 *>(p);
}
__device__ __forceinline__ f32x4 loadf4(const float *p) {
  return *reinterpret_cast<const f32x4 *>(p);
}

// D = A * B + C for a 16x16 tile with K = 32 (bf16 in, fp32 accumulate).
// Lane l supplies A[m = l % 16][k = 8 (l / 16) + j] and B[k = 8 (l / 16) + j][n = l % 16]
// for j < 8, and receives D[m = 4 (l / 16) + i][n = l % 16] for i < 4.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D[32][32] += A[32][16] B[16][32] (v_mfma_f32_32x32x16_bf16; on gfx950 it
// runs at twice the flop rate of the 16x16x32 form).  Lane l holds
// A[m = l % 32][k = 8 (l / 32) + e], B[k = 8 (l / 32) + e][n = l % 32], and
// D[m = 8 (i / 4) + 4 (l / 32) + i % 4][n = l % 32] in register i.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------- wave reductions --

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

// Block-wide sum for blockDim.x = 64 * nwaves; every thread gets the result.
template <int NWAVES>
__device__ __forceinline__ float block_sum(float v, float *lds) {
  v = wave_sum(v);
  const int w = threadIdx.x / WAVE;
  if ((threadIdx.x & (WAVE - 1)) == 0) lds[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) t += lds[i];
  __syncthreads();
  return t;
}

// (value, index) order of the greedy choice: larger value first, lower index on ties.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// The better (value, index) of a wave under `better`, in every lane.
__device__ __forceinline__ void wave_best(float &v, int &i) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(v, o, WAVE);
    const int oi = __shfl_xor(i, o, WAVE);
    if (better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

// MoE routing of one row by one wave (pipeline.rs MoeFfn): softmax over all
// E <= 256 router logits (lane l holds experts l + 64 i), then the kk <= 8
// largest, one wave arg-max per pick over the experts not yet taken (larger
// first, lower index on ties).  Every lane returns the same ids isel[0..kk),
// their probabilities wsel[0..kk) and the probabilities' sum.
__device__ __forceinline__ void moe_topk(const float *row, int E, int kk, int lane, int (&isel)[8],
                                         float (&wsel)[8], float &sel) {
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + WAVE * i;
    v[i] = row[min(e, E - 1)];
    if (e >= E) v[i] = -INFINITY;
  }
  const float m = wave_max(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
  float zs = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) zs += lane + WAVE * i < E ? expf(v[i] - m) : 0.f;
  const float z = wave_sum(zs);
  unsigned taken = 0;
  sel = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= kk) break;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + WAVE * i;
      if (e < E && !(taken >> i & 1u) && better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
    wave_best(bv, bi);
    if (bi % WAVE == lane) taken |= 1u << (bi / WAVE);
    isel[j] = bi;
    wsel[j] = expf(bv - m) / z;
    sel += wsel[j];
  }
}

// ------------------------------------------------------ launch structs --

// Epilogues of the projection kernel.
enum {
  EPI_STORE = 0,     // C[m][n] = acc (+ bias[n])                 fp32
  EPI_ADD = 1,       // C[m][n] += acc                              fp32 (residual stream)
  EPI_SWIGLU = 2,    // H[m][n] = split(silu(acc_gate) * acc_up)   gate rows n, up rows n + N
  EPI_QKV = 3,       // bias + RoPE; q -> bf16 buffer, k/v -> KV cache
  EPI_LOGITS = 4,    // C = acc (fp32 logits) and each tile's greedy candidate per row
  EPI_MOE_ADD = 5,   // batch-1 GEMV only: C[n] += sum_j w_j y_j[n] + gate * acc (MoE combine)
};

// Where position pos of sequence seq sits in a KV cache: in the sequence's
// own contiguous region (pt null: unit seq, row pos) or, with a paged cache,
// in pool page pt[seq * mp + pos / P] at row pos % P.  `stride` is the
// elements of one unit (a sequence, or a page); the caller adds the layer
// offset and indexes rows with the unit's positions per head (S, or P).
__device__ __forceinline__ int64_t kv_loc(const int32_t *pt, int32_t mp, int32_t P, int64_t stride, int seq,
                                          int pos, int &row) {
  if (pt) {
    row = pos % P;
    return (int64_t)pt[(int64_t)seq * mp + pos / P] * stride;
  }
  row = pos;
  return (int64_t)seq * stride;
}

struct QkvEpi {
  const float *bias;       // fp32 [qkv rows] or null
  const float2 *cs;        // (cos, sin) [S][d/2]
  const int32_t *row_seq, *row_pos;  // device positions, or null: pos_arg / seq_arg (one row)
  int32_t pos_arg, seq_arg;
  uint16_t *q;             // split bf16 [rows][Hq][d], lo plane at q + q_lo
  int64_t q_lo;
  uint16_t *kcache, *vcache;
  int64_t seq_stride, layer_off;  // elements per sequence (per page when paged); layer offset
  int32_t S, Hq, Hkv, d;          // S: positions per (unit, layer, head) (the page size when paged)
  const int32_t *pt;              // paged cache: page table [seq][mp], else null
  int32_t mp, P;
};

struct ArgmaxEpi {
  float *part_val;         // [rows][ntiles] best logit of each 16-column tile
  int32_t *part_idx;       // [rows][ntiles]
};

struct GemmArgs {
  const uint16_t *A;      // bf16 activations, row m at A + row(m) * lda
  int64_t a_lo;           // element offset of A's lo plane (0: A is plain bf16)
  const int32_t *a_rows;  // optional gather: A row of output row m (grouped mode: by pair)
  int64_t lda;
  // fused RMSNorm prologue: when x is set, A = bf16(x * rsqrt(mean(x^2) + eps) * gamma)
  const float *x;
  const float *gamma;
  float eps;
  const uint16_t *W;      // bf16 weights [rows][K] row-major (per group: W + expert * w_group_stride)
  const uint16_t *Wp;     // the same weights packed in 32-row x 16-k MFMA tiles (chunk kernel), or null
  // int8 codes of W [rows][K] with per-row scales (power-of-two): when set,
  // the multi-row kernel streams these instead of W and scales each output
  // by its row's scale (the dequantised W is exactly code x scale)
  const int8_t *Wq;
  const float *wscale;
  int64_t w_group_stride;
  int32_t M, N, K;
  int32_t np_off;         // row offset of the second weight tile (SwiGLU: N, QKV: d / 2)
  float *C;               // fp32 output / residual, row m at C + m * ldc
  uint16_t *Hout;         // split bf16 output for EPI_SWIGLU, row m at Hout + m * ldc
  int64_t h_lo;           // element offset of Hout's lo plane
  int64_t ldc;
  const float *bias;      // optional, EPI_STORE only
  // grouped (MoE) mode: blockIdx.y = group; rows of group g are
  // group_start[g] .. group_start[g] + group_count[g]; weights of expert group_expert[g]
  const int32_t *n_groups;
  const int32_t *group_expert;
  const int32_t *group_start;
  const int32_t *group_count;
  // split-K: blockIdx.z = split; partial sums go to Cpart[split][M][np * N]
  float *Cpart;
  int32_t ksplit;
  // chunk projections of 256+ rows: 1 lets launch_gemm_chunk take the wide
  // kernel (256 x 256 blocks; the caller sized ksplit for its row blocks)
  int32_t wide;
  // EPI_ADD with split K: the reduce also writes RMSNorm(new x; norm_gamma)
  // as split bf16 [M][N] at norm_out (lo plane at + norm_lo), if set
  const float *norm_gamma;
  float norm_eps;
  uint16_t *norm_out;
  int64_t norm_lo;
  QkvEpi qkv;
  ArgmaxEpi am;
};
