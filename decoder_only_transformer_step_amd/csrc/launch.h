// Host-side launchers of the gfx950 kernels (one per kernel family) and the
// argument structs they take.  All launchers enqueue on the given stream and
// return the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "common.h"

// ------------------------------------------------------------ projection --
// decode-size row counts get the RMSNorm fused into the projection prologue
constexpr int GEMM_NORM_MAX_ROWS = 4;
constexpr size_t GEMM_NORM_MAX_LDS = 48 * 1024;
int gemm_mtiles(int rows);
int gemm_ntiles(const GemmArgs &g, int epi);
bool gemm_norm_fits(int rows, int K);
// max_rows: the largest row count of any group (dense: M); n_group_slots:
// grid size over groups in grouped mode (blocks past *n_groups exit).
hipError_t launch_gemm(const GemmArgs &g, int epi, int max_rows, int n_group_slots, hipStream_t st);
// the fixed-order split-K reduction plus epilogue over Cpart (ntiles 16-row tiles)
hipError_t launch_gemm_reduce(const GemmArgs &g, int epi, int ntiles, hipStream_t st);
// Chunk projection (up to 512 rows, A in global memory, no grouping): blocks
// of 256 weight rows (128 row pairs for the paired epilogues) times g.ksplit
// k ranges.
bool gemm_chunk_fits(const GemmArgs &g, int epi);
// Packed weight copy for the chunk kernel: P[((nt * K / 16 + kt) * 64 + l) * 8 + e]
// = W[32 nt + l % 32][16 kt + 8 (l / 32) + e] (rows % 32 == 0, K % 16 == 0).
bool pack_w32_fits(int64_t rows, int K);
hipError_t launch_pack_w32(const uint16_t *W, int64_t rows, int K, uint16_t *P, hipStream_t st);
// the same for a [rows][K] slice of a matrix whose rows are ld elements apart
// (ld % 8 == 0, W 16-byte aligned)
hipError_t launch_pack_w32_ld(const uint16_t *W, int64_t ld, int64_t rows, int K, uint16_t *P, hipStream_t st);
int gemm_chunk_tiles(const GemmArgs &g, int epi);
int gemm_chunk_mblocks(int rows);
hipError_t launch_gemm_chunk(const GemmArgs &g, int epi, hipStream_t st);
// Grouped chunk projection (MoE experts, EPI_SWIGLU or EPI_STORE, no split):
// g.Wp packs the stacked [E][rows][K] expert weights, g.w_group_stride is
// one expert's rows x K; rows of group i are group_start[i] ..
// + group_count[i] (A row through a_rows when set).  pairs: the groups'
// rows in total (the output rows); group_slots bounds the device-side group
// count.
bool gemm_chunk_grouped_fits(const GemmArgs &g, int epi);
hipError_t launch_gemm_chunk_grouped(const GemmArgs &g, int epi, int pairs, int group_slots, hipStream_t st);
// Chunks of GEMM_WIDE_MIN_ROWS or more rows (not the logits) with g.wide
// set take the wide kernel inside launch_gemm_chunk: 256 x 256 blocks, both
// operands in LDS.
constexpr int GEMM_WIDE_MIN_ROWS = 256;
bool gemm_wide_takes(const GemmArgs &g, int epi);
int gemm_wide_mblocks(int rows);
hipError_t launch_gemm_wide(const GemmArgs &g, int epi, int ntiles16, int units, hipStream_t st);
// Projection of 2 .. GEMV_ROWS_MAX rows with bf16 weights, each weight row
// streamed once (verify passes, small decode batches): K split over the waves
// of a block, the rows' activations in registers (x + gamma: fused RMSNorm;
// else split-bf16 A).  No split-K partials, no grouping.
constexpr int GEMV_ROWS_MAX = 8;
bool gemv_rows_fits(const GemmArgs &g, int epi);
// whether rows x K activations fit the kernel's registers (for choosing the
// fused RMSNorm prologue before the weights are known)
bool gemv_rows_takes(int rows, int K);
// grid size: the argmax partials per row of an EPI_LOGITS launch
int gemv_rows_grid(const GemmArgs &g, int epi);
hipError_t launch_gemv_rows(const GemmArgs &g, int epi, hipStream_t st);

// ------------------------------------------------ single-token projection --
struct GemvArgs {
  const uint16_t *W;          // bf16 [rows][K]
  const int8_t *Wq;           // or int8 codes [rows][K] with per-row scales wscale [rows],
  const float *wscale;        //   or (qbits 4) 4-bit codes [rows][K / 2] with exponents wexp
  const int8_t *wexp;         //   [rows][K / 32] (one power of two per group of 32 weights)
  int32_t qbits;              // 0 bf16 W, 8 int8 Wq + wscale, 4 packed 4-bit Wq + wexp
  int64_t w_group_stride;     // grouped mode: elements between experts
  const int32_t *slot_expert; // grouped mode: expert of each routing slot (blockIdx.y), else null
  int32_t n_slots;
  const float *a_f32;         // fp32 activation [K] (per slot: + slot * a_slot_stride), or null
  int64_t a_slot_stride;
  const uint16_t *a_bf16;     // bf16 activation [K] when a_f32 is null
  const float *gamma;         // fused RMSNorm gain (a_f32 is then the raw residual x)
  float eps;
  int32_t K, N, n_items;      // N: rows of the first half (SwiGLU), n_items: rows or row pairs
  float *C;                   // fp32 output (per slot: + slot * ldc)
  int64_t ldc;
  const float *bias;          // EPI_STORE only
  QkvEpi qkv;                 // EPI_QKV
  float *part_val;            // EPI_LOGITS: best logit of each block
  int32_t *part_idx;
  // EPI_MOE_ADD: routed expert outputs y [k][N], their weights w [k] and the
  // shared-expert scale gate [1] (the kernel's own rows are the shared expert's)
  const float *moe_y, *moe_w, *moe_gate;
  int32_t moe_k;
  // optional second part of an EPI_SWIGLU grouped launch (the shared expert):
  // weights W2 [2 N2][K], N2 row pairs into C2 [N2]; blocks1 is set by the launcher
  const uint16_t *W2;
  const int8_t *W2q;          // its codes and row scales (or exponents) when the first part is quantised
  const float *w2scale;
  const int8_t *w2exp;
  int32_t N2, n_items2;
  float *C2;
  int32_t blocks1;
  // grouped mode routed in the kernel (batch-1 MoE decode), in place of
  // slot_expert: the expert of slot j is the j-th pick of the top-k of the
  // router logits route_logits [route_E] (moe_topk).  Block (0, slot 0)
  // also publishes the ids (route_ids [k], route_rec [k] if set), their
  // weights (route_wts [k], renormalised over the picks if route_renorm) and
  // the shared-expert scale route_gate [1] = sigmoid(route_w_sg . b), or 1
  // without a gate vector, for the launches that follow.
  const float *route_logits;
  int32_t route_E, route_renorm;
  int32_t *route_ids, *route_rec;
  float *route_wts, *route_gate;
  const uint16_t *route_w_sg;
};
constexpr size_t GEMV_MAX_LDS = 60 * 1024;
// LDS of one GEMV block: the fp32 activation padded to whole load steps
// (512 elements of bf16 weights, 1024 of int8, 2048 of 4-bit weights; the
// 4-bit path adds one fp32 group sum per lane and step)
inline size_t gemv_lds(int K, int qbits = 0) {
  const size_t step = qbits == 4 ? 2048 : qbits == 8 ? 1024 : 512;
  const size_t steps = (size_t)(K + step - 1) / step;
  return steps * step * 4 + (qbits == 4 ? steps * 64 * 4 : 0);
}
// blocks of a GEMV launch over n_items items (one argmax partial each for EPI_LOGITS)
int gemv_blocks(int n_items);
// `blocks` (optional) receives the grid size, i.e. the number of argmax
// partials an EPI_LOGITS launch writes
hipError_t launch_gemv(const GemvArgs &g, int epi, hipStream_t st, int *blocks = nullptr);
// Arrival counters of the fused launches sit SYNC_STRIDE words apart (one
// 128-byte line each).  Device-scope atomics on one address are serialised
// where memory performs them, so a launch whose many blocks arrive together
// spreads them over GV_NCNT counters.
constexpr int SYNC_STRIDE = 32;
constexpr int GV_NCNT = 64;
// Batch-1 dense FFN in one launch: the SwiGLU gate/up GEMV (gu, output gu.C)
// and the down GEMV of that output (dn, activation dn.a_f32 == gu.C), the
// down blocks waiting for the gate/up blocks' arrivals.  Block b of the
// first part counts on cnt[(b % GV_NCNT) SYNC_STRIDE]; base[i] is counter
// i's value when the step began (all cumulative).  bf16 weights only.
bool gemv_ffn_fits(const GemvArgs &gu, const GemvArgs &dn);
hipError_t launch_gemv_ffn(const GemvArgs &gu, const GemvArgs &dn, uint32_t *cnt, const uint32_t *base,
                           hipStream_t st);

// idx[r] = argmax over part_val[r][0 .. nparts) (lowest index on ties), and
// next_token[row_seq[r]] = idx[r] for the last row of each run of rows with
// equal row_seq (callers keep a sequence's rows consecutive)
hipError_t launch_argmax_finalize(const float *part_val, const int32_t *part_idx, int nparts, int rows,
                                  int32_t *idx, int32_t *next_token, const int32_t *row_seq,
                                  hipStream_t st);

// ------------------------------------------------------------- attention --
struct AttnArgs {
  const uint16_t *q;       // split bf16 [rows][Hq][d], rotated; lo plane at q + q_lo
  int64_t q_lo;
  uint16_t *out;           // split bf16 [rows][Hq][d] (lo plane at out + out_lo), or null
  int64_t out_lo;
  float *out_f32;          // fp32 [rows][Hq][d] (batch-1 decode feeds the fp32 projection)
  const uint16_t *kcache;  // K cache base: [seq][layer][Hkv][S][d]
  const uint16_t *vcache;  // V cache base, transposed: [seq][layer][Hkv][d][S]
  const int32_t *row_seq;  // [rows]
  const int32_t *row_pos;  // [rows]: absolute position of each query row
  int64_t seq_stride;      // elements per sequence in either cache (per page when paged)
  int64_t layer_off;       // element offset of this layer inside a sequence (a page)
  int32_t S;               // positions per (seq or page, layer, head), multiple of 32
  const int32_t *pt;       // paged cache: page table [seq][mp] (pages of S positions), else null
  int32_t mp;
  int32_t Hq, Hkv, G;
  int32_t rows, rows_per_group, n_groups;
  int32_t kc, n_splits;    // keys per split (multiple of 32), splits per group
  float scale_log2;        // log2(e) / sqrt(d)
  float *part_o;           // [n_groups * n_splits][16][d]
  float *part_ml;          // [n_groups * n_splits][16][2]
  // arrival counters [n_groups], zero between launches: when set, the last
  // block of a group to finish merges the group's splits (no merge launch)
  int32_t *counters;
  // Where the kernel takes each row's position and sequence from:
  // 0: row_pos / row_seq in device memory; 1: pos_arg / seq_arg (one row per
  // group, rows <= 16; no dependent load before the cache reads); 2: a chunk
  // of one sequence, row r at position pos0 + r of sequence seq0.
  int32_t pos_mode, pos0, seq0;
  int32_t pos_arg[16], seq_arg[16];
  // Variants (engine.zig Engine.forward passes a logit soft-cap and, on a
  // sliding layer, a window to its attention; decoder.rs AttnWeights::sinks)
  int32_t window;          // 0: every earlier key; W > 0: keys pos - W < t <= pos
  float softcap;           // 0: off; c > 0: scaled score s -> c tanh(s / c)
  float scale;             // 1 / sqrt(d), for the soft-cap
  const float *sinks;      // [Hq] sink logits of this layer, or null
  // Batch-1 decode with the output projection fused (wo set; fp32 output,
  // in-kernel merge): o_blocks blocks past the attention grid each own
  // 4 ATTN_O_RPW rows of the bf16 matrix wo [o_rows][Hq d] and finish
  // o_x[n] = o_x[n] + wo[n] . o once every column group has published o.
  // *o_done counts the groups that have, over every fused launch of this
  // layer (it is never reset); *o_base is its value when the step began
  // (copied by the step's embedding launch), so this launch's groups are
  // all in once it reaches *o_base + n_groups (modulo 2^32).  Both live
  // in device memory, so a captured graph replays correctly.
  const uint16_t *wo;
  float *o_x;
  int32_t o_rows, o_blocks;
  uint32_t *o_done;
  const uint32_t *o_base;
};

// fused output projection: rows per wave, and the widest input it holds
// (one row of at most ATTN_O_MAX_K bf16 weights per register set)
constexpr int ATTN_O_RPW = 4;
constexpr int ATTN_O_MAX_K = 4096;

constexpr float ATTN_LOG2E = 1.4426950408889634f;
// splits per group that attn_kernel merges itself (its last block to finish)
constexpr int ATTN_FUSED_MAX_SPLITS = 32;

// Score of a raw q.k product in log2 units (scaled, soft-capped when set).
__device__ __forceinline__ float attn_logit2(const AttnArgs &a, float s) {
  if (a.softcap > 0.f) return a.softcap * tanhf(s * a.scale / a.softcap) * ATTN_LOG2E;
  return s * a.scale_log2;
}

// Whether key t is visible to a query at position pos (causal, windowed).
__device__ __forceinline__ bool attn_key_ok(const AttnArgs &a, int t, int pos) {
  return t <= pos && (a.window <= 0 || t > pos - a.window);
}

// First key (a multiple of 32) that a group whose lowest query position is
// minpos can see: the key ranges of its splits start there.
__host__ __device__ inline int attn_key_start(int window, int minpos) {
  return window > 0 ? (max(0, minpos - window + 1) & ~31) : 0;
}

// Fold head's sink logit into a finished softmax with running maximum M and
// sum L (log2 units): L becomes the full denominator and the return value
// is the factor that rescales the accumulated output to the new maximum.
__device__ __forceinline__ float attn_sink_fold(const AttnArgs &a, int head, float &M, float &L) {
  if (!a.sinks) return 1.f;
  const float z = a.sinks[head] * ATTN_LOG2E;
  const float Mn = fmaxf(M, z);
  const float r = exp2f(M - Mn);
  L = L * r + exp2f(z - Mn);
  M = Mn;
  return r;
}

hipError_t launch_attention(const AttnArgs &a, int head_dim, hipStream_t st);
// Prefill-chunk attention (pos_mode 2, split-bf16 output, d = 64 or 128);
// sets its own groups and splits.  Uses part_o / part_ml like the general
// kernel (at most ATTN_MAX_TASKS * 16 columns of partials).
bool attention_chunk_fits(const AttnArgs &a, int head_dim);
hipError_t launch_attention_chunk(const AttnArgs &a, int head_dim, hipStream_t st);

// ------------------------------------------------------ row-wise kernels --
// x[r][:] = E[tok(r)][:], tok(r) = next_token[row_seq[r]] if use_next else ids[r]
// (o_base[i] = o_cnt[i * o_stride] for i < n_o: the snapshot of the fused
// launches' arrival counters that this step's launches count from)
hipError_t launch_embed(const uint16_t *E, const int32_t *ids, const int32_t *next_token,
                        const int32_t *row_seq, int use_next, int rows, int H, float *x,
                        const uint32_t *o_cnt, uint32_t *o_base, int n_o, int o_stride, hipStream_t st);
// out[r] = x[r] * rsqrt(mean(x^2) + eps) * g as split bf16 (lo plane at out + out_lo),
// or fp32 into out_f32 when it is set
hipError_t launch_rmsnorm(const float *x, int64_t ldx, const float *g, int rows, int H, float eps,
                          uint16_t *out, int64_t ldo, int64_t out_lo, hipStream_t st, float *out_f32 = nullptr);

// Per-head RMSNorm of q and k (gains [d], eps), then RoPE, the q store
// (split bf16 [rows][Hq][d], lo plane at q + q_lo) and the KV-cache append,
// from the projection's fp32 output qkv [rows][ld] (bias already added).
struct QkNormArgs {
  const float *qkv;
  int64_t ld;
  const float *q_norm, *k_norm;
  float eps;
  const float2 *cs;                  // (cos, sin) [S][d/2]
  const int32_t *row_seq, *row_pos;  // [rows]
  uint16_t *q;
  int64_t q_lo;
  uint16_t *kcache, *vcache;
  int64_t seq_stride, layer_off;
  int32_t S, Hq, Hkv, d, rows;
  const int32_t *pt;                 // paged cache: page table [seq][mp] (pages of S positions)
  int32_t mp;
};
hipError_t launch_qk_norm_rope(const QkNormArgs &a, hipStream_t st);

// One thread: out[1 + out[0]] = next_token[seq], out[0] += 1, row_pos[0] += 1
// (the last node of a captured decode step).
hipError_t launch_decode_advance(int32_t *row_pos, const int32_t *next_token, int seq, int32_t *out,
                                 hipStream_t st);

// Per-row int8 quantisation with a power-of-two scale: q [rows][K] int8,
// scale [rows] fp32 (= 2^e), deq [rows][K] the dequantised bf16 weights.
hipError_t launch_quantize_rows(const uint16_t *W, int64_t rows, int K, int8_t *q, float *scale, uint16_t *deq,
                                hipStream_t st);
// 4-bit quantisation, one power-of-two scale per group of 32 weights: codes
// [rows][K / 2] (nibble q + 8; element 2j low, 2j + 1 high in byte j), exps
// [rows][K / 32] int8, deq [rows][K] the dequantised bf16 weights.  K % 32 == 0.
hipError_t launch_quantize_q4(const uint16_t *W, int64_t rows, int K, uint8_t *codes, int8_t *exps, uint16_t *deq,
                              hipStream_t st);

// Paged-cache import of one layer of one sequence: K and V [Hkv][len][d]
// into the pages listed by pt (that sequence's page-table row; pages of P
// positions, unit elements per page, the layer at layer_off inside a page)
hipError_t launch_kv_load_paged(const uint16_t *src_k, const uint16_t *src_v, uint16_t *kpool, uint16_t *vpool,
                                const int32_t *pt, int64_t unit, int64_t layer_off, int Hkv, int len, int d, int P,
                                hipStream_t st);

// V^T cache import: src [Hkv][len][d] -> dst [Hkv][d][S] (positions < len)
hipError_t launch_kv_load_v(const uint16_t *src, uint16_t *dst, int Hkv, int len, int d, int S,
                            hipStream_t st);

// ------------------------------------------------------------------- MoE --
struct MoeRouteArgs {
  const float *logits;     // fp32 [rows][E] router logits
  const uint16_t *w_router;  // bf16 [E][H]: when set, the route launch computes the logits itself
                             // from RMSNorm(act_f32 rows; gamma) (act_f32 and gamma required)
  float *logits_out;       // with w_router: optional copy of the computed logits [rows][E]
  const uint16_t *act;     // split bf16 [rows][H] normed FFN input (for the shared gate)
  int64_t act_lo;
  const float *act_f32;    // or fp32 [rows][H] when set
  const float *gamma;      // with act_f32: act_f32 is the raw residual x, normed here (RMSNorm, gain gamma)
  float eps;
  const uint16_t *w_sh_gate;  // bf16 [H] or null
  int32_t rows, E, k, H, renorm;
  int32_t *ids;            // [rows][k]
  float *wts;              // [rows][k]
  float *gate;             // [rows] shared-expert scale (optional)
  int32_t *ids_record;     // optional copy of ids (per-layer record)
  // grouping outputs
  int32_t *n_groups, *group_expert, *group_start, *group_count;
  int32_t *pair_row;       // [rows*k]: token row of sorted pair p
  int32_t *pair_of;        // [rows*k]: sorted pair index of (row, slot)
  // shared expert as extra_groups pseudo-experts (ids E .. E + extra_groups
  // - 1, every row): group table entries after the routed groups, pairs
  // rows*k + j*rows + r (pair_row then holds rows*(k + extra_groups))
  int32_t extra_groups;
  // with w_router and grouping: a zeroed arrival counter; the router launch
  // then builds the group table itself (its last block), and leaves the
  // counter zero again
  int32_t *arrive;
};
hipError_t launch_moe_route(const MoeRouteArgs &a, bool group, hipStream_t st);
// the largest hidden size the fused router (w_router set) keeps in LDS
constexpr int MOE_ROUTER_MAX_H = 8192;

// x[r][:] += sum_j wts[r][j] * y[pair_of[r*k+j]][:] + gate[r] * sum_i ysh[i*sh_stride + r*H][:]
// over sh_parts shared-expert parts (pair_of null: y is indexed by r*k+j directly)
hipError_t launch_moe_combine(float *x, const float *y, const float *ysh, const float *wts,
                              const float *gate, const int32_t *pair_of, int rows, int k, int H,
                              hipStream_t st, int sh_parts = 1, int64_t sh_stride = 0);
