// Host-side launchers of the gfx950 kernels (one per kernel family) and the
// argument structs they take.  All launchers enqueue on the given stream and
// return the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "common.h"

// ------------------------------------------------------------ projection --
int gemm_mtiles(int rows);
// max_rows: the largest row count of any group (dense: M); n_group_slots:
// grid size over groups in grouped mode (blocks past *n_groups exit).
hipError_t launch_gemm(const GemmArgs &g, int epi, int max_rows, int n_group_slots, hipStream_t st);

// ------------------------------------------------------------- attention --
struct AttnArgs {
  const uint16_t *q;       // bf16 [rows][Hq][d], rotated
  uint16_t *out;           // bf16 [rows][Hq][d]
  const uint16_t *kcache;  // K cache base: [seq][layer][Hkv][S][d]
  const uint16_t *vcache;  // V cache base, transposed: [seq][layer][Hkv][d][S]
  const int32_t *row_seq;  // [rows]
  const int32_t *row_pos;  // [rows]: absolute position of each query row
  int64_t seq_stride;      // elements per sequence in either cache
  int64_t layer_off;       // element offset of this layer inside a sequence
  int32_t S;               // positions allocated per (seq, layer, head), multiple of 32
  int32_t Hq, Hkv, G;
  int32_t rows, rows_per_group, n_groups;
  int32_t kc, n_splits;    // keys per split (multiple of 32), splits per group
  float scale_log2;        // log2(e) / sqrt(d)
  float *part_o;           // [n_groups * n_splits][16][d]
  float *part_ml;          // [n_groups * n_splits][16][2]
};
hipError_t launch_attention(const AttnArgs &a, int head_dim, hipStream_t st);

// ------------------------------------------------------ row-wise kernels --
// x[r][:] = E[tok(r)][:], tok(r) = next_token[row_seq[r]] if use_next else ids[r]
hipError_t launch_embed(const uint16_t *E, const int32_t *ids, const int32_t *next_token,
                        const int32_t *row_seq, int use_next, int rows, int H, float *x,
                        hipStream_t st);
// out[r] = bf16(x[r0 + r] * rsqrt(mean(x^2) + eps) * g)
hipError_t launch_rmsnorm(const float *x, int64_t ldx, const float *g, int rows, int H, float eps,
                          uint16_t *out, int64_t ldo, hipStream_t st);

struct RopeArgs {
  const float *qkv;        // fp32 [rows][qkv_rows]
  const float *bias;       // fp32 [qkv_rows] or null
  const float2 *cs;        // (cos, sin) [S][d/2]
  const int32_t *row_seq, *row_pos;
  uint16_t *q;             // bf16 [rows][Hq][d]
  uint16_t *kcache, *vcache;
  int64_t seq_stride, layer_off;
  int32_t S, Hq, Hkv, d, rows;
};
hipError_t launch_rope_append(const RopeArgs &a, hipStream_t st);

// V^T cache import: src [Hkv][len][d] -> dst [Hkv][d][S] (positions < len)
hipError_t launch_kv_load_v(const uint16_t *src, uint16_t *dst, int Hkv, int len, int d, int S,
                            hipStream_t st);

// idx[r] = argmax_v logits[r][v] (lowest v on ties); also next_token[row_seq[r]] = idx[r]
hipError_t launch_argmax(const float *logits, int64_t ld, int rows, int V, int32_t *idx,
                         int32_t *next_token, const int32_t *row_seq, hipStream_t st);

// ------------------------------------------------------------------- MoE --
struct MoeRouteArgs {
  const float *logits;     // fp32 [rows][E] router logits
  const uint16_t *act;     // bf16 [rows][H] normed FFN input (for the shared gate)
  const uint16_t *w_sh_gate;  // bf16 [H] or null
  int32_t rows, E, k, H, renorm;
  int32_t *ids;            // [rows][k]
  float *wts;              // [rows][k]
  float *gate;             // [rows] shared-expert scale
  int32_t *ids_record;     // optional copy of ids (per-layer record)
  // grouping outputs
  int32_t *n_groups, *group_expert, *group_start, *group_count;
  int32_t *pair_row;       // [rows*k]: token row of sorted pair p
  int32_t *pair_of;        // [rows*k]: sorted pair index of (row, slot)
};
hipError_t launch_moe_route(const MoeRouteArgs &a, hipStream_t st);

// x[r][:] += sum_j wts[r][j] * y[pair_of[r*k+j]][:] + gate[r] * ysh[r][:]
hipError_t launch_moe_combine(float *x, const float *y, const float *ysh, const float *wts,
                              const float *gate, const int32_t *pair_of, int rows, int k, int H,
                              hipStream_t st);
