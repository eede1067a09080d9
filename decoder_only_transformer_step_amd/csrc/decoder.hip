// Host runtime and C ABI of libdecoder.so (declared in include/decoder.h and
// include/decoder_diag.h).
//
// The decoder owns no device memory: decoder_init carves the KV cache, the
// RoPE table and every scratch buffer out of the caller's workspace once,
// so a step never allocates (pipeline.rs ForwardScratch: steady-state decode
// preallocates its buffers).  Per call the host validates everything, copies
// the token ids / row positions / row sequences into the workspace from a
// pinned staging ring, and enqueues the kernels of the step on the stream.
#include <hip/hip_runtime.h>

#include <array>
#include <cmath>
#include <mutex>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/decoder.h"
#include "../../include/decoder_diag.h"
#include "launch.h"

namespace {

constexpr int STAGE_RING = 64;     // pinned staging slots (one per call in flight)
constexpr int ATTN_TARGET_BLOCKS = 1024;
constexpr int ATTN_MAX_TASKS = 8192;
constexpr int GEMM_MAX_SPLIT = 8;
constexpr int CHUNK_MIN_ROWS = 16;   // more rows than this take the chunk projection kernel
// Batched decode: from this many rows, projections whose weights are at least
// CHUNK_BATCH_MIN_BYTES also take the chunk kernel (measured on the 8B shape
// at 8 and 16 rows: faster for qkv, gate_up and down; not for the 33.5 MB o_proj)
constexpr int CHUNK_BATCH_MIN_ROWS = 8;
constexpr double CHUNK_BATCH_MIN_BYTES = 40e6;
constexpr int CHUNK_MAX_SPLIT = 16;
constexpr int WIDE_MAX_SPLIT = 6;  // largest split-K the wide chunk kernel takes
constexpr int MAX_CHUNK = 512;     // largest prefill chunk (rows per call)

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Layout {
  size_t kcache, vcache, rope, x, act, attn, q, qkv, h, logits, stage, next_token;
  size_t part_o, part_ml, attn_cnt, gpart, am_val, am_idx, am_out, f32_attn, f32_h, f32_act, f32_hexp;
  size_t gout;                 // decode_run: step counter, then the generated tokens [max_seq]
  size_t rlogits, rids, rids_rec, rwts, rgate, groups, pair_row, pair_of, hexp, yexp, hsh, ysh;
  size_t total;
  int S, R, RL;
  int64_t seq_stride;
  size_t gpart_elems, am_n;
  size_t packed;               // packed weight copies for the chunk kernel (or 0 bytes)
  size_t quant;                // quantised weights (codes, scales, dequantised copies), or 0
  // KV-cache units: a sequence each (contiguous), or pool pages (paged)
  int kvS;                     // positions per (unit, layer, head): S, or the page size
  int64_t kv_unit;             // elements of one unit in either cache
  size_t kv_units;             // max_batch, or the pool's page count
  int mp;                      // page-table entries per sequence (0: contiguous)
  size_t stage_n;              // int32 words of one staging slot (rows, then the page table)
};

// Matrices of a quantised model (weight_quant): per layer qkv, o, gate_up,
// down, then the lm-head; each takes int8 codes, fp32 scales and a
// dequantised bf16 copy, every piece 256-byte aligned.
// Dense: qkv, o, gate_up, down.  MoE: qkv, o, the shared expert's gate_up
// and down (when it has one), then every routed expert's gate_up rows
// [E * 2 Ie][H] and down rows [E * H][Ie].  Rows 0 leave a matrix out.
constexpr int QUANT_MATS = 6;
struct QuantSpec {
  int64_t rows[QUANT_MATS];
  int K[QUANT_MATS];
};

QuantSpec quant_spec(const decoder_config_t *c) {
  const int d = c->head_dim, H = c->hidden, qd = c->n_heads * d, qkvr = (c->n_heads + 2 * c->n_kv_heads) * d;
  if (c->n_experts > 0) {
    const int E = c->n_experts, Ie = c->expert_inter, Is = c->shared_inter;
    return QuantSpec{{qkvr, H, 2 * (int64_t)Is, Is > 0 ? H : 0, (int64_t)E * 2 * Ie, (int64_t)E * H},
                     {H, qd, H, Is, H, Ie}};
  }
  const int I = c->ffn_inter;
  return QuantSpec{{qkvr, H, 2 * (int64_t)I, H, 0, 0}, {H, qd, H, I, 0, 0}};
}

size_t quant_piece(size_t bytes) { return (bytes + 255) / 256 * 256; }

// int8: codes [rows][K], scales [rows] fp32; 4-bit: codes [rows][K / 2],
// exponents [rows][K / 32] int8; both: the dequantised bf16 copy [rows][K]
size_t quant_code_bytes(int wq, int64_t rows, int K) { return wq == 2 ? (size_t)rows * K / 2 : (size_t)rows * K; }
size_t quant_scale_bytes(int wq, int64_t rows, int K) { return wq == 2 ? (size_t)rows * (K / 32) : (size_t)rows * 4; }

size_t quant_matrix_bytes(int wq, int64_t rows, int K) {
  return quant_piece(quant_code_bytes(wq, rows, K)) + quant_piece(quant_scale_bytes(wq, rows, K)) +
         quant_piece((size_t)rows * K * 2);
}

size_t quant_bytes(const decoder_config_t *c) {
  if (!c->weight_quant) return 0;
  const QuantSpec qs = quant_spec(c);
  size_t b = quant_matrix_bytes(c->weight_quant, c->vocab, c->hidden);
  for (int i = 0; i < QUANT_MATS; ++i)
    if (qs.rows[i] > 0) b += (size_t)c->n_layers * quant_matrix_bytes(c->weight_quant, qs.rows[i], qs.K[i]);
  return b;
}

// Weight matrices that get a packed copy for the chunk projection kernel:
// only when prefill chunks or decode batches can reach the chunk kernel, and
// only the shapes the packed tiles cover.  Order within a layer: qkv, o, gate_up /
// shared gate_up, down / shared down, then (MoE, prefill chunks only) the
// stacked expert gate/up and down matrices for the grouped form.
constexpr int PACK_MATS = 6;
struct PackSpec {
  int64_t rows[PACK_MATS];
  int K[PACK_MATS];
};

// The grouped expert projection of a prefill chunk streams the routed
// experts from a packed copy of their stacked weights; when the shared
// expert's intermediate size is a multiple of an expert's, the shared expert
// joins that copy as Is / Ie pseudo-experts (pseudo-expert j: gate and up
// rows j Ie .. (j + 1) Ie, and those columns of the down projection), which
// every row takes with the shared gate as its weight, and the combine sums
// their down outputs.  Returns that count, or 0 (the shared expert then runs
// as its own two chunk projections).
constexpr int MOE_MAX_SHARED_PARTS = 8;

bool moe_grouped_packed(const decoder_config_t *c) {
  return c->n_experts > 0 && c->max_chunk > CHUNK_MIN_ROWS && c->expert_inter > 0 && c->expert_inter % 32 == 0 &&
         c->hidden % 32 == 0;
}

int moe_shared_parts(const decoder_config_t *c) {
  if (!moe_grouped_packed(c) || c->shared_inter <= 0 || c->shared_inter % c->expert_inter) return 0;
  const int s = c->shared_inter / c->expert_inter;
  return s <= MOE_MAX_SHARED_PARTS ? s : 0;
}

PackSpec pack_spec(const decoder_config_t *c) {
  PackSpec p{};
  if (c->max_chunk <= CHUNK_MIN_ROWS && c->max_batch < CHUNK_BATCH_MIN_ROWS) return p;
  const int d = c->head_dim, H = c->hidden, qd = c->n_heads * d, qkvr = (c->n_heads + 2 * c->n_kv_heads) * d;
  const int I = c->n_experts > 0 ? c->shared_inter : c->ffn_inter;
  // the grouped form needs each expert's slice (and its up half) on a
  // 32-row tile boundary; the shared expert's pseudo-experts follow the
  // routed ones
  const int Ie = c->expert_inter;
  const bool grouped = moe_grouped_packed(c);
  const int64_t ex = (int64_t)c->n_experts + moe_shared_parts(c);
  const int64_t rows[PACK_MATS] = {qkvr, H, 2 * (int64_t)I, I > 0 ? H : 0, grouped ? 2 * ex * Ie : 0,
                                   grouped ? ex * H : 0};
  const int K[PACK_MATS] = {H, qd, H, I, H, Ie};
  for (int i = 0; i < PACK_MATS; ++i) {
    const bool ok = rows[i] > 0 && K[i] > 0 && pack_w32_fits(rows[i], K[i]);
    p.rows[i] = ok ? rows[i] : 0;
    p.K[i] = ok ? K[i] : 0;
  }
  return p;
}

size_t pack_layer_elems(const PackSpec &p) {
  size_t n = 0;
  for (int i = 0; i < PACK_MATS; ++i) n += (size_t)p.rows[i] * p.K[i];
  return n;
}

bool config_ok(const decoder_config_t *c) {
  if (!c) return false;
  if (c->hidden <= 0 || c->hidden % 8 || c->n_layers <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0)
    return false;
  if (c->n_heads % c->n_kv_heads || c->n_heads / c->n_kv_heads > 16) return false;
  // attention work lists: a decode batch has max_batch x Hkv (row, kv head)
  // groups, a prefill chunk ceil(max_chunk / (16 / G)) x Hkv; each must fit
  // the split partial buffers with at least one split
  {
    const int64_t G = c->n_heads / c->n_kv_heads, rpg = 16 / G;
    if ((int64_t)c->max_batch * c->n_kv_heads > ATTN_MAX_TASKS ||
        ((int64_t)c->max_chunk + rpg - 1) / rpg * c->n_kv_heads > ATTN_MAX_TASKS)
      return false;
  }
  if (c->head_dim != 64 && c->head_dim != 128) return false;
  if (c->vocab <= 0 || c->max_seq <= 0 || c->max_chunk <= 0 || c->max_chunk > MAX_CHUNK ||
      c->max_batch <= 0 || c->max_batch > 256)
    return false;
  if (!(c->rope_base > 0.0) || !(c->rms_eps >= 0.0)) return false;
  if (c->sliding_window < 0 || !(c->attn_softcap >= 0.0) || c->attn_softcap > 1e30) return false;
  if (c->qk_norm != 0 && c->qk_norm != 1) return false;
  if (c->kv_page_size < 0 || (c->kv_page_size > 0 && (c->kv_page_size % 32 || c->kv_pages < 1)))
    return false;
  // quantised GEMVs load 16 int8 codes (one row scale) or 32 4-bit codes (one
  // group of 32 with its scale) per lane: every row length a multiple of that
  if (c->weight_quant < 0 || c->weight_quant > 2) return false;
  if (c->weight_quant != 0) {
    const int m = c->weight_quant == 2 ? 32 : 16;
    if (c->hidden % m || c->ffn_inter % m || c->expert_inter % m || c->shared_inter % m) return false;
  }
  if (c->n_experts > 0) {
    if (c->n_experts > 256 || c->top_k <= 0 || c->top_k > 8 || c->top_k > c->n_experts) return false;
    if (c->hidden > MOE_ROUTER_MAX_H) return false;  // the router keeps the normed row in LDS
    if (c->expert_inter <= 0 || c->expert_inter % 8 || c->shared_inter < 0 || c->shared_inter % 8)
      return false;
  } else {
    if (c->ffn_inter <= 0 || c->ffn_inter % 8) return false;
  }
  return true;
}

// Words of the attention counter block: the split-merge counters and the
// router's, the step snapshots of the fused launches' arrival counters, then
// those counters, one 128-byte line each.
int n_sync(const decoder_config_t &c) { return c.n_layers * (1 + GV_NCNT); }
size_t sync_cnt_off(const decoder_config_t &c) {
  return align_up((size_t)(ATTN_MAX_TASKS + 1 + n_sync(c)), SYNC_STRIDE);
}
size_t attn_cnt_words(const decoder_config_t &c) { return sync_cnt_off(c) + (size_t)n_sync(c) * SYNC_STRIDE; }

Layout make_layout(const decoder_config_t *c) {
  Layout L{};
  const size_t A = 256;
  const int d = c->head_dim, H = c->hidden, Hq = c->n_heads, Hkv = c->n_kv_heads;
  const int qd = Hq * d, qkvr = (Hq + 2 * Hkv) * d;
  L.S = (int)align_up((size_t)c->max_seq, 32);
  L.R = std::max(c->max_chunk, c->max_batch);
  L.RL = std::max(c->max_chunk, c->max_batch);
  L.seq_stride = (int64_t)c->n_layers * Hkv * (int64_t)L.S * d;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + std::max<size_t>(bytes, 1), A);
    return o;
  };
  if (c->kv_page_size > 0) {
    L.kvS = c->kv_page_size;
    L.kv_unit = (int64_t)c->n_layers * Hkv * (int64_t)L.kvS * d;
    L.kv_units = (size_t)c->kv_pages;
    L.mp = (c->max_seq + c->kv_page_size - 1) / c->kv_page_size;
  } else {
    L.kvS = L.S;
    L.kv_unit = L.seq_stride;
    L.kv_units = (size_t)c->max_batch;
    L.mp = 0;
  }
  L.stage_n = (size_t)3 * L.R + (size_t)c->max_batch * L.mp;
  const size_t kv = L.kv_units * L.kv_unit * 2;
  L.kcache = take(kv);
  L.vcache = take(kv);
  L.rope = take((size_t)L.S * (d / 2) * sizeof(float2));
  L.x = take((size_t)L.R * H * 4);
  // split-bf16 activations: hi plane then lo plane
  L.act = take((size_t)L.R * H * 4);
  L.attn = take((size_t)L.R * qd * 4);
  L.q = take((size_t)L.R * qd * 4);
  L.qkv = take((size_t)L.R * qkvr * 4);
  L.h = take((size_t)L.R * std::max(c->ffn_inter, 1) * 4);
  L.logits = take((size_t)L.RL * c->vocab * 4);
  L.stage = take(L.stage_n * 4);
  L.next_token = take((size_t)c->max_batch * 4);
  L.gout = take((size_t)(c->max_seq + 1) * 4);
  L.part_o = take((size_t)ATTN_MAX_TASKS * 16 * d * 4);
  L.part_ml = take((size_t)ATTN_MAX_TASKS * 16 * 2 * 4);
  // one arrival counter per attention group, then the MoE router's, then
  // per layer the fused output projection's arrival counter, then per
  // layer that counter's value at the start of the current step
  L.attn_cnt = take((size_t)attn_cnt_words(*c) * 4);
  int max_small_n = std::max(qkvr, H);
  if (c->n_experts > 0) max_small_n = std::max(max_small_n, 2 * c->shared_inter);
  L.gpart_elems = (size_t)GEMM_MAX_SPLIT * L.R * 2 * (size_t)max_small_n;
  L.gpart = take(L.gpart_elems * 4);
  // argmax candidates: one per 16-column tile per row (multi-row lm-head),
  // or one per 8-row block (batch-1 lm-head)
  const size_t am_n = std::max((size_t)L.RL * ((c->vocab + 15) / 16), (size_t)(c->vocab + 3) / 4);
  L.am_n = am_n;
  L.am_val = take(am_n * 4);
  L.am_idx = take(am_n * 4);
  L.am_out = take((size_t)L.RL * 4);
  // fp32 activations of the batch-1 decode path
  L.f32_attn = take((size_t)qd * 4);
  L.f32_h = take((size_t)std::max(std::max(c->ffn_inter, c->shared_inter), 1) * 4);
  L.f32_act = take((size_t)H * 4);
  L.f32_hexp = take((size_t)std::max(c->top_k, 1) * std::max(c->expert_inter, 1) * 4);
  if (c->n_experts > 0) {
    const int E = c->n_experts, k = c->top_k, P = L.R * k, S = moe_shared_parts(c);
    const size_t PS = (size_t)L.R * (k + S);  // pairs, the shared pseudo-experts' included
    L.rlogits = take((size_t)L.R * E * 4);
    L.rids = take((size_t)P * 4);
    L.rids_rec = take((size_t)c->n_layers * P * 4);
    L.rwts = take((size_t)P * 4);
    L.rgate = take((size_t)L.R * 4);
    L.groups = take((size_t)(1 + 3 * (E + S)) * 4);
    L.pair_row = take(PS * 4);
    L.pair_of = take((size_t)P * 4);
    L.hexp = take(PS * c->expert_inter * 4);
    L.yexp = take(PS * H * 4);
    L.hsh = take((size_t)L.R * std::max(c->shared_inter, 1) * 4);
    L.ysh = take((size_t)L.R * H * 4);
  }
  // packed weight copies (each matrix 256-byte aligned: element counts are
  // multiples of 512)
  L.packed = take(pack_layer_elems(pack_spec(c)) * 2 * c->n_layers);
  L.quant = take(quant_bytes(c));
  L.total = off;
  return L;
}

}  // namespace

struct decoder {
  decoder_config_t c;
  Layout L;
  std::vector<decoder_layer_weights_t> layers;
  struct Packed {
    // qkv, o, gate_up (or shared gate_up), down (or shared down), expert
    // gate_up, expert down; null if not packed
    const uint16_t *w[PACK_MATS];
  };
  std::vector<Packed> packed;
  struct QuantW {
    const int8_t *q = nullptr;  // int8 codes [rows][K], or 4-bit codes [rows][K / 2]
    const float *s = nullptr;   // int8: per-row scales 2^e
    const int8_t *e = nullptr;  // 4-bit: per-group exponents [rows][K / 32]
  };
  std::vector<std::array<QuantW, 6>> qw;  // per layer, in quant_spec order (weight_quant)
  QuantW qhead;                           // the lm-head (weight_quant)
  const uint16_t *embed = nullptr, *lm_head = nullptr;
  const float *final_norm = nullptr;
  hipStream_t stream = nullptr;
  char *ws = nullptr;
  // carved workspace
  uint16_t *kcache, *vcache, *act, *attn, *q, *h, *hexp, *hsh;
  float2 *rope;
  float *x, *qkv, *logits, *part_o, *part_ml, *gpart, *rlogits, *rwts, *rgate, *yexp, *ysh, *am_val;
  int32_t *ids, *row_seq, *row_pos, *next_token, *attn_cnt, *rids, *rids_rec, *groups, *pair_row, *pair_of;
  int32_t *am_idx, *am_out;
  int32_t *gout;
  // decode_run captures a step: positions come from device memory (row_pos)
  // instead of kernel arguments, so one captured step serves every position
  bool graph_mode = false;
  hipStream_t gstream = nullptr;  // decode_run's capture stream (the caller's may be the null stream)
  float *f32_attn, *f32_h, *f32_act, *f32_hexp;
  size_t am_cap = 0;           // argmax partials the am_val / am_idx buffers hold
  int cus = 256;               // compute units of the device
  // D->act holds RMSNorm(x; act_norm) of the first act_rows rows of x (split
  // bf16), written by a fused reduce; null when x has changed since
  const float *act_norm = nullptr;
  int act_rows = 0;
  bool single_row_ok = false;  // the batch-1 GEMV path fits every K of this config
  int64_t act_lo = 0, attn_lo = 0, q_lo = 0, h_lo = 0, hexp_lo = 0, hsh_lo = 0;  // lo-plane offsets
  // host state
  std::vector<int32_t> len;
  std::vector<int32_t> hseq;  // host copy of the current call's row sequences
  std::vector<char> has_next;
  std::vector<std::vector<int32_t>> kv_pending;  // per seq: layers loaded with the pending len
  int layer_limit = -1;
  bool stop_after_attn = false;  // the last layer run stops after o_proj + residual
  int stop_mid_layer = -1;       // that layer, for the current step (-1: none)
  bool fuse_o = true;            // batch-1 decode: output projection inside the attention launch
  bool fuse_ffn = true;          // batch-1 decode: gate/up and down projections in one launch
  int last_rows = 0;
  int32_t *pinned = nullptr;
  // paged KV cache: device page table [max_batch][mp] (staged with the rows),
  // each sequence's pages in position order, and the free pages
  int32_t *page_table = nullptr;
  std::vector<std::vector<int32_t>> seq_pages;
  std::vector<int32_t> free_pages;
  hipEvent_t ev[STAGE_RING];
  bool ev_used[STAGE_RING];
  int ring = 0;
  std::string err;
  // per-node timing (decoder_stats_enable)
  uint32_t stats_mask = 0;
  std::vector<hipEvent_t> tev;
  struct Pending {
    int node, ev;
    double bytes, flops;
  };
  std::vector<Pending> pend;
  int tnext = 0;
  decoder_stats_t stats{};
};

namespace {

int fail(decoder *D, int code, const std::string &msg) {
  if (D) D->err = msg;
  return code;
}

int hip_fail(decoder *D, hipError_t e, const char *where) {
  return fail(D, DEC_E_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

#define HIP_TRY(D, expr, where)                    \
  do {                                             \
    hipError_t _e = (expr);                        \
    if (_e != hipSuccess) return hip_fail(D, _e, where); \
  } while (0)

template <typename T>
T *carve(decoder *D, size_t off) {
  return reinterpret_cast<T *>(D->ws + off);
}

constexpr int TIMER_EVENTS = 8192;

int stats_harvest(decoder *D) {
  if (D->pend.empty()) return DEC_OK;
  HIP_TRY(D, hipStreamSynchronize(D->stream), "stats sync");
  for (const auto &p : D->pend) {
    float ms = 0.f;
    HIP_TRY(D, hipEventElapsedTime(&ms, D->tev[p.ev], D->tev[p.ev + 1]), "stats elapsed");
    D->stats.launches[p.node] += 1;
    D->stats.ms[p.node] += ms;
    D->stats.bytes[p.node] += p.bytes;
    D->stats.flops[p.node] += p.flops;
  }
  D->pend.clear();
  D->tnext = 0;
  return DEC_OK;
}

// Brackets the launches of one node with events while stats are enabled.
struct NodeTimer {
  decoder *D;
  int node, ev = -1;
  double bytes, flops;
  NodeTimer(decoder *D_, int node_, double bytes_, double flops_)
      : D(D_), node(node_), bytes(bytes_), flops(flops_) {
    if (!((D->stats_mask >> node) & 1u)) return;
    if (D->tnext + 2 > (int)D->tev.size() && stats_harvest(D) != DEC_OK) return;
    ev = D->tnext;
    if (hipEventRecord(D->tev[ev], D->stream) != hipSuccess) ev = -1;
  }
  ~NodeTimer() {
    if (ev < 0) return;
    if (hipEventRecord(D->tev[ev + 1], D->stream) != hipSuccess) return;
    D->pend.push_back({node, ev, bytes, flops});
    D->tnext += 2;
  }
};

// Stage rows' ids / seqs / positions to the device through a pinned slot.
int stage_rows(decoder *D, int rows, const int32_t *ids, const int32_t *seqs, const int32_t *pos) {
  const int slot = D->ring;
  D->ring = (D->ring + 1) % STAGE_RING;
  if (D->ev_used[slot]) HIP_TRY(D, hipEventSynchronize(D->ev[slot]), "stage wait");
  int32_t *h = D->pinned + (size_t)slot * D->L.stage_n;
  D->hseq.assign(seqs, seqs + rows);
  for (int r = 0; r < rows; ++r) {
    h[r] = ids ? ids[r] : 0;
    h[D->L.R + r] = seqs[r];
    h[2 * D->L.R + r] = pos[r];
  }
  if (D->L.mp) {  // the page table travels with the rows
    int32_t *t = h + 3 * D->L.R;
    for (int s = 0; s < D->c.max_batch; ++s) {
      const std::vector<int32_t> &pg = D->seq_pages[s];
      for (int j = 0; j < D->L.mp; ++j) t[(size_t)s * D->L.mp + j] = j < (int)pg.size() ? pg[j] : 0;
    }
  }
  HIP_TRY(D, hipMemcpyAsync(D->ids, h, D->L.stage_n * 4, hipMemcpyHostToDevice, D->stream), "stage copy");
  HIP_TRY(D, hipEventRecord(D->ev[slot], D->stream), "stage event");
  D->ev_used[slot] = true;
  return DEC_OK;
}

// Element offset of layer l inside a KV unit, and the page table (or null).
int64_t kv_layer_off(const decoder *D, int l) {
  return (int64_t)l * D->c.n_kv_heads * (int64_t)D->L.kvS * D->c.head_dim;
}
const int32_t *kv_pt(const decoder *D) { return D->L.mp ? D->page_table : nullptr; }

// Paged cache: give each listed sequence the pages its new length needs
// (all or nothing: a pool too small for the call launches nothing).
int ensure_pages(decoder *D, int n, const int32_t *seqs, const int32_t *new_len) {
  if (!D->L.mp) return DEC_OK;
  const int P = D->c.kv_page_size;
  size_t need = 0;
  for (int i = 0; i < n; ++i) {
    const size_t want = (size_t)(new_len[i] + P - 1) / P, have = D->seq_pages[seqs[i]].size();
    if (want > have) need += want - have;
  }
  if (need > D->free_pages.size()) return fail(D, DEC_E_CONTEXT_OVERFLOW, "KV page pool exhausted");
  for (int i = 0; i < n; ++i) {
    std::vector<int32_t> &pg = D->seq_pages[seqs[i]];
    while ((int64_t)pg.size() * P < new_len[i]) {
      pg.push_back(D->free_pages.back());
      D->free_pages.pop_back();
    }
  }
  return DEC_OK;
}

// Paged cache: return the pages of sequence s past its first keep positions.
void release_pages(decoder *D, int s, int keep) {
  if (!D->L.mp) return;
  const int P = D->c.kv_page_size;
  std::vector<int32_t> &pg = D->seq_pages[s];
  while ((int64_t)pg.size() * P >= (int64_t)keep + P) {
    D->free_pages.push_back(pg.back());
    pg.pop_back();
  }
}

// Launch one projection (plus its split-K reduction) as node `node`.  For
// EPI_LOGITS, *nparts receives the number of argmax partials per row.
int proj(decoder *D, int node, int epi, GemmArgs g, int max_rows, int *nparts = nullptr) {
  const double npd = (epi == EPI_SWIGLU || epi == EPI_QKV) ? 2.0 : 1.0;
  const double out_b = epi == EPI_ADD ? 8.0 : ((epi == EPI_SWIGLU || epi == EPI_QKV) ? 2.0 * npd : 4.0);
  const double a_b = (g.x || g.a_lo) ? 4.0 : 2.0;
  const double ncols = epi == EPI_QKV ? g.N / 2.0 : g.N;
  // int8 codes stream on the one-tile (<= 16 rows) path only; wider calls
  // read the dequantised copies.  For a batch of 8-16 rows the packed bf16
  // chunk kernel is the faster one on long rows (8B-class down projection,
  // K = 14336, 16 rows: 32 us against 41 us on codes), so those keep it.
  if (g.M > 16 || (g.M >= CHUNK_BATCH_MIN_ROWS && g.K > 8192 && g.Wp)) g.Wq = nullptr;
  const double wrow = g.Wq ? (double)g.K + 4.0 : (double)g.K * 2;
  NodeTimer timer(D, node, npd * ncols * wrow + (double)g.M * g.K * a_b + (double)g.M * ncols * out_b,
                  2.0 * npd * g.M * ncols * (double)g.K);
  const int ntiles = gemm_ntiles(g, epi);
  g.Cpart = D->gpart;
  if (epi == EPI_ADD) D->act_norm = nullptr;  // x changes
  if (g.norm_gamma) {
    g.norm_eps = (float)D->c.rms_eps;
    g.norm_out = D->act;
    g.norm_lo = D->act_lo;
  }
  // the split reduce of a residual projection also writes the next RMSNorm
  auto note_norm = [&]() {
    if (epi == EPI_ADD && g.norm_gamma && g.ksplit > 1 && g.C == D->x) {
      D->act_norm = g.norm_gamma;
      D->act_rows = g.M;
    }
  };
  if (nparts) *nparts = gemm_ntiles(g, epi);
  // 2-8 rows of bf16 weights: the multi-row GEMV streams each weight row once
  if (gemv_rows_fits(g, epi)) {
    if (nparts) *nparts = gemv_rows_grid(g, epi);
    hipError_t e = launch_gemv_rows(g, epi, D->stream);
    if (e != hipSuccess) return hip_fail(D, e, "multi-row projection");
    return DEC_OK;
  }
  const bool chunk_rows = g.M > CHUNK_MIN_ROWS ||
                          (!g.Wq && g.M >= CHUNK_BATCH_MIN_ROWS && npd * ncols * (double)g.K * 2 >= CHUNK_BATCH_MIN_BYTES);
  if (chunk_rows && gemm_chunk_fits(g, epi)) {
    // chunk kernel: split K so that the blocks (weight tiles x row blocks x
    // splits) fill the compute units about once, with at least two 64-wide k
    // steps per split (fewer, longer blocks measured faster than two rounds)
    // 256+ rows: the wide kernel (256-row blocks) where its split stays at
    // most WIDE_MAX_SPLIT (measured at 512 rows: gate_up 213 against 230 us,
    // QKV 78 against 85 with 5 splits; o_proj and down, which need 8 splits
    // there, were slower: 60.5 and 132 against 49 and 124, from the partials)
    const int tiles = gemm_chunk_tiles(g, epi);
    const int nsteps = (g.K + 63) / 64;
    auto split_for = [&](int nbt) {
      int kc = std::max(1, D->cus / nbt);
      kc = std::min(std::min(kc, CHUNK_MAX_SPLIT), std::max(1, nsteps / 2));
      while (kc > 1 && (size_t)kc * g.M * (size_t)npd * ntiles * 16 > D->L.gpart_elems) --kc;
      return kc;
    };
    int kc = 1;
    g.wide = 0;
    if (epi != EPI_LOGITS) {
      const int kw = split_for(tiles * gemm_wide_mblocks(g.M));
      g.ksplit = kw;
      if (g.M >= GEMM_WIDE_MIN_ROWS && kw <= WIDE_MAX_SPLIT && gemm_wide_takes(g, epi)) {
        g.wide = 1;
        kc = kw;
      } else {
        kc = split_for(tiles * gemm_chunk_mblocks(g.M));
      }
    }
    g.ksplit = kc;
    if (g.ksplit <= 1) g.norm_out = nullptr;
    hipError_t e = launch_gemm_chunk(g, epi, D->stream);
    if (e != hipSuccess) return hip_fail(D, e, "chunk projection");
    note_norm();
    return DEC_OK;
  }
  const int steps = (g.K + 31) / 32;
  int ks = 1;
  if (epi != EPI_LOGITS && !g.n_groups && ntiles < 192 && steps >= 16) {
    ks = std::min(GEMM_MAX_SPLIT, std::max(1, 384 / ntiles));
    ks = std::min(ks, steps / 8);
  }
  // a residual projection of a batch on int8 codes splits K in two, so its
  // reduce also writes the next RMSNorm (the fused prologue cannot hold
  // 8-16 rows of a wide activation), which saves that norm's own launch
  if (g.Wq && epi == EPI_ADD && g.norm_gamma && g.M >= CHUNK_BATCH_MIN_ROWS && steps >= 16) ks = std::max(ks, 2);
  while (ks > 1 && (size_t)ks * g.M * (size_t)npd * ntiles * 16 > D->L.gpart_elems) --ks;
  g.ksplit = std::max(ks, 1);
  if (g.ksplit <= 1 || g.n_groups) g.norm_out = nullptr;
  hipError_t e = launch_gemm(g, epi, max_rows, 1, D->stream);
  if (e != hipSuccess) return hip_fail(D, e, "projection");
  if (g.norm_out) note_norm();
  return DEC_OK;
}

// With int8 weights, the multi-row projection of a decode batch or a verify
// pass (<= 16 rows) streams the codes of matrix i of layer l (as quant());
// 4-bit weights keep the dequantised copies on this path.
GemmArgs qcodes(const decoder *D, GemmArgs g, int l, int i) {
  if (D->c.weight_quant != 1) return g;
  const decoder::QuantW &w = l < 0 ? D->qhead : D->qw[l][i];
  g.Wq = w.q;
  g.wscale = w.s;
  return g;
}

GemmArgs dense_args(const uint16_t *A, int64_t lda, const uint16_t *W, int M, int N, int K) {
  GemmArgs g{};
  g.A = A;
  g.lda = lda;
  g.W = W;
  g.M = M;
  g.N = N;
  g.K = K;
  g.np_off = N;
  return g;
}

// RMSNorm of x rows into the projection's A operand: fused into the
// projection prologue for decode-size row counts, else a separate kernel.
int norm_into(decoder *D, GemmArgs &g, const float *x, const float *gamma, int rows) {
  const int H = D->c.hidden;
  // fused into the projection's prologue: decode-size row counts of the
  // one-tile GEMM, and the 2-8 rows of the multi-row GEMV (bf16 weights)
  if (gemm_norm_fits(rows, H) || (D->c.weight_quant != 1 && gemv_rows_takes(rows, H))) {
    g.x = x;
    g.gamma = gamma;
    g.eps = (float)D->c.rms_eps;
    g.lda = H;
    g.A = nullptr;
    return DEC_OK;
  }
  if (x == D->x && gamma == D->act_norm && rows == D->act_rows) {
    // the previous residual projection's reduce already wrote it
    g.A = D->act;
    g.a_lo = D->act_lo;
    g.lda = H;
    return DEC_OK;
  }
  hipError_t e;
  {
    NodeTimer t(D, DEC_NODE_NORM, rows * (double)H * 6 + H * 4.0, rows * (double)H * 4);
    e = launch_rmsnorm(x, H, gamma, rows, H, (float)D->c.rms_eps, D->act, H, D->act_lo, D->stream);
  }
  if (e != hipSuccess) return hip_fail(D, e, "rmsnorm");
  g.A = D->act;
  g.a_lo = D->act_lo;
  g.lda = H;
  return DEC_OK;
}

// The arrival counters of the fused launches (cumulative, never reset),
// SYNC_STRIDE words apart from sync_cnt_off on: counter l is layer l's
// output projection's, counters n_layers + GV_NCNT l + i the dense FFN's of
// layer l; sync_base(D)[j] is counter j's value when the current step began.
uint32_t *sync_base(decoder *D) { return reinterpret_cast<uint32_t *>(D->attn_cnt + ATTN_MAX_TASKS + 1); }
uint32_t *sync_cnt(decoder *D) { return reinterpret_cast<uint32_t *>(D->attn_cnt + sync_cnt_off(D->c)); }

// wo (batch-1 decode, bf16 weights): the output projection x += wo . o runs
// inside the attention launch where the kernel takes it; *o_fused says
// whether it did (otherwise the caller launches it).
int attention(decoder *D, int layer, int rows, int rows_per_group, int max_pos, const int32_t *hpos,
              float *out_f32 = nullptr, const uint16_t *wo = nullptr, bool *o_fused = nullptr) {
  const decoder_config_t &c = D->c;
  const int W = c.sliding_window;
  double kv_rows = 0, qk = 0;
  for (int r = 0; r < rows; ++r) {
    const double seen = W > 0 ? std::min(hpos[r] + 1, W) : hpos[r] + 1.0;
    qk += seen;
    if (rows_per_group == 1) kv_rows += seen;
  }
  if (rows_per_group != 1) kv_rows = W > 0 ? std::min(max_pos + 1, W + rows) : max_pos + 1.0;
  NodeTimer timer(D, DEC_NODE_ATTN,
                  kv_rows * c.n_kv_heads * c.head_dim * 4.0 + (double)rows * c.n_heads * c.head_dim * 4.0,
                  qk * c.n_heads * c.head_dim * 4.0);
  AttnArgs a{};
  a.q = D->q;
  a.q_lo = D->q_lo;
  a.out = out_f32 ? nullptr : D->attn;
  a.out_lo = D->attn_lo;
  a.out_f32 = out_f32;
  a.kcache = D->kcache;
  a.vcache = D->vcache;
  a.row_seq = D->row_seq;
  a.row_pos = D->row_pos;
  a.seq_stride = D->L.kv_unit;
  a.layer_off = kv_layer_off(D, layer);
  a.S = D->L.kvS;
  a.pt = kv_pt(D);
  a.mp = D->L.mp;
  a.Hq = c.n_heads;
  a.Hkv = c.n_kv_heads;
  a.G = c.n_heads / c.n_kv_heads;
  a.rows = rows;
  a.rows_per_group = rows_per_group;
  a.n_groups = (rows + rows_per_group - 1) / rows_per_group * c.n_kv_heads;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));
  a.scale = (float)(1.0 / std::sqrt((double)c.head_dim));
  a.window = W;
  a.softcap = (float)c.attn_softcap;
  a.sinks = D->layers[layer].attn_sinks;
  a.part_o = D->part_o;
  a.part_ml = D->part_ml;
  a.counters = nullptr;  // set below once the split count is known
  // positions as kernel arguments where the host has them in a usable form
  if (rows_per_group == 1 && rows <= 16 && (int)D->hseq.size() == rows && !D->graph_mode) {
    a.pos_mode = 1;
    for (int r = 0; r < rows; ++r) {
      a.pos_arg[r] = hpos[r];
      a.seq_arg[r] = D->hseq[r];
    }
  } else if (rows_per_group > 1 && (int)D->hseq.size() == rows) {
    // a prefill chunk: one sequence, consecutive positions
    a.pos_mode = 2;
    a.pos0 = hpos[0];
    a.seq0 = D->hseq[0];
    for (int r = 1; r < rows; ++r)
      if (hpos[r] != hpos[0] + r || D->hseq[r] != a.seq0) a.pos_mode = 0;
  }
  // split the keys so that about ATTN_TARGET_BLOCKS blocks run, each at
  // least one 32-key tile per wave; with a window (position modes 1 and 2)
  // a group's keys start at its window, so they span at most its rows, the
  // window and the 32-key alignment
  int keys = max_pos + 1;
  if (W > 0 && a.pos_mode != 0) keys = std::min(keys, W + rows_per_group + 31);
  int ns = std::max(1, (ATTN_TARGET_BLOCKS + a.n_groups - 1) / a.n_groups);
  int kc = (int)align_up((size_t)((keys + ns - 1) / ns), 128);
  ns = (keys + kc - 1) / kc;
  while ((int64_t)a.n_groups * ns > ATTN_MAX_TASKS && ns > 1) {
    kc *= 2;
    ns = (keys + kc - 1) / kc;
  }
  if ((int64_t)a.n_groups * ns > ATTN_MAX_TASKS) return fail(D, DEC_E_INVALID, "attention work list too long");
  a.kc = kc;
  a.n_splits = ns;
  // the group's last block merges the splits (counters zero again after
  // every launch) when a group holds at most two values per thread, at most
  // ATTN_FUSED_MAX_SPLITS splits and at most 256 (split, column) pairs;
  // otherwise the merge is its own launch
  const int ncols = std::min(16, rows_per_group * a.G);
  if (ncols * c.head_dim <= 512 && ns <= ATTN_FUSED_MAX_SPLITS && ns * ncols <= 256) a.counters = D->attn_cnt;
  // the chunk kernel shares each key tile among up to 128 query columns; a
  // chunk that fits one column group per kv head (a verify pass of a few
  // drafted rows) takes the decode kernel, whose waves each own a tile
  const bool chunk_kernel = rows > rows_per_group && attention_chunk_fits(a, c.head_dim);
  const int qd = c.n_heads * c.head_dim;
  if (o_fused) *o_fused = false;
  if (wo && o_fused && D->fuse_o && !chunk_kernel && a.pos_mode != 2 && rows == 1 && out_f32 && a.counters &&
      qd <= ATTN_O_MAX_K) {
    const int H = c.hidden;
    a.wo = wo;
    a.o_x = D->x;
    a.o_rows = H;
    a.o_blocks = (H + 4 * ATTN_O_RPW - 1) / (4 * ATTN_O_RPW);
    a.o_done = sync_cnt(D) + (int64_t)layer * SYNC_STRIDE;
    a.o_base = sync_base(D) + layer;
    D->act_norm = nullptr;  // x changes
    timer.bytes += (double)H * qd * 2 + (double)qd * 4 + (double)H * 8;
    timer.flops += 2.0 * H * qd;
    *o_fused = true;
  }
  hipError_t e = chunk_kernel ? launch_attention_chunk(a, c.head_dim, D->stream)
                              : launch_attention(a, c.head_dim, D->stream);
  if (e != hipSuccess) return hip_fail(D, e, "attention");
  return DEC_OK;
}

// Launch one batch-1 projection (GEMV) as node `node`.
int gemv(decoder *D, int node, int epi, const GemvArgs &g, int *blocks = nullptr) {
  if (epi == EPI_ADD || epi == EPI_MOE_ADD) D->act_norm = nullptr;  // x changes
  const double nr = (epi == EPI_SWIGLU || epi == EPI_QKV) ? 2.0 : 1.0;
  const double slots = (g.slot_expert || g.route_logits) ? g.n_slots : 1;
  const double out_words = epi == EPI_ADD ? 2 : epi == EPI_MOE_ADD ? 2 + g.moe_k : 1;
  // weight bytes per row (+ its scale or group exponents)
  const double wrow = g.qbits == 8 ? (double)g.K + 4.0 : g.qbits == 4 ? g.K / 2.0 + g.K / 32.0 : (double)g.K * 2;
  const double part2 = g.W2 ? g.n_items2 * (nr * wrow + 4.0) : 0.0;
  NodeTimer timer(D, node,
                  slots * (nr * g.n_items * wrow + g.K * 4.0 + g.n_items * 4.0 * out_words) + part2,
                  slots * 2.0 * nr * g.n_items * (double)g.K + (g.W2 ? 2.0 * nr * g.n_items2 * (double)g.K : 0.0));
  hipError_t e = launch_gemv(g, epi, D->stream, blocks);
  if (e != hipSuccess) return hip_fail(D, e, "gemv");
  return DEC_OK;
}

// With quantised weights, GEMVs stream the int8 codes (and row scales) of
// matrix i of layer l (i: 0 qkv, 1 o, 2 gate_up, 3 down; l < 0: the lm-head).
GemvArgs quant(const decoder *D, GemvArgs g, int l, int i) {
  if (!D->c.weight_quant) return g;
  const decoder::QuantW &w = l < 0 ? D->qhead : D->qw[l][i];
  g.Wq = w.q;
  g.wscale = w.s;
  g.wexp = w.e;
  g.qbits = D->c.weight_quant == 2 ? 4 : 8;
  return g;
}

GemvArgs gemv_args(const uint16_t *W, const float *a, int K, int n_items, float *C) {
  GemvArgs g{};
  g.W = W;
  g.a_f32 = a;
  g.K = K;
  g.N = n_items;
  g.n_items = n_items;
  g.C = C;
  return g;
}

// With per-head QK-norm the QKV projection stores its raw output (bias
// added) in D->qkv, and this pass norms each q and k head, rotates, stores
// q and appends K and V (the fused QKV epilogue cannot: one head's outputs
// come from many waves).
int qk_norm_pass(decoder *D, int l, int rows) {
  const decoder_config_t &c = D->c;
  const decoder_layer_weights_t &W = D->layers[l];
  const int d = c.head_dim;
  const int qkvr = (c.n_heads + 2 * c.n_kv_heads) * d;
  NodeTimer t(D, DEC_NODE_ROPE, rows * (double)qkvr * 8.0, rows * (double)qkvr * 6.0);
  QkNormArgs a{};
  a.qkv = D->qkv;
  a.ld = qkvr;
  a.q_norm = W.q_norm;
  a.k_norm = W.k_norm;
  a.eps = (float)c.rms_eps;
  a.cs = D->rope;
  a.row_seq = D->row_seq;
  a.row_pos = D->row_pos;
  a.q = D->q;
  a.q_lo = D->q_lo;
  a.kcache = D->kcache;
  a.vcache = D->vcache;
  a.seq_stride = D->L.kv_unit;
  a.layer_off = kv_layer_off(D, l);
  a.S = D->L.kvS;
  a.pt = kv_pt(D);
  a.mp = D->L.mp;
  a.Hq = c.n_heads;
  a.Hkv = c.n_kv_heads;
  a.d = d;
  a.rows = rows;
  hipError_t e = launch_qk_norm_rope(a, D->stream);
  if (e != hipSuccess) return hip_fail(D, e, "qk norm");
  return DEC_OK;
}

// One decode row: every projection is a GEMV over fp32 activations.
int run_layer_single(decoder *D, int l, int max_pos, const int32_t *hpos) {
  const decoder_config_t &c = D->c;
  const decoder_layer_weights_t &W = D->layers[l];
  const int H = c.hidden, d = c.head_dim, qd = c.n_heads * d;
  const float eps = (float)c.rms_eps;
  int rc;
  hipError_t e;

  if (c.qk_norm) {
    GemvArgs qs = gemv_args(W.w_qkv, D->x, H, (c.n_heads + 2 * c.n_kv_heads) * d, D->qkv);
    qs.gamma = W.attn_norm;
    qs.eps = eps;
    qs.bias = c.qkv_bias ? W.b_qkv : nullptr;
    if ((rc = gemv(D, DEC_NODE_QKV, EPI_STORE, quant(D, qs, l, 0)))) return rc;
    if ((rc = qk_norm_pass(D, l, 1))) return rc;
  }
  GemvArgs q = gemv_args(W.w_qkv, D->x, H, (c.n_heads + 2 * c.n_kv_heads) * d / 2, nullptr);
  q.gamma = W.attn_norm;
  q.eps = eps;
  q.qkv.bias = c.qkv_bias ? W.b_qkv : nullptr;
  q.qkv.cs = D->rope;
  if (D->hseq.size() == 1 && !D->graph_mode) {  // the position as a kernel argument: no load before RoPE
    q.qkv.pos_arg = hpos[0];
    q.qkv.seq_arg = D->hseq[0];
  } else {
    q.qkv.row_seq = D->row_seq;
    q.qkv.row_pos = D->row_pos;
  }
  q.qkv.q = D->q;
  q.qkv.q_lo = D->q_lo;
  q.qkv.kcache = D->kcache;
  q.qkv.vcache = D->vcache;
  q.qkv.seq_stride = D->L.kv_unit;
  q.qkv.layer_off = kv_layer_off(D, l);
  q.qkv.S = D->L.kvS;
  q.qkv.pt = kv_pt(D);
  q.qkv.mp = D->L.mp;
  q.qkv.P = D->L.kvS;
  q.qkv.Hq = c.n_heads;
  q.qkv.Hkv = c.n_kv_heads;
  q.qkv.d = d;
  if (!c.qk_norm && (rc = gemv(D, DEC_NODE_QKV, EPI_QKV, quant(D, q, l, 0)))) return rc;
  bool o_fused = false;
  if ((rc = attention(D, l, 1, 1, max_pos, hpos, D->f32_attn, D->c.weight_quant ? nullptr : W.w_o, &o_fused)))
    return rc;
  if (!o_fused && (rc = gemv(D, DEC_NODE_O, EPI_ADD, quant(D, gemv_args(W.w_o, D->f32_attn, qd, H, D->x), l, 1))))
    return rc;
  if (l == D->stop_mid_layer) return DEC_OK;

  if (c.n_experts == 0) {
    const int I = c.ffn_inter;
    GemvArgs gu = gemv_args(W.w_gate_up, D->x, H, I, D->f32_h);
    gu.gamma = W.ffn_norm;
    gu.eps = eps;
    const GemvArgs dn = gemv_args(W.w_down, D->f32_h, I, H, D->x);
    if (D->fuse_ffn && !c.weight_quant && gemv_ffn_fits(gu, dn)) {
      // one launch: the down blocks wait for the gate/up blocks' arrivals
      D->act_norm = nullptr;  // x changes
      NodeTimer timer(D, DEC_NODE_GATE_UP,
                      2.0 * I * H * 2.0 + H * 4.0 + I * 4.0 + H * I * 2.0 + I * 4.0 + H * 8.0,
                      2.0 * 2.0 * I * (double)H + 2.0 * H * (double)I);
      const int j = c.n_layers + GV_NCNT * l;
      const hipError_t e =
          launch_gemv_ffn(gu, dn, sync_cnt(D) + (int64_t)j * SYNC_STRIDE, sync_base(D) + j, D->stream);
      if (e != hipSuccess) return hip_fail(D, e, "fused FFN");
      return DEC_OK;
    }
    if ((rc = gemv(D, DEC_NODE_GATE_UP, EPI_SWIGLU, quant(D, gu, l, 2)))) return rc;
    return gemv(D, DEC_NODE_DOWN, EPI_ADD, quant(D, dn, l, 3));
  }
  // MoE FFN for one row: the FFN RMSNorm runs inside the router GEMV and the
  // expert GEMVs (each from x).  The routed gate/up launch routes by itself
  // (each block takes the top-k of the router logits) and publishes the ids,
  // weights and shared gate; the shared expert's down projection also does
  // the combine into x.  (The router GEMV spreads the router rows over many
  // compute units; one block computing all the logits and routing, as the
  // multi-row path does, measured slower for a single row: 13.4 us against
  // 2 x 5.8 us for the router GEMV and a route kernel.)
  const int E = c.n_experts, k = c.top_k, Ie = c.expert_inter, Is = c.shared_inter;
  GemvArgs rg = gemv_args(W.w_router, D->x, H, E, D->rlogits);
  rg.gamma = W.ffn_norm;
  rg.eps = eps;
  if ((rc = gemv(D, DEC_NODE_ROUTER, EPI_STORE, rg))) return rc;
  // routed gate_up (k slots) and, in the same launch, the shared expert's
  GemvArgs eg = gemv_args(W.w_exp_gate_up, D->x, H, Ie, D->f32_hexp);
  eg.gamma = W.ffn_norm;
  eg.eps = eps;
  eg.route_logits = D->rlogits;
  eg.route_E = E;
  eg.route_renorm = c.norm_topk_prob;
  eg.route_ids = D->rids;
  eg.route_rec = D->rids_rec + (size_t)l * k;
  eg.route_wts = D->rwts;
  eg.route_gate = D->rgate;
  eg.route_w_sg = (Is > 0 && c.shared_gate) ? W.w_sh_gate : nullptr;
  eg.n_slots = k;
  eg.w_group_stride = (int64_t)2 * Ie * H;
  eg.ldc = Ie;
  if (Is > 0) {
    eg.W2 = W.w_sh_gate_up;
    eg.N2 = Is;
    eg.n_items2 = Is;
    eg.C2 = D->f32_h;
  }
  eg = quant(D, eg, l, 4);
  if (c.weight_quant && Is > 0) {
    eg.W2q = D->qw[l][2].q;
    eg.w2scale = D->qw[l][2].s;
    eg.w2exp = D->qw[l][2].e;
  }
  if ((rc = gemv(D, DEC_NODE_EXPERTS, EPI_SWIGLU, eg))) return rc;
  GemvArgs ed = gemv_args(W.w_exp_down, D->f32_hexp, Ie, H, D->yexp);
  ed.slot_expert = D->rids;
  ed.n_slots = k;
  ed.w_group_stride = (int64_t)H * Ie;
  ed.a_slot_stride = Ie;
  ed.ldc = H;
  if ((rc = gemv(D, DEC_NODE_EXPERTS, EPI_STORE, quant(D, ed, l, 5)))) return rc;
  if (Is > 0) {
    GemvArgs sd = gemv_args(W.w_sh_down, D->f32_h, Is, H, D->x);
    sd.moe_y = D->yexp;
    sd.moe_w = D->rwts;
    sd.moe_gate = D->rgate;
    sd.moe_k = k;
    return gemv(D, DEC_NODE_EXPERTS, EPI_MOE_ADD, quant(D, sd, l, 3));
  }
  NodeTimer tcomb(D, DEC_NODE_EXPERTS, H * (8.0 + 4.0 * k + 4.0), H * 2.0 * (k + 1));
  D->act_norm = nullptr;
  e = launch_moe_combine(D->x, D->yexp, Is > 0 ? D->ysh : nullptr, D->rwts, D->rgate, nullptr, 1, k, H, D->stream);
  if (e != hipSuccess) return hip_fail(D, e, "moe combine");
  return DEC_OK;
}

int run_layer(decoder *D, int l, int rows, int rows_per_group, int max_pos, const int32_t *hpos) {
  if (rows == 1 && D->single_row_ok) return run_layer_single(D, l, max_pos, hpos);
  const decoder_config_t &c = D->c;
  const decoder_layer_weights_t &W = D->layers[l];
  const int H = c.hidden, d = c.head_dim, qd = c.n_heads * d;
  const int qkvr = (c.n_heads + 2 * c.n_kv_heads) * d;
  hipStream_t st = D->stream;
  int rc;
  hipError_t e;

  // RMSNorm -> QKV (+bias) -> RoPE -> KV append, one projection launch
  GemmArgs q = dense_args(nullptr, H, W.w_qkv, rows, qkvr, H);
  if ((rc = norm_into(D, q, D->x, W.attn_norm, rows))) return rc;
  q.np_off = d / 2;
  q.qkv.bias = c.qkv_bias ? W.b_qkv : nullptr;
  q.qkv.cs = D->rope;
  if (D->hseq.size() == 1 && !D->graph_mode) {  // the position as a kernel argument: no load before RoPE
    q.qkv.pos_arg = hpos[0];
    q.qkv.seq_arg = D->hseq[0];
  } else {
    q.qkv.row_seq = D->row_seq;
    q.qkv.row_pos = D->row_pos;
  }
  q.qkv.q = D->q;
  q.qkv.q_lo = D->q_lo;
  q.qkv.kcache = D->kcache;
  q.qkv.vcache = D->vcache;
  q.qkv.seq_stride = D->L.kv_unit;
  q.qkv.layer_off = kv_layer_off(D, l);
  q.qkv.S = D->L.kvS;
  q.qkv.pt = kv_pt(D);
  q.qkv.mp = D->L.mp;
  q.qkv.P = D->L.kvS;
  q.qkv.Hq = c.n_heads;
  q.qkv.Hkv = c.n_kv_heads;
  q.qkv.d = d;
  q.Wp = D->packed[l].w[0];
  q = qcodes(D, q, l, 0);
  if (c.qk_norm) {
    // plain projection (bias added) into D->qkv, then the per-head norm pass
    q.np_off = qkvr;
    q.bias = c.qkv_bias ? W.b_qkv : nullptr;
    q.C = D->qkv;
    q.ldc = qkvr;
    if ((rc = proj(D, DEC_NODE_QKV, EPI_STORE, q, rows))) return rc;
    if ((rc = qk_norm_pass(D, l, rows))) return rc;
  } else if ((rc = proj(D, DEC_NODE_QKV, EPI_QKV, q, rows))) {
    return rc;
  }
  if ((rc = attention(D, l, rows, rows_per_group, max_pos, hpos))) return rc;
  GemmArgs o = dense_args(D->attn, qd, W.w_o, rows, H, qd);
  o.Wp = D->packed[l].w[1];
  o = qcodes(D, o, l, 1);
  o.norm_gamma = W.ffn_norm;
  o.a_lo = D->attn_lo;
  o.C = D->x;
  o.ldc = H;
  if ((rc = proj(D, DEC_NODE_O, EPI_ADD, o, rows))) return rc;
  if (l == D->stop_mid_layer) return DEC_OK;

  if (c.n_experts == 0) {
    const int I = c.ffn_inter;
    GemmArgs gu = dense_args(nullptr, H, W.w_gate_up, rows, I, H);
    if ((rc = norm_into(D, gu, D->x, W.ffn_norm, rows))) return rc;
    gu.Hout = D->h;
    gu.h_lo = D->h_lo;
    gu.ldc = I;
    gu.Wp = D->packed[l].w[2];
    gu = qcodes(D, gu, l, 2);
    if ((rc = proj(D, DEC_NODE_GATE_UP, EPI_SWIGLU, gu, rows))) return rc;
    GemmArgs dn = dense_args(D->h, I, W.w_down, rows, H, I);
    dn.Wp = D->packed[l].w[3];
    dn = qcodes(D, dn, l, 3);
    if (l + 1 < c.n_layers) dn.norm_gamma = (const float *)D->layers[l + 1].attn_norm;
    dn.a_lo = D->h_lo;
    dn.C = D->x;
    dn.ldc = H;
    return proj(D, DEC_NODE_DOWN, EPI_ADD, dn, rows);
  }

  // routed experts + shared expert: the router, the shared gate and the
  // experts all read the same normed input b (bf16 in D->act)
  {
    NodeTimer t(D, DEC_NODE_NORM, rows * (double)H * 6 + H * 4.0, rows * (double)H * 4);
    e = (D->act_norm == (const float *)W.ffn_norm && D->act_rows == rows)
            ? hipSuccess
            : launch_rmsnorm(D->x, H, W.ffn_norm, rows, H, (float)c.rms_eps, D->act, H, D->act_lo, st);
  }
  if (e != hipSuccess) return hip_fail(D, e, "rmsnorm");
  const int E = c.n_experts, k = c.top_k, Ie = c.expert_inter, Is = c.shared_inter;
  // router logits, top-k and the shared gate in one launch (from x, normed
  // in fp32), then the grouping of (row, expert) pairs
  MoeRouteArgs mr{};
  mr.w_router = W.w_router;
  mr.logits_out = D->rlogits;
  mr.act_f32 = D->x;
  mr.gamma = W.ffn_norm;
  mr.eps = (float)c.rms_eps;
  mr.w_sh_gate = (Is > 0 && c.shared_gate) ? W.w_sh_gate : nullptr;
  mr.rows = rows;
  mr.E = E;
  mr.k = k;
  mr.H = H;
  mr.renorm = c.norm_topk_prob;
  mr.ids = D->rids;
  mr.wts = D->rwts;
  mr.gate = D->rgate;
  mr.ids_record = D->rids_rec + (size_t)l * rows * k;
  // a prefill chunk: the grouped form of the chunk kernel on the packed
  // expert weights (32-row tiles of the groups' pairs), with the shared
  // expert as S pseudo-experts when it divides into experts
  const bool packed = rows > CHUNK_MIN_ROWS && D->packed[l].w[4] && D->packed[l].w[5];
  const int GS = E + moe_shared_parts(&c);  // group table slots
  const int S = packed ? moe_shared_parts(&c) : 0;
  mr.n_groups = D->groups;
  mr.group_expert = D->groups + 1;
  mr.group_start = D->groups + 1 + GS;
  mr.group_count = D->groups + 1 + 2 * GS;
  mr.pair_row = D->pair_row;
  mr.pair_of = D->pair_of;
  mr.extra_groups = S;
  mr.arrive = D->attn_cnt + ATTN_MAX_TASKS;  // the router's arrival counter
  {
    NodeTimer t(D, DEC_NODE_ROUTER, E * (double)H * 2 + rows * (double)H * 4 + rows * (double)E * 4,
                rows * (double)E * H * 2 + rows * (double)E * 8);
    e = launch_moe_route(mr, true, st);
  }
  if (e != hipSuccess) return hip_fail(D, e, "moe_route");
  const int slots = std::min(E, rows * k);
  const int grp_rows = std::min(rows, 32);
  const double exp_bytes = (double)(slots + S) * 3.0 * Ie * H, kp = k + S;
  GemmArgs g = dense_args(D->act, H, W.w_exp_gate_up, rows * k, Ie, H);
  g.a_lo = D->act_lo;
  g.a_rows = D->pair_row;
  g.w_group_stride = (int64_t)2 * Ie * H;
  g.Hout = D->hexp;
  g.h_lo = D->hexp_lo;
  g.ldc = Ie;
  g.n_groups = mr.n_groups;
  g.group_expert = mr.group_expert;
  g.group_start = mr.group_start;
  g.group_count = mr.group_count;
  g.ksplit = 1;
  if (rows <= 16) g = qcodes(D, g, l, 4);
  const double exp_wb = g.Wq ? 1.0 : 2.0;  // weight bytes per expert weight streamed
  {
    NodeTimer t(D, DEC_NODE_EXPERTS, exp_bytes * exp_wb * 2.0 / 3.0 + rows * (double)H * 2 + rows * kp * Ie * 2,
                2.0 * rows * kp * 2.0 * Ie * H);
    if (packed) {
      g.Wp = D->packed[l].w[4];
      e = launch_gemm_chunk_grouped(g, EPI_SWIGLU, rows * (k + S), slots + S, st);
    } else {
      e = launch_gemm(g, EPI_SWIGLU, grp_rows, slots, st);
    }
  }
  if (e != hipSuccess) return hip_fail(D, e, "moe gate_up");
  g.A = D->hexp;
  g.a_lo = D->hexp_lo;
  g.a_rows = nullptr;
  g.lda = Ie;
  g.W = W.w_exp_down;
  if (g.Wq) g = qcodes(D, g, l, 5);
  g.w_group_stride = (int64_t)H * Ie;
  g.N = H;
  g.K = Ie;
  g.np_off = H;
  g.Hout = nullptr;
  g.C = D->yexp;
  g.ldc = H;
  {
    NodeTimer t(D, DEC_NODE_EXPERTS, exp_bytes * exp_wb / 3.0 + rows * kp * Ie * 2 + rows * kp * H * 4,
                2.0 * rows * kp * (double)Ie * H);
    if (packed) {
      g.Wp = D->packed[l].w[5];
      e = launch_gemm_chunk_grouped(g, EPI_STORE, rows * (k + S), slots + S, st);
    } else {
      e = launch_gemm(g, EPI_STORE, grp_rows, slots, st);
    }
  }
  if (e != hipSuccess) return hip_fail(D, e, "moe down");
  if (Is > 0 && S == 0) {
    GemmArgs sg = dense_args(D->act, H, W.w_sh_gate_up, rows, Is, H);
    sg.a_lo = D->act_lo;
    sg.Hout = D->hsh;
    sg.h_lo = D->hsh_lo;
    sg.ldc = Is;
    sg.Wp = D->packed[l].w[2];
    sg = qcodes(D, sg, l, 2);
    if ((rc = proj(D, DEC_NODE_EXPERTS, EPI_SWIGLU, sg, rows))) return rc;
    GemmArgs sd = dense_args(D->hsh, Is, W.w_sh_down, rows, H, Is);
    sd.a_lo = D->hsh_lo;
    sd.Wp = D->packed[l].w[3];
    sd = qcodes(D, sd, l, 3);
    sd.C = D->ysh;
    sd.ldc = H;
    if ((rc = proj(D, DEC_NODE_EXPERTS, EPI_STORE, sd, rows))) return rc;
  }
  NodeTimer tcomb(D, DEC_NODE_EXPERTS, rows * (double)H * (8.0 + 4.0 * k + 4.0), rows * (double)H * 2 * (k + 1));
  D->act_norm = nullptr;
  if (S > 0)  // the shared expert's S partial outputs follow the routed pairs
    e = launch_moe_combine(D->x, D->yexp, D->yexp + (size_t)rows * k * H, D->rwts, D->rgate, D->pair_of, rows, k,
                           H, st, S, (int64_t)rows * H);
  else
    e = launch_moe_combine(D->x, D->yexp, Is > 0 ? D->ysh : nullptr, D->rwts, D->rgate, D->pair_of, rows, k, H,
                           st);
  if (e != hipSuccess) return hip_fail(D, e, "moe combine");
  return DEC_OK;
}

// Embedding, all layers, then (optionally) final norm + lm-head + argmax on
// rows [first, first + nout).
int run_step(decoder *D, int rows, int rows_per_group, int max_pos, const int32_t *hpos, int use_next,
             int first, int nout, float *d_logits, int32_t *d_argmax, int argmax_rows) {
  const decoder_config_t &c = D->c;
  hipStream_t st = D->stream;
  hipError_t e;
  {
    NodeTimer t(D, DEC_NODE_EMBED, rows * (double)c.hidden * 6, 0);
    D->act_norm = nullptr;
    e = launch_embed(D->embed, D->ids, D->next_token, D->row_seq, use_next, rows, c.hidden, D->x, sync_cnt(D),
                     sync_base(D), n_sync(c), SYNC_STRIDE, st);
  }
  if (e != hipSuccess) return hip_fail(D, e, "embed");
  const int nl = D->layer_limit >= 0 ? std::min(D->layer_limit, c.n_layers) : c.n_layers;
  D->stop_mid_layer = D->stop_after_attn ? nl - 1 : -1;
  for (int l = 0; l < nl; ++l) {
    int rc = run_layer(D, l, rows, rows_per_group, max_pos, hpos);
    if (rc) return rc;
  }
  D->last_rows = rows;
  if (nout <= 0) return DEC_OK;
  // final RMSNorm + lm-head + greedy argmax (pipeline.rs lm_head_forward;
  // decoder.rs folded lm-head + argmax: only the token id has to leave the GPU)
  const int H = c.hidden;
  float *out = d_logits ? d_logits : D->logits;
  int nparts, rc;
  if (nout == 1 && D->single_row_ok) {
    GemvArgs g = gemv_args(D->lm_head, D->x + (size_t)first * H, H, c.vocab, out);
    g.gamma = D->final_norm;
    g.eps = (float)c.rms_eps;
    g.part_val = D->am_val;
    g.part_idx = D->am_idx;
    if ((size_t)gemv_blocks(c.vocab) > D->am_cap) return fail(D, DEC_E_HIP, "lm-head grid exceeds the argmax partial buffer");
    if ((rc = gemv(D, DEC_NODE_HEAD, EPI_LOGITS, quant(D, g, -1, 0), &nparts))) return rc;
  } else {
    GemmArgs g = dense_args(nullptr, H, D->lm_head, nout, c.vocab, H);
    g = qcodes(D, g, -1, 0);
    if ((rc = norm_into(D, g, D->x + (size_t)first * H, D->final_norm, nout))) return rc;
    g.C = out;
    g.ldc = c.vocab;
    g.am.part_val = D->am_val;
    g.am.part_idx = D->am_idx;
    if ((rc = proj(D, DEC_NODE_HEAD, EPI_LOGITS, g, nout, &nparts))) return rc;
  }
  {
    NodeTimer t(D, DEC_NODE_HEAD, nout * (double)nparts * 8, 0);
    e = launch_argmax_finalize(D->am_val, D->am_idx, nparts, nout, D->am_out, D->next_token, D->row_seq + first, st);
  }
  if (e != hipSuccess) return hip_fail(D, e, "argmax");
  if (d_argmax) {
    const int a0 = nout - argmax_rows;
    HIP_TRY(D, hipMemcpyAsync(d_argmax, D->am_out + a0, (size_t)argmax_rows * 4, hipMemcpyDeviceToDevice, st),
            "argmax copy");
  }
  return DEC_OK;
}

int check_dec(const decoder *D) { return D ? DEC_OK : DEC_E_INVALID; }

}  // namespace

// ------------------------------------------------------------------ ABI --

extern "C" {

size_t decoder_workspace_bytes(const decoder_config_t *cfg) {
  if (!config_ok(cfg)) return 0;
  return make_layout(cfg).total;
}

const char *decoder_strerror(int code) {
  switch (code) {
    case DEC_OK: return "ok";
    case DEC_E_CONTEXT_OVERFLOW: return "context overflow";
    case DEC_E_INVALID: return "invalid argument";
    case DEC_E_TOKEN: return "token id out of range";
    case DEC_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case DEC_E_HIP: return "HIP runtime error";
    default: return "unknown error";
  }
}

const char *decoder_last_error(const decoder_t *dec) { return dec ? dec->err.c_str() : ""; }

int decoder_init(const decoder_config_t *cfg, const decoder_weights_t *w, void *d_workspace,
                 size_t workspace_bytes, void *stream, decoder_t **out) {
  if (!out) return DEC_E_INVALID;
  *out = nullptr;
  if (!config_ok(cfg) || !w || !w->layers || !w->embed || !w->lm_head || !w->final_norm)
    return DEC_E_INVALID;
  const Layout L = make_layout(cfg);
  if (!d_workspace || workspace_bytes < L.total || ((uintptr_t)d_workspace & 255)) return DEC_E_WORKSPACE;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const decoder_layer_weights_t &lw = w->layers[l];
    if (!lw.attn_norm || !lw.ffn_norm || !lw.w_qkv || !lw.w_o) return DEC_E_INVALID;
    if (cfg->qkv_bias && !lw.b_qkv) return DEC_E_INVALID;
    if (cfg->qk_norm && (!lw.q_norm || !lw.k_norm)) return DEC_E_INVALID;
    if (cfg->n_experts == 0 && (!lw.w_gate_up || !lw.w_down)) return DEC_E_INVALID;
    if (cfg->n_experts > 0) {
      if (!lw.w_router || !lw.w_exp_gate_up || !lw.w_exp_down) return DEC_E_INVALID;
      if (cfg->shared_inter > 0 && (!lw.w_sh_gate_up || !lw.w_sh_down)) return DEC_E_INVALID;
      if (cfg->shared_inter > 0 && cfg->shared_gate && !lw.w_sh_gate) return DEC_E_INVALID;
    }
  }
  decoder *D = new decoder();
  D->c = *cfg;
  D->L = L;
  {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      D->cus = cus;
  }
  D->layers.assign(w->layers, w->layers + cfg->n_layers);
  D->embed = w->embed;
  D->lm_head = w->lm_head;
  D->final_norm = w->final_norm;
  D->stream = (hipStream_t)stream;
  D->ws = (char *)d_workspace;
  D->kcache = carve<uint16_t>(D, L.kcache);
  D->vcache = carve<uint16_t>(D, L.vcache);
  D->rope = carve<float2>(D, L.rope);
  D->x = carve<float>(D, L.x);
  D->act = carve<uint16_t>(D, L.act);
  D->attn = carve<uint16_t>(D, L.attn);
  D->q = carve<uint16_t>(D, L.q);
  D->qkv = carve<float>(D, L.qkv);
  D->h = carve<uint16_t>(D, L.h);
  D->logits = carve<float>(D, L.logits);
  D->ids = carve<int32_t>(D, L.stage);
  D->row_seq = D->ids + L.R;
  D->row_pos = D->ids + 2 * L.R;
  D->page_table = D->ids + 3 * L.R;
  D->seq_pages.assign(cfg->max_batch, std::vector<int32_t>());
  D->free_pages.clear();
  for (int64_t p = (int64_t)L.kv_units - 1; L.mp && p >= 0; --p) D->free_pages.push_back((int32_t)p);
  D->next_token = carve<int32_t>(D, L.next_token);
  D->gout = carve<int32_t>(D, L.gout);
  D->part_o = carve<float>(D, L.part_o);
  D->part_ml = carve<float>(D, L.part_ml);
  D->attn_cnt = carve<int32_t>(D, L.attn_cnt);
  D->gpart = carve<float>(D, L.gpart);
  D->am_val = carve<float>(D, L.am_val);
  D->am_cap = L.am_n;
  D->am_idx = carve<int32_t>(D, L.am_idx);
  D->am_out = carve<int32_t>(D, L.am_out);
  D->act_lo = (int64_t)L.R * cfg->hidden;
  D->attn_lo = D->q_lo = (int64_t)L.R * cfg->n_heads * cfg->head_dim;
  D->h_lo = (int64_t)L.R * std::max(cfg->ffn_inter, 1);
  D->hexp_lo = (int64_t)L.R * (std::max(cfg->top_k, 1) + moe_shared_parts(cfg)) * std::max(cfg->expert_inter, 1);
  D->hsh_lo = (int64_t)L.R * std::max(cfg->shared_inter, 1);
  D->f32_attn = carve<float>(D, L.f32_attn);
  D->f32_h = carve<float>(D, L.f32_h);
  D->f32_act = carve<float>(D, L.f32_act);
  D->f32_hexp = carve<float>(D, L.f32_hexp);
  {
    const int qd = cfg->n_heads * cfg->head_dim;
    const int kmax = std::max(std::max(cfg->hidden, qd), std::max(std::max(cfg->ffn_inter, cfg->shared_inter),
                                                                      cfg->expert_inter));
    D->single_row_ok = gemv_lds(kmax, cfg->weight_quant == 2 ? 4 : cfg->weight_quant == 1 ? 8 : 0) <= GEMV_MAX_LDS;
  }
  if (cfg->n_experts > 0) {
    D->rlogits = carve<float>(D, L.rlogits);
    D->rids = carve<int32_t>(D, L.rids);
    D->rids_rec = carve<int32_t>(D, L.rids_rec);
    D->rwts = carve<float>(D, L.rwts);
    D->rgate = carve<float>(D, L.rgate);
    D->groups = carve<int32_t>(D, L.groups);
    D->pair_row = carve<int32_t>(D, L.pair_row);
    D->pair_of = carve<int32_t>(D, L.pair_of);
    D->hexp = carve<uint16_t>(D, L.hexp);
    D->yexp = carve<float>(D, L.yexp);
    D->hsh = carve<uint16_t>(D, L.hsh);
    D->ysh = carve<float>(D, L.ysh);
  } else {
    D->rlogits = D->rwts = D->rgate = D->yexp = D->ysh = nullptr;
    D->rids = D->rids_rec = D->groups = D->pair_row = D->pair_of = nullptr;
    D->hexp = D->hsh = nullptr;
  }
  // quantised weights: codes, scales and dequantised copies, made on the
  // stream now; every bf16 consumer then reads the dequantised copies
  if (cfg->weight_quant) {
    const QuantSpec qs = quant_spec(cfg);
    char *qp = carve<char>(D, L.quant);
    const int wq = cfg->weight_quant;
    auto quant = [&](const uint16_t *src, int64_t rows, int K, const uint16_t **dst, decoder::QuantW &qw) {
      int8_t *q = reinterpret_cast<int8_t *>(qp);
      qp += quant_piece(quant_code_bytes(wq, rows, K));
      char *sc = qp;
      qp += quant_piece(quant_scale_bytes(wq, rows, K));
      uint16_t *dq = reinterpret_cast<uint16_t *>(qp);
      qp += quant_piece((size_t)rows * K * 2);
      qw.q = q;
      *dst = dq;
      if (wq == 2) {
        int8_t *ex = reinterpret_cast<int8_t *>(sc);
        qw.e = ex;
        return launch_quantize_q4(src, rows, K, reinterpret_cast<uint8_t *>(q), ex, dq, (hipStream_t)stream) ==
               hipSuccess;
      }
      qw.s = reinterpret_cast<float *>(sc);
      return launch_quantize_rows(src, rows, K, q, reinterpret_cast<float *>(sc), dq, (hipStream_t)stream) ==
             hipSuccess;
    };
    D->qw.assign(cfg->n_layers, std::array<decoder::QuantW, 6>{});
    bool ok = quant(D->lm_head, cfg->vocab, cfg->hidden, &D->lm_head, D->qhead);
    for (int l = 0; l < cfg->n_layers && ok; ++l) {
      decoder_layer_weights_t &lw = D->layers[l];
      const bool moe = cfg->n_experts > 0;
      const uint16_t **m[QUANT_MATS] = {&lw.w_qkv, &lw.w_o, moe ? &lw.w_sh_gate_up : &lw.w_gate_up,
                                        moe ? &lw.w_sh_down : &lw.w_down, &lw.w_exp_gate_up, &lw.w_exp_down};
      for (int i = 0; i < QUANT_MATS && ok; ++i)
        if (qs.rows[i] > 0) ok = quant(*m[i], qs.rows[i], qs.K[i], m[i], D->qw[l][i]);
    }
    if (!ok) {
      D->err = "weight quantisation failed";
      delete D;
      return DEC_E_HIP;
    }
  }
  // packed weight copies for the chunk projections, made on the stream now
  {
    const PackSpec ps = pack_spec(cfg);
    uint16_t *pk = carve<uint16_t>(D, L.packed);
    D->packed.assign(cfg->n_layers, decoder::Packed{});
    for (int l = 0; l < cfg->n_layers; ++l) {
      const decoder_layer_weights_t &lw = D->layers[l];
      const uint16_t *src[PACK_MATS] = {
          (const uint16_t *)lw.w_qkv, (const uint16_t *)lw.w_o,
          (const uint16_t *)(cfg->n_experts > 0 ? lw.w_sh_gate_up : lw.w_gate_up),
          (const uint16_t *)(cfg->n_experts > 0 ? lw.w_sh_down : lw.w_down),
          (const uint16_t *)lw.w_exp_gate_up, (const uint16_t *)lw.w_exp_down};
      const int E = cfg->n_experts, S = moe_shared_parts(cfg), Ie = cfg->expert_inter, Is = cfg->shared_inter;
      const int H = cfg->hidden;
      for (int i = 0; i < PACK_MATS; ++i) {
        D->packed[l].w[i] = nullptr;
        if (!ps.rows[i] || !src[i]) continue;
        hipError_t pe;
        if (i < 4) {
          pe = launch_pack_w32(src[i], ps.rows[i], ps.K[i], pk, (hipStream_t)stream);
        } else if (i == 4) {
          // routed experts, then shared pseudo-expert j: its gate rows, its up rows
          pe = launch_pack_w32(src[i], 2 * (int64_t)E * Ie, H, pk, (hipStream_t)stream);
          for (int j = 0; j < S && pe == hipSuccess; ++j) {
            uint16_t *dst = pk + (size_t)(E + j) * 2 * Ie * H;
            const uint16_t *gsh = (const uint16_t *)lw.w_sh_gate_up;
            pe = launch_pack_w32(gsh + (size_t)j * Ie * H, Ie, H, dst, (hipStream_t)stream);
            if (pe == hipSuccess)
              pe = launch_pack_w32(gsh + ((size_t)Is + (size_t)j * Ie) * H, Ie, H, dst + (size_t)Ie * H,
                                   (hipStream_t)stream);
          }
        } else {
          // routed experts, then shared pseudo-expert j: columns j Ie .. (j + 1) Ie of the shared down
          pe = launch_pack_w32(src[i], (int64_t)E * H, Ie, pk, (hipStream_t)stream);
          for (int j = 0; j < S && pe == hipSuccess; ++j)
            pe = launch_pack_w32_ld((const uint16_t *)lw.w_sh_down + (size_t)j * Ie, Is, H, Ie,
                                    pk + (size_t)(E + j) * H * Ie, (hipStream_t)stream);
        }
        if (pe != hipSuccess) {
          D->err = "weight packing failed";
          delete D;
          return DEC_E_HIP;
        }
        D->packed[l].w[i] = pk;
        pk += (size_t)ps.rows[i] * ps.K[i];
      }
    }
  }
  D->len.assign(cfg->max_batch, 0);
  D->has_next.assign(cfg->max_batch, 0);
  D->kv_pending.assign(cfg->max_batch, std::vector<int32_t>(cfg->n_layers, -1));
  for (int i = 0; i < STAGE_RING; ++i) D->ev_used[i] = false;

  auto cleanup = [&](int code) {
    if (D->pinned) (void)hipHostFree(D->pinned);
    for (int i = 0; i < STAGE_RING; ++i) (void)hipEventDestroy(D->ev[i]);
    delete D;
    return code;
  };
  if (hipHostMalloc((void **)&D->pinned, (size_t)STAGE_RING * L.stage_n * 4, hipHostMallocDefault) != hipSuccess) {
    D->pinned = nullptr;
    return cleanup(DEC_E_HIP);
  }
  for (int i = 0; i < STAGE_RING; ++i)
    if (hipEventCreateWithFlags(&D->ev[i], hipEventDisableTiming) != hipSuccess) return cleanup(DEC_E_HIP);

  // RoPE table: angle pos * base^(-2i/d) evaluated in fp64, stored as fp32
  // (cos, sin) pairs (pipeline.rs Pipeline::new keeps a head_dim/2 table of
  // inverse frequencies).
  const int half = cfg->head_dim / 2;
  std::vector<float2> tab((size_t)L.S * half);
  for (int p = 0; p < L.S; ++p)
    for (int i = 0; i < half; ++i) {
      const double ang = (double)p * std::pow(cfg->rope_base, -2.0 * i / cfg->head_dim);
      tab[(size_t)p * half + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
    }
  if (hipMemcpy(D->rope, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice) != hipSuccess)
    return cleanup(DEC_E_HIP);
  const size_t kvb = L.kv_units * L.kv_unit * 2;
  if (hipMemsetAsync(D->kcache, 0, kvb, D->stream) != hipSuccess ||
      hipMemsetAsync(D->vcache, 0, kvb, D->stream) != hipSuccess ||
      hipMemsetAsync(D->next_token, 0, (size_t)cfg->max_batch * 4, D->stream) != hipSuccess ||
      hipMemsetAsync(D->attn_cnt, 0, (size_t)attn_cnt_words(*cfg) * 4, D->stream) != hipSuccess ||
      hipStreamSynchronize(D->stream) != hipSuccess)
    return cleanup(DEC_E_HIP);
  *out = D;
  return DEC_OK;
}

void decoder_free(decoder_t *D) {
  if (!D) return;
  (void)hipStreamSynchronize(D->stream);
  for (auto &ev : D->tev) (void)hipEventDestroy(ev);
  if (D->pinned) (void)hipHostFree(D->pinned);
  for (int i = 0; i < STAGE_RING; ++i) (void)hipEventDestroy(D->ev[i]);
  if (D->gstream) (void)hipStreamDestroy(D->gstream);
  delete D;
}

int decoder_set_stream(decoder_t *D, void *stream) {
  if (!D) return DEC_E_INVALID;
  // the work already on the old stream finishes first: later calls share
  // the decoder's buffers and the fused launches' arrival counters with it
  if ((hipStream_t)stream != D->stream) HIP_TRY(D, hipStreamSynchronize(D->stream), "set_stream");
  D->stream = (hipStream_t)stream;
  return DEC_OK;
}

int32_t decoder_seq_len(const decoder_t *D, int32_t seq) {
  if (!D || seq < 0 || seq >= D->c.max_batch) return -1;
  return D->len[seq];
}

int prefill_chunk(decoder_t *D, int32_t seq, const int32_t *ids, int32_t n, int32_t start_pos,
                  int32_t logits_mode, float *d_logits, int32_t *d_argmax) {
  if (check_dec(D)) return DEC_E_INVALID;
  const decoder_config_t &c = D->c;
  if (seq < 0 || seq >= c.max_batch) return fail(D, DEC_E_INVALID, "seq out of range");
  if (!ids || n <= 0 || n > c.max_chunk) return fail(D, DEC_E_INVALID, "chunk length outside [1, max_chunk]");
  if (logits_mode < 0 || logits_mode > 2) return fail(D, DEC_E_INVALID, "logits_mode");
  if (start_pos != D->len[seq]) return fail(D, DEC_E_INVALID, "start_pos differs from the sequence length");
  if ((int64_t)start_pos + n > c.max_seq) return fail(D, DEC_E_CONTEXT_OVERFLOW, "prefill past max_seq");
  for (int i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= c.vocab) return fail(D, DEC_E_TOKEN, "token id out of range");
  std::vector<int32_t> seqs(n, seq), pos(n);
  for (int i = 0; i < n; ++i) pos[i] = start_pos + i;
  const int32_t new_len = start_pos + n;
  int rc = ensure_pages(D, 1, &seq, &new_len);
  if (rc) return rc;
  rc = stage_rows(D, n, ids, seqs.data(), pos.data());
  if (rc) return rc;
  const int G = c.n_heads / c.n_kv_heads;
  const int nout = logits_mode == 0 ? 0 : (logits_mode == 1 ? 1 : n);
  const int first = logits_mode == 1 ? n - 1 : 0;
  // logits_mode 2 (a multi-position verify) returns every row's greedy id
  rc = run_step(D, n, 16 / G, start_pos + n - 1, pos.data(), 0, first, nout, d_logits, d_argmax,
                logits_mode == 2 ? n : (nout ? 1 : 0));
  if (rc) return rc;
  D->len[seq] = start_pos + n;
  if (nout) D->has_next[seq] = 1;
  return DEC_OK;
}

int decode_step(decoder_t *D, int32_t batch, const int32_t *seqs, const int32_t *tokens,
                float *d_logits, int32_t *d_argmax) {
  if (check_dec(D)) return DEC_E_INVALID;
  const decoder_config_t &c = D->c;
  if (batch <= 0 || batch > c.max_batch || !seqs) return fail(D, DEC_E_INVALID, "batch outside [1, max_batch]");
  std::vector<int32_t> pos(batch);
  int max_pos = 0;
  for (int b = 0; b < batch; ++b) {
    const int s = seqs[b];
    if (s < 0 || s >= c.max_batch) return fail(D, DEC_E_INVALID, "seq out of range");
    for (int b2 = 0; b2 < b; ++b2)
      if (seqs[b2] == s) return fail(D, DEC_E_INVALID, "duplicate seq in batch");
    if (D->len[s] >= c.max_seq) return fail(D, DEC_E_CONTEXT_OVERFLOW, "sequence full");
    if (tokens) {
      if (tokens[b] < 0 || tokens[b] >= c.vocab) return fail(D, DEC_E_TOKEN, "token id out of range");
    } else if (!D->has_next[s]) {
      return fail(D, DEC_E_INVALID, "no previous greedy token for this sequence");
    }
    pos[b] = D->len[s];
    max_pos = std::max(max_pos, pos[b]);
  }
  std::vector<int32_t> new_len(batch);
  for (int b = 0; b < batch; ++b) new_len[b] = pos[b] + 1;
  int rc = ensure_pages(D, batch, seqs, new_len.data());
  if (rc) return rc;
  rc = stage_rows(D, batch, tokens, seqs, pos.data());
  if (rc) return rc;
  rc = run_step(D, batch, 1, max_pos, pos.data(), tokens ? 0 : 1, 0, batch, d_logits, d_argmax, batch);
  if (rc) return rc;
  for (int b = 0; b < batch; ++b) {
    D->len[seqs[b]] += 1;
    D->has_next[seqs[b]] = 1;
  }
  return DEC_OK;
}

int decode_run(decoder_t *D, int32_t seq, int32_t n_steps, int32_t *d_tokens) {
  if (check_dec(D)) return DEC_E_INVALID;
  const decoder_config_t &c = D->c;
  if (seq < 0 || seq >= c.max_batch) return fail(D, DEC_E_INVALID, "seq out of range");
  if (n_steps < 1 || !d_tokens) return fail(D, DEC_E_INVALID, "decode_run needs n_steps >= 1 and d_tokens");
  if (!D->has_next[seq]) return fail(D, DEC_E_INVALID, "no previous greedy token for this sequence");
  if ((int64_t)D->len[seq] + n_steps > c.max_seq) return fail(D, DEC_E_CONTEXT_OVERFLOW, "decode_run past max_seq");
  if (D->stats_mask) return fail(D, DEC_E_INVALID, "decode_run with node timers enabled");
  if (!D->gstream) HIP_TRY(D, hipStreamCreateWithFlags(&D->gstream, hipStreamNonBlocking), "decode_run stream");
  const int32_t pos0 = D->len[seq], last = pos0 + n_steps;
  int rc = ensure_pages(D, 1, &seq, &last);
  if (rc) return rc;
  rc = stage_rows(D, 1, nullptr, &seq, &pos0);
  if (rc) return rc;
  HIP_TRY(D, hipMemsetAsync(D->gout, 0, 4, D->stream), "decode_run counter");
  // everything before (the caller's work, the staged rows) is done before
  // the capture stream starts
  HIP_TRY(D, hipStreamSynchronize(D->stream), "decode_run sync");
  // capture one step: attention splits sized for the run's last position
  // (splits past a step's keys exit at once), positions read from row_pos
  hipStream_t user = D->stream;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  D->stream = D->gstream;
  hipError_t e = hipStreamBeginCapture(D->stream, hipStreamCaptureModeRelaxed);
  if (e != hipSuccess) {
    D->stream = user;
    return hip_fail(D, e, "decode_run capture");
  }
  D->graph_mode = true;
  rc = run_step(D, 1, 1, last - 1, &pos0, 1, 0, 1, nullptr, nullptr, 0);
  e = rc ? hipSuccess : launch_decode_advance(D->row_pos, D->next_token, seq, D->gout, D->stream);
  D->graph_mode = false;
  const hipError_t ec = hipStreamEndCapture(D->stream, &graph);
  D->stream = user;
  if (rc || e != hipSuccess || ec != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    if (rc) return rc;
    return hip_fail(D, e != hipSuccess ? e : ec, "decode_run capture");
  }
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  for (int i = 0; e == hipSuccess && i < n_steps; ++i) e = hipGraphLaunch(exec, D->gstream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(d_tokens, D->gout + 1, (size_t)n_steps * 4, hipMemcpyDeviceToDevice, D->gstream);
  // the graph is released only after its launches have drained
  const hipError_t es = hipStreamSynchronize(D->gstream);
  if (exec) (void)hipGraphExecDestroy(exec);
  (void)hipGraphDestroy(graph);
  if (e != hipSuccess || es != hipSuccess) return hip_fail(D, e != hipSuccess ? e : es, "decode_run");
  D->len[seq] = last;
  D->has_next[seq] = 1;
  return DEC_OK;
}

int kv_reset(decoder_t *D, int32_t seq) {
  if (check_dec(D)) return DEC_E_INVALID;
  const decoder_config_t &c = D->c;
  if (seq < -1 || seq >= c.max_batch) return fail(D, DEC_E_INVALID, "seq out of range");
  const int s0 = seq < 0 ? 0 : seq, s1 = seq < 0 ? c.max_batch : seq + 1;
  if (D->L.mp) {
    // paged: the pages go back to the pool (their stale rows are finite and
    // never read: a key past a query's position gets probability exactly 0)
    for (int s = s0; s < s1; ++s) release_pages(D, s, 0);
  } else {
    const size_t bytes = (size_t)(s1 - s0) * D->L.seq_stride * 2;
    HIP_TRY(D, hipMemsetAsync(D->kcache + (size_t)s0 * D->L.seq_stride, 0, bytes, D->stream), "kv_reset");
    HIP_TRY(D, hipMemsetAsync(D->vcache + (size_t)s0 * D->L.seq_stride, 0, bytes, D->stream), "kv_reset");
  }
  for (int s = s0; s < s1; ++s) {
    D->len[s] = 0;
    D->has_next[s] = 0;
    std::fill(D->kv_pending[s].begin(), D->kv_pending[s].end(), -1);
  }
  return DEC_OK;
}

int kv_truncate(decoder_t *D, int32_t seq, int32_t len) {
  if (check_dec(D)) return DEC_E_INVALID;
  if (seq < 0 || seq >= D->c.max_batch) return fail(D, DEC_E_INVALID, "seq out of range");
  if (len < 0 || len > D->len[seq]) return fail(D, DEC_E_INVALID, "kv_truncate length outside [0, current length]");
  // Rows past len keep their old values.  No kernel reads them: attention
  // at position p reads keys 0..p only (later keys of a loaded tile get
  // probability exactly 0), and every row below the next position is
  // rewritten before a query at or past it runs.
  D->len[seq] = len;
  D->has_next[seq] = 0;
  release_pages(D, seq, len);
  return DEC_OK;
}

int kv_load(decoder_t *D, int32_t seq, int32_t layer, const uint16_t *d_k, const uint16_t *d_v,
            int32_t len) {
  if (check_dec(D)) return DEC_E_INVALID;
  const decoder_config_t &c = D->c;
  if (seq < 0 || seq >= c.max_batch || layer < 0 || layer >= c.n_layers || !d_k || !d_v)
    return fail(D, DEC_E_INVALID, "kv_load argument");
  if (len < 0) return fail(D, DEC_E_INVALID, "kv_load length");
  if (len > c.max_seq) return fail(D, DEC_E_CONTEXT_OVERFLOW, "kv_load past max_seq");
  if (D->L.mp) {
    // paged: the sequence gets the pages len needs (all or nothing), the
    // page table travels to the device in a staging slot, and one kernel
    // scatters K rows and V^T columns into the pages
    int rc = ensure_pages(D, 1, &seq, &len);
    if (rc) return rc;
    if (len > 0) {
      rc = stage_rows(D, 0, nullptr, &seq, nullptr);
      if (rc) return rc;
      HIP_TRY(D, launch_kv_load_paged(d_k, d_v, D->kcache, D->vcache, D->page_table + (int64_t)seq * D->L.mp,
                                      D->L.kv_unit, kv_layer_off(D, layer), c.n_kv_heads, len, c.head_dim,
                                      D->L.kvS, D->stream), "kv_load paged");
    }
  } else {
    const int d = c.head_dim, S = D->L.S;
    const int64_t loff = (int64_t)seq * D->L.seq_stride + (int64_t)layer * c.n_kv_heads * (int64_t)S * d;
    for (int g = 0; g < c.n_kv_heads; ++g)
      HIP_TRY(D, hipMemcpyAsync(D->kcache + loff + (int64_t)g * S * d, d_k + (int64_t)g * len * d,
                                (size_t)len * d * 2, hipMemcpyDeviceToDevice, D->stream), "kv_load k");
    if (len > 0) HIP_TRY(D, launch_kv_load_v(d_v, D->vcache + loff, c.n_kv_heads, len, d, S, D->stream), "kv_load v");
  }
  D->kv_pending[seq][layer] = len;
  bool all = true;
  for (int l = 0; l < c.n_layers; ++l) all = all && D->kv_pending[seq][l] == len;
  if (all) {
    D->len[seq] = len;
    D->has_next[seq] = 0;
    std::fill(D->kv_pending[seq].begin(), D->kv_pending[seq].end(), -1);
    release_pages(D, seq, len);  // a paged sequence keeps only the pages len needs
  }
  return DEC_OK;
}

// ----------------------------------------------------------------- diag --

int dec_diag_gemm(const uint16_t *d_A, int32_t M, int32_t K, const uint16_t *d_W, int32_t N, float *d_C,
                  void *stream) {
  if (!d_A || !d_W || !d_C || M < 1 || M > 256 || N < 1 || K < 8 || K % 8) return DEC_E_INVALID;
  GemmArgs g{};
  g.A = d_A;
  g.lda = K;
  g.W = d_W;
  g.M = M;
  g.N = N;
  g.K = K;
  g.C = d_C;
  g.ldc = N;
  g.ksplit = 1;
  return launch_gemm(g, EPI_STORE, M, 1, (hipStream_t)stream) == hipSuccess ? DEC_OK : DEC_E_HIP;
}

int dec_diag_pack_w32(const uint16_t *d_W, int32_t rows, int32_t K, uint16_t *d_P, void *stream) {
  if (!d_W || !d_P || !pack_w32_fits(rows, K)) return DEC_E_INVALID;
  return launch_pack_w32(d_W, rows, K, d_P, (hipStream_t)stream) == hipSuccess ? DEC_OK : DEC_E_HIP;
}

int dec_diag_gemm_chunk(const uint16_t *d_A, int32_t planes, int32_t M, int32_t K, const uint16_t *d_Wp, int32_t N,
                        float *d_C, int32_t ksplit, float *d_part, int64_t part_elems, void *stream) {
  if (!d_A || !d_Wp || !d_C || (planes != 1 && planes != 2) || M < 1 || M > MAX_CHUNK || N < 1 || K < 16 ||
      K % 16 || ksplit < 1 || ksplit > 64)
    return DEC_E_INVALID;
  GemmArgs g{};
  g.A = d_A;
  g.a_lo = planes == 2 ? (int64_t)M * K : 0;
  g.lda = K;
  g.W = d_Wp;
  g.Wp = d_Wp;
  g.M = M;
  g.N = N;
  g.K = K;
  g.np_off = N;
  g.C = d_C;
  g.ldc = N;
  g.ksplit = ksplit;
  g.Cpart = d_part;
  g.wide = 1;
  if (ksplit > 1 && (!d_part || part_elems < (int64_t)ksplit * M * gemm_ntiles(g, EPI_STORE) * 16)) return DEC_E_INVALID;
  if (!gemm_chunk_fits(g, EPI_STORE)) return DEC_E_INVALID;
  return launch_gemm_chunk(g, EPI_STORE, (hipStream_t)stream) == hipSuccess ? DEC_OK : DEC_E_HIP;
}

int dec_diag_gemm_grouped(const uint16_t *d_A, int32_t planes, int32_t M, int32_t K, const uint16_t *d_Wp,
                          int32_t E, int32_t N, const int32_t *d_a_rows, int32_t P, const int32_t *d_groups,
                          float *d_C, void *stream) {
  if (!d_A || !d_Wp || !d_C || !d_a_rows || !d_groups || (planes != 1 && planes != 2) || M < 1 || E < 1 ||
      N < 32 || N % 32 || K < 16 || K % 16 || P < 1)
    return DEC_E_INVALID;
  GemmArgs g{};
  g.A = d_A;
  g.a_lo = planes == 2 ? (int64_t)M * K : 0;
  g.a_rows = d_a_rows;
  g.lda = K;
  g.W = d_Wp;
  g.Wp = d_Wp;
  g.w_group_stride = (int64_t)N * K;
  g.M = P;
  g.N = N;
  g.K = K;
  g.np_off = N;
  g.C = d_C;
  g.ldc = N;
  g.ksplit = 1;
  g.n_groups = d_groups;
  g.group_expert = d_groups + 1;
  g.group_start = d_groups + 1 + E;
  g.group_count = d_groups + 1 + 2 * E;
  if (!gemm_chunk_grouped_fits(g, EPI_STORE)) return DEC_E_INVALID;
  return launch_gemm_chunk_grouped(g, EPI_STORE, P, std::min(E, P), (hipStream_t)stream) == hipSuccess
             ? DEC_OK
             : DEC_E_HIP;
}

}  // extern "C"

// Split-K partials of dec_diag_gemm_chunk_noalloc: a file-scope device array,
// so that entry point allocates nothing.  Each device holds its own copy at
// its own address; host code uses that address (scratch_device), never the
// array's name, which on the host only stands in for the symbol.
constexpr int64_t NOALLOC_SCRATCH_FLOATS = int64_t(4) << 20;  // 16 MiB per device
static __device__ __align__(256) float scratch[NOALLOC_SCRATCH_FLOATS];

namespace {
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex scratch_mu;
float *scratch_addr[NOALLOC_MAX_DEVICES] = {};

// The current device's address of `scratch`, looked up once per device.
hipError_t scratch_device(float **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_addr[dev] = static_cast<float *>(p);
  }
  *out = scratch_addr[dev];
  return hipSuccess;
}
}  // namespace

extern "C" {

int dec_diag_gemm_chunk_noalloc(const uint16_t *d_A, int32_t planes, int32_t M, int32_t K, const uint16_t *d_Wp,
                                int32_t N, float *d_C, int32_t ksplit, void *stream) {
  if (!d_A || !d_Wp || !d_C || (planes != 1 && planes != 2) || M < 1 || M > MAX_CHUNK || N < 1 || K < 16 ||
      K % 16 || ksplit < 1 || ksplit > 64)
    return DEC_E_INVALID;
  GemmArgs g{};
  g.A = d_A;
  g.a_lo = planes == 2 ? (int64_t)M * K : 0;
  g.lda = K;
  g.W = d_Wp;
  g.Wp = d_Wp;
  g.M = M;
  g.N = N;
  g.K = K;
  g.np_off = N;
  g.C = d_C;
  g.ldc = N;
  g.ksplit = ksplit;
  g.wide = 1;
  if (!gemm_chunk_fits(g, EPI_STORE)) return DEC_E_INVALID;
  if (ksplit > 1) {
    // every partial the reduce reads is rewritten by this call's blocks, so
    // the previous call's contents need no clearing
    if ((int64_t)ksplit * M * gemm_ntiles(g, EPI_STORE) * 16 > NOALLOC_SCRATCH_FLOATS) return DEC_E_WORKSPACE;
    if (scratch_device(&g.Cpart) != hipSuccess) return DEC_E_HIP;
  }
  return launch_gemm_chunk(g, EPI_STORE, (hipStream_t)stream) == hipSuccess ? DEC_OK : DEC_E_HIP;
}

int dec_diag_gemv(const float *d_a, int32_t K, const uint16_t *d_W, int32_t N, float *d_y, void *stream) {
  if (!d_a || !d_W || !d_y || N < 1 || K < 8 || K % 8 || gemv_lds(K) > GEMV_MAX_LDS) return DEC_E_INVALID;
  GemvArgs g = gemv_args(d_W, d_a, K, N, d_y);
  return launch_gemv(g, EPI_STORE, (hipStream_t)stream) == hipSuccess ? DEC_OK : DEC_E_HIP;
}

int dec_diag_quantize_q4(const uint16_t *d_W, int64_t rows, int32_t K, uint8_t *d_codes, int8_t *d_exps,
                         uint16_t *d_deq, void *stream) {
  if (!d_W || !d_codes || !d_exps || !d_deq || rows < 1 || K < 32 || K % 32) return DEC_E_INVALID;
  return launch_quantize_q4(d_W, rows, K, d_codes, d_exps, d_deq, (hipStream_t)stream) == hipSuccess ? DEC_OK
                                                                                                 : DEC_E_HIP;
}

int dec_diag_gemv_q4(const float *d_a, int32_t K, const uint8_t *d_codes, const int8_t *d_exps, int32_t N,
                     float *d_y, void *stream) {
  if (!d_a || !d_codes || !d_exps || !d_y || N < 1 || K < 32 || K % 32 || gemv_lds(K, 4) > GEMV_MAX_LDS)
    return DEC_E_INVALID;
  GemvArgs g = gemv_args(nullptr, d_a, K, N, d_y);
  g.Wq = reinterpret_cast<const int8_t *>(d_codes);
  g.wexp = d_exps;
  g.qbits = 4;
  return launch_gemv(g, EPI_STORE, (hipStream_t)stream) == hipSuccess ? DEC_OK : DEC_E_HIP;
}

int dec_diag_moe_route(const float *d_logits, int32_t rows, int32_t E, int32_t k, int32_t renorm,
                       int32_t *d_ids, float *d_wts, void *stream) {
  if (!d_logits || !d_ids || !d_wts || rows < 1 || E < 1 || E > 256 || k < 1 || k > 8 || k > E)
    return DEC_E_INVALID;
  MoeRouteArgs mr{};
  mr.logits = d_logits;
  mr.rows = rows;
  mr.E = E;
  mr.k = k;
  mr.renorm = renorm;
  mr.ids = d_ids;
  mr.wts = d_wts;
  return launch_moe_route(mr, false, (hipStream_t)stream) == hipSuccess ? DEC_OK : DEC_E_HIP;
}

int dec_diag_rmsnorm(const float *d_x, const float *d_g, int32_t rows, int32_t H, double eps, uint16_t *d_out,
                     void *stream) {
  if (!d_x || !d_g || !d_out || rows < 1 || H < 4 || H % 4) return DEC_E_INVALID;
  return launch_rmsnorm(d_x, H, d_g, rows, H, (float)eps, d_out, H, 0, (hipStream_t)stream) == hipSuccess
             ? DEC_OK
             : DEC_E_HIP;
}

int dec_diag_quantize_rows(const uint16_t *d_W, int64_t rows, int32_t K, int8_t *d_q, float *d_scale,
                           uint16_t *d_deq, void *stream) {
  if (!d_W || !d_q || !d_scale || !d_deq || rows < 1 || K < 1) return DEC_E_INVALID;
  return launch_quantize_rows(d_W, rows, K, d_q, d_scale, d_deq, (hipStream_t)stream) == hipSuccess ? DEC_OK
                                                                                                 : DEC_E_HIP;
}

int decoder_stats_enable(decoder_t *D, int32_t node_mask) {
  if (check_dec(D)) return DEC_E_INVALID;
  if (node_mask) {
    if (D->tev.empty()) {
      D->tev.resize(TIMER_EVENTS);
      // timing-only events: no system-scope cache writeback when they are
      // recorded, which would add to the bracketed kernel's time (the
      // results are read after a stream synchronisation)
      for (auto &ev : D->tev) HIP_TRY(D, hipEventCreateWithFlags(&ev, hipEventDisableSystemFence), "stats events");
    }
    int rc = stats_harvest(D);
    if (rc) return rc;
    D->stats = decoder_stats_t{};
  } else {
    int rc = stats_harvest(D);
    if (rc) return rc;
  }
  D->stats_mask = (uint32_t)node_mask;
  return DEC_OK;
}

int decoder_stats_mask(decoder_t *D, int32_t node_mask) {
  if (check_dec(D)) return DEC_E_INVALID;
  if (node_mask && D->tev.empty()) return fail(D, DEC_E_INVALID, "stats not enabled");
  D->stats_mask = (uint32_t)node_mask;
  return DEC_OK;
}

int decoder_stats_read(decoder_t *D, decoder_stats_t *out) {
  if (check_dec(D) || !out) return DEC_E_INVALID;
  int rc = stats_harvest(D);
  if (rc) return rc;
  *out = D->stats;
  return DEC_OK;
}

int decoder_debug_layer_limit(decoder_t *D, int32_t layers) {
  if (check_dec(D)) return DEC_E_INVALID;
  D->layer_limit = layers;
  return DEC_OK;
}

int decoder_debug_stop_after_attention(decoder_t *D, int32_t on) {
  if (check_dec(D) || (on != 0 && on != 1)) return DEC_E_INVALID;
  D->stop_after_attn = on != 0;
  return DEC_OK;
}

int decoder_debug_fuse_o_proj(decoder_t *D, int32_t on) {
  if (check_dec(D) || (on != 0 && on != 1)) return DEC_E_INVALID;
  D->fuse_o = on != 0;
  return DEC_OK;
}

int decoder_debug_fuse_ffn(decoder_t *D, int32_t on) {
  if (check_dec(D) || (on != 0 && on != 1)) return DEC_E_INVALID;
  D->fuse_ffn = on != 0;
  return DEC_OK;
}

int decoder_debug_read_x(decoder_t *D, float *d_out, int32_t rows) {
  if (check_dec(D) || !d_out || rows < 1 || rows > D->L.R) return DEC_E_INVALID;
  HIP_TRY(D, hipMemcpyAsync(d_out, D->x, (size_t)rows * D->c.hidden * 4, hipMemcpyDeviceToDevice, D->stream),
          "read_x");
  return DEC_OK;
}

int decoder_debug_read_routes(decoder_t *D, int32_t *d_out, int32_t rows) {
  if (check_dec(D) || !d_out || rows < 1 || rows > D->L.R || D->c.n_experts == 0) return DEC_E_INVALID;
  HIP_TRY(D, hipMemcpyAsync(d_out, D->rids_rec, (size_t)D->c.n_layers * rows * D->c.top_k * 4,
                            hipMemcpyDeviceToDevice, D->stream), "read_routes");
  return DEC_OK;
}

}  // extern "C"
