/*
 * decoder_diag.h -- inspection entry points of libdecoder.so, for checking
 * single steps of the path against an independent reference.  The idea is
 * engine.zig's Engine.diagnose (each kernel against a CPU matmul on the same
 * weights) and Engine.stopAfterLayer (run a prefix of the layers, then look
 * at the hidden state).  Same conventions as decoder.h: device pointers for
 * data, asynchronous on the given stream (or the decoder's stream), status
 * returned synchronously.
 */
#ifndef DECODER_DIAG_H
#define DECODER_DIAG_H

#include <stddef.h>
#include <stdint.h>

#include "decoder.h"

#ifdef __cplusplus
extern "C" {
#endif

/* C[m][n] = sum_k A[m][k] W[n][k] with the decode/prefill projection kernel
 * (engine.zig: every projection is y = W x per token).  A bf16 [M][K],
 * W bf16 [N][K], C fp32 [M][N]; 1 <= M <= 256, K % 8 == 0. */
int dec_diag_gemm(const uint16_t *d_A, int32_t M, int32_t K, const uint16_t *d_W, int32_t N,
                  float *d_C, void *stream);

/* Packed copy of a bf16 weight matrix W [rows][K] for the chunk projection
 * kernel: P[((nt * K / 16 + kt) * 64 + l) * 8 + e] = W[32 nt + l % 32][16 kt + 8 (l / 32) + e]
 * (32-row x 16-k tiles of 1 KB in MFMA lane order).  rows % 32 == 0,
 * K % 16 == 0; P holds rows * K bf16 values.  DEC_E_INVALID otherwise. */
int dec_diag_pack_w32(const uint16_t *d_W, int32_t rows, int32_t K, uint16_t *d_P, void *stream);

/* C = A W^T with the chunk projection kernel (prefill chunks; engine.zig
 * Engine.prefill: a chunk of token columns shares one pass over the
 * weights).  A bf16 [planes][M][K]: planes 1 = plain bf16, 2 = hi plane then
 * lo plane (the activation is their sum); d_Wp = W [N][K] packed by
 * dec_diag_pack_w32; C fp32 [M][N].  2 <= M <= 512, N % 32 == 0,
 * K % 16 == 0.  ksplit > 1 splits K over blocks; the fp32 partials need
 * part_elems >= ksplit * M * N floats at d_part, reduced in fixed split
 * order.  DEC_E_INVALID on bad sizes. */
int dec_diag_gemm_chunk(const uint16_t *d_A, int32_t planes, int32_t M, int32_t K, const uint16_t *d_Wp,
                        int32_t N, float *d_C, int32_t ksplit, float *d_part, int64_t part_elems,
                        void *stream);

/* Grouped expert projection with the chunk kernel's grouped form (MoE
 * prefill; engine.zig Engine.prefill: a chunk's token columns are batched by
 * chosen expert, so each chosen expert's weights are read once).
 * C[p][n] = sum_k A[a_rows[p]][k] W_e[n][k] for pair p of group i, e =
 * expert[i].  A bf16 [planes][M][K] (planes as dec_diag_gemm_chunk);
 * d_Wp = the stacked expert weights [E][N][K], taken as one [E N][K] matrix
 * and packed by dec_diag_pack_w32; d_a_rows int32 [P]; C fp32 [P][N].
 * d_groups (device int32, the layout the MoE router's grouping writes):
 * [0] = group count G <= min(E, P), then expert[E], start[E], count[E];
 * group i covers pairs start[i] .. start[i] + count[i] - 1.  The table's
 * contents are the caller's contract, not checked: every a_rows value < M,
 * the groups' counts positive, summing to at most P, their ranges inside
 * [0, P), every expert < E.  N % 32 == 0, K % 16 == 0.  DEC_E_INVALID on
 * bad sizes. */
int dec_diag_gemm_grouped(const uint16_t *d_A, int32_t planes, int32_t M, int32_t K, const uint16_t *d_Wp,
                          int32_t E, int32_t N, const int32_t *d_a_rows, int32_t P, const int32_t *d_groups,
                          float *d_C, void *stream);

/* dec_diag_gemm_chunk without the partial-sum workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments,
 * layouts and results as dec_diag_gemm_chunk; with ksplit > 1 the fp32
 * partials live in a 16 MiB array that the library holds on each device
 * (static device memory, kept until the process ends), so this call never
 * allocates.  ksplit * M * ceil(N / 16) * 16 floats must fit in 4 Mi
 * (4 194 304) floats, else DEC_E_WORKSPACE and nothing is launched.  Every
 * call on one device shares that device's array: two calls that overlap on
 * one device (different streams, no ordering between them) race and give
 * undefined results; calls ordered on one stream are safe.  The first call
 * on a device looks the array's address up once (DEC_E_HIP if that fails). */
int dec_diag_gemm_chunk_noalloc(const uint16_t *d_A, int32_t planes, int32_t M, int32_t K,
                                const uint16_t *d_Wp, int32_t N, float *d_C, int32_t ksplit,
                                void *stream);

/* y[n] = sum_k W[n][k] a[k] with the batch-1 decode projection kernel.
 * a fp32 [K], W bf16 [N][K], y fp32 [N]; K % 8 == 0, K * 4 <= 61440. */
int dec_diag_gemv(const float *d_a, int32_t K, const uint16_t *d_W, int32_t N, float *d_y, void *stream);

/* out[r] = bf16(x[r] / sqrt(mean(x[r]^2) + eps) * g) for r < rows
 * (engine.zig rmsnormColumn).  x fp32 [rows][H], g fp32 [H], out bf16 [rows][H]. */
int dec_diag_rmsnorm(const float *d_x, const float *d_g, int32_t rows, int32_t H, double eps,
                     uint16_t *d_out, void *stream);

/* Per-row int8 weight quantisation as decoder_init does it with
 * weight_quant (a power-of-two scale 2^e per row, e the smallest integer
 * with 127 * 2^e >= the row's largest magnitude, codes rounded to nearest,
 * ties to even).  W bf16 [rows][K]; q int8 [rows][K]; scale fp32 [rows];
 * deq bf16 [rows][K] the dequantised weights. */
int dec_diag_quantize_rows(const uint16_t *d_W, int64_t rows, int32_t K, int8_t *d_q, float *d_scale,
                           uint16_t *d_deq, void *stream);

/* 4-bit quantisation as decoder_init does it with weight_quant 2: per group
 * of 32 consecutive weights of a row, e is the smallest integer with
 * 7 * 2^e >= the group's largest magnitude, codes q = rint(w / 2^e) (ties to
 * even, |q| <= 7).  W bf16 [rows][K], K % 32 == 0; codes [rows][K / 2] bytes,
 * q + 8 of element 2j in the low nibble of byte j and of 2j + 1 in the high
 * one; exps int8 [rows][K / 32]; deq bf16 [rows][K] the dequantised weights. */
int dec_diag_quantize_q4(const uint16_t *d_W, int64_t rows, int32_t K, uint8_t *d_codes, int8_t *d_exps,
                         uint16_t *d_deq, void *stream);

/* y[n] = sum_k W[n][k] a[k] with the batch-1 decode projection kernel on
 * 4-bit weights (codes and exps as dec_diag_quantize_q4 writes them; W is
 * their dequantised value).  a fp32 [K], y fp32 [N]; K % 32 == 0. */
int dec_diag_gemv_q4(const float *d_a, int32_t K, const uint8_t *d_codes, const int8_t *d_exps, int32_t N,
                     float *d_y, void *stream);

/* MoE routing of rows router-logit vectors (pipeline.rs MoeFfn: softmax
 * over all experts, top-k, optional renormalisation; lower index first on
 * ties).  logits fp32 [rows][E]; ids int32 [rows][k] in router order,
 * wts fp32 [rows][k]; E <= 256, k <= 8. */
int dec_diag_moe_route(const float *d_logits, int32_t rows, int32_t E, int32_t k, int32_t renorm,
                       int32_t *d_ids, float *d_wts, void *stream);

/* Run only the first `layers` layers in later calls (-1: all of them); the
 * final norm and lm-head still run (engine.zig Engine.stopAfterLayer). */
int decoder_debug_layer_limit(decoder_t *dec, int32_t layers);

/* on = 1: the last layer that later calls run (the layer limit's last, or
 * the model's last) stops after its attention sub-block, o_proj and the
 * residual add included, so decoder_debug_read_x returns that layer's FFN
 * input before its RMSNorm (the residual the router and the experts read).
 * engine.zig Engine.stopAfterLayer, taken to the sub-block inside a layer.
 * on = 0 restores full layers.  DEC_E_INVALID for other values. */
int decoder_debug_stop_after_attention(decoder_t *dec, int32_t on);

/* on = 0: a batch-1 decode step launches each layer's output projection as
 * its own GEMV after the attention; on = 1 (the default): the attention
 * launch runs it where the kernel takes it (bf16 weights, fp32 attention
 * output, the in-kernel split merge).  Both give the same bits; the switch
 * exists so that tests can compare them.  DEC_E_INVALID for other values. */
int decoder_debug_fuse_o_proj(decoder_t *dec, int32_t on);

/* on = 0: a batch-1 decode step launches each dense layer's gate/up and down
 * projections as two GEMVs; on = 1 (the default): one launch runs both, the
 * down projection's blocks waiting for the gate/up blocks' outputs, where
 * it pays (bf16 weights and a gate/up grid of at least two blocks per
 * compute unit).  Both give the same bits; the switch exists so that tests can
 * compare them.  DEC_E_INVALID for other values. */
int decoder_debug_fuse_ffn(decoder_t *dec, int32_t on);

/* Copy the residual stream x (fp32 [rows][H]) left by the last prefill_chunk
 * or decode_step (row i = token i of the chunk, or batch entry i) to d_out. */
int decoder_debug_read_x(decoder_t *dec, float *d_out, int32_t rows);

/* Copy the MoE expert choices of the last call, int32 [n_layers][rows][top_k]
 * in router order, to d_out. */
int decoder_debug_read_routes(decoder_t *dec, int32_t *d_out, int32_t rows);

/* Per-node timing (engine.zig Engine Stats: time and evaluation count per
 * node, so a slow node shows by itself).  While enabled, every kernel launch
 * of a node is bracketed by HIP events on the decoder's stream, and the
 * node's algorithmic traffic (bytes that must cross HBM: weights read once,
 * KV rows read, activations in and out) and arithmetic (2 flops per
 * multiply-add) are added up on the host. */
enum {
  DEC_NODE_QKV = 0,      /* QKV projection (+ its split-K reduction) */
  DEC_NODE_ROPE = 1,     /* bias + RoPE + KV append */
  DEC_NODE_ATTN = 2,     /* attention (+ split merge) */
  DEC_NODE_O = 3,        /* o_proj + residual */
  DEC_NODE_GATE_UP = 4,  /* dense gate/up projection with the SwiGLU epilogue (batch-1 decode with the
                            fused FFN launch: also the down projection and residual) */
  DEC_NODE_DOWN = 5,     /* dense down projection + residual */
  DEC_NODE_ROUTER = 6,   /* MoE router logits, top-k and grouping */
  DEC_NODE_EXPERTS = 7,  /* MoE routed + shared experts and the combine */
  DEC_NODE_HEAD = 8,     /* final norm, lm-head, argmax */
  DEC_NODE_NORM = 9,     /* RMSNorm launches inside the layers */
  DEC_NODE_EMBED = 10,   /* embedding gather */
  DEC_NODE_COUNT = 11
};

typedef struct {
  int64_t launches[DEC_NODE_COUNT]; /* kernel launches timed */
  double ms[DEC_NODE_COUNT];        /* summed kernel time (event to event) */
  double bytes[DEC_NODE_COUNT];     /* summed algorithmic HBM bytes */
  double flops[DEC_NODE_COUNT];     /* summed algorithmic flops */
} decoder_stats_t;

/* node_mask != 0: clear the counters and start timing the nodes whose bit
 * (1 << DEC_NODE_*) is set (-1: every node); 0: stop timing (counters are
 * kept for decoder_stats_read).  Timing fewer nodes perturbs the step less. */
int decoder_stats_enable(decoder_t *dec, int32_t node_mask);
/* Change which nodes are timed without clearing the counters or waiting
 * for the stream (for timing a sample of the steps of a timed region). */
int decoder_stats_mask(decoder_t *dec, int32_t node_mask);
/* Wait for the decoder's stream, then return the totals since enabling. */
int decoder_stats_read(decoder_t *dec, decoder_stats_t *out);

#ifdef __cplusplus
}
#endif
#endif /* DECODER_DIAG_H */
