/*
 * decoder.h -- C ABI of libdecoder.so: one forward step of a decoder-only
 * GQA transformer on an MI355X (gfx950), for single-token decode (batch of
 * sequences) and chunked prefill, ending in the lm-head and a greedy argmax.
 *
 * The block (frink_models/decoder.rs, module doc; engine.zig, Engine.forward):
 *   x = E[token]
 *   per layer:  a = RMSNorm(x; g_attn)                 (engine.zig rmsnormColumn)
 *               [q;k;v] = W_qkv a (+ b_qkv)            (decoder.rs AttnWeights: bias before RoPE)
 *               q, k rotated at their position (RoPE),  (engine.zig ropeAndCache)
 *               k, v appended to the layer's KV cache
 *               o = causal GQA softmax attention        (engine.zig Engine.forward, attentionDecode;
 *                                                        pipeline.rs Pipeline::new: scale 1/sqrt(d))
 *               x += W_o o
 *               b = RMSNorm(x; g_ffn)
 *               x += W_down(silu(W_gate b) * W_up b)    dense SwiGLU, or
 *               x += sum_top-k p_e FFN_e(b) + sigmoid(w_sg . b) FFN_shared(b)
 *                                                       (pipeline.rs MoeFfn; engine.zig Engine.forward
 *                                                        shared-expert gate; decoder.rs MoeWeights)
 *   logits = W_head RMSNorm(x; g_final)                 (pipeline.rs lm_head_forward)
 *   next token = argmax(logits), lowest id on ties.
 * Prefill/decode contract (pipeline.rs module doc): every token is forwarded
 * exactly once and enters the KV cache exactly once.
 *
 * Readings where the pages leave a step open: RoPE pairs element i with
 * element i + d/2 and rotates it by pos * base^(-2i/d); q head h reads kv
 * head floor(h * Hkv / Hq); top-k ties go to the lower expert index.
 *
 * Conventions
 *  - All matrices are bf16 (uint16 bit patterns), row-major [out][in].
 *    Norm gains and biases are fp32.  Logits are fp32.
 *  - Weight pointers are DEVICE pointers, BORROWED: the caller keeps them
 *    alive and unchanged until decoder_free (engine.zig module doc: the
 *    engine borrows its weights, which must outlive it).
 *  - The caller allocates one device workspace of decoder_workspace_bytes()
 *    bytes and passes it in; the library lays out the KV cache, the RoPE
 *    table and all scratch inside it and never allocates device memory.
 *  - Token ids and sequence indices are HOST arrays (validated on the host
 *    before anything is launched).  Output buffers are DEVICE pointers.
 *    Host ids are a deliberate choice over device id arrays: the checks that
 *    refuse a bad call before anything runs (ids in [0, vocab), distinct
 *    sequences, lengths against max_seq, pages available) and the sizing of
 *    the attention splits need the values on the host, and they reach the
 *    device in one pinned copy per call.  Greedy decode keeps its tokens on
 *    the device (decode_step with tokens = NULL, decode_run).
 *  - Every call is asynchronous on the decoder's stream; only the returned
 *    status is synchronous.  Outputs are valid once the stream has drained.
 *  - A failing call returns a nonzero DEC_E_* code and launches nothing
 *    (DEC_E_HIP excepted: the HIP error text is kept for decoder_last_error).
 *    There is no silent fallback to another code path.
 */
#ifndef DECODER_H
#define DECODER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DEC_OK = 0,
  DEC_E_CONTEXT_OVERFLOW = 1, /* start_pos + n > max_seq, a full sequence on decode, or no free
                                 page left in a paged cache */
  DEC_E_INVALID = 2,          /* bad argument: n <= 0, n > max_chunk, batch > max_batch,
                                 start_pos != current length, bad seq, bad config, ... */
  DEC_E_TOKEN = 3,            /* token id outside [0, vocab) */
  DEC_E_WORKSPACE = 4,        /* workspace NULL, too small or misaligned */
  DEC_E_HIP = 5,              /* a HIP runtime call failed */
};

typedef struct decoder decoder_t; /* opaque */

typedef struct {
  int32_t hidden;          /* H */
  int32_t n_layers;        /* L */
  int32_t n_heads;         /* Hq */
  int32_t n_kv_heads;      /* Hkv; Hq % Hkv == 0 and Hq / Hkv <= 16 */
  int32_t head_dim;        /* d: 64 or 128 */
  int32_t ffn_inter;       /* I: dense SwiGLU width; 0 for an MoE model */
  int32_t n_experts;       /* E (0 for a dense model), <= 256 */
  int32_t top_k;           /* k <= 8 */
  int32_t expert_inter;    /* Ie */
  int32_t shared_inter;    /* Is; 0 = no shared expert */
  int32_t shared_gate;     /* 1: shared expert scaled by sigmoid(w_sg . b) */
  int32_t norm_topk_prob;  /* 1: renormalise the top-k probabilities to sum to one */
  int32_t vocab;           /* V */
  int32_t qkv_bias;        /* 1: b_qkv is present */
  double rope_base;        /* RoPE base */
  double rms_eps;          /* RMSNorm epsilon */
  int32_t max_seq;         /* KV capacity per sequence (positions) */
  int32_t max_chunk;       /* largest prefill chunk (tokens per call), <= 512 */
  int32_t max_batch;       /* number of sequences (KV slots); largest decode batch */
  /* Attention variants (engine.zig Engine.forward hands its attention a
   * logit soft-cap and, on a sliding layer, a window): */
  int32_t sliding_window;  /* 0: a query attends to every earlier position; W > 0:
                              the query at position p sees keys t with p - W < t <= p
                              (every layer) */
  double attn_softcap;     /* 0: off; c > 0: each scaled score s becomes c tanh(s / c) */
  int32_t qk_norm;         /* 1: RMSNorm (gains q_norm / k_norm [d], eps rms_eps) of every q
                              and k head after the bias and before RoPE (engine.zig
                              applyHeadNorm) */
  int32_t weight_quant;    /* 1: quantised weight streaming (pipeline.rs streams row-quantised
                              int8 "q8_row" weights): decoder_init turns the attention
                              projections, the FFN (dense, or every routed expert and the
                              shared expert) and the lm-head into int8 codes with one
                              power-of-two scale per row, 2^e with e the smallest integer for
                              which 127 * 2^e covers the row's largest magnitude, codes
                              rounded to nearest (ties to even).  The model then computes with
                              the dequantised weights (exactly bf16 values) on every path; the
                              embedding gather keeps the caller's table.
                              2: the same matrices as 4-bit codes (decoder.rs names packed
                              4-bit expert planes) with one power-of-two scale 2^e per group of
                              32 consecutive weights of a row, e the smallest integer for which
                              7 * 2^e covers the group's largest magnitude, codes in [-7, 7]
                              rounded to nearest (ties to even); every row length must be a
                              multiple of 32.  Batch-1 decode streams the codes (a quarter of
                              the bf16 bytes); the other paths read the dequantised copies */
  int32_t kv_page_size;    /* 0: each sequence owns max_seq cache rows; P > 0 (a multiple of 32):
                              the cache is a pool of kv_pages pages of P positions, handed to
                              sequences as they grow and returned by kv_reset / kv_truncate
                              (a paged cache for sequences of ragged lengths) */
  int32_t kv_pages;        /* pages in the pool when kv_page_size > 0 */
} decoder_config_t;

typedef struct {
  const float *attn_norm;          /* [H] */
  const float *ffn_norm;           /* [H] */
  const uint16_t *w_qkv;           /* [(Hq + 2 Hkv) d][H]: q rows, then k rows, then v rows */
  const float *b_qkv;              /* [(Hq + 2 Hkv) d], or NULL when qkv_bias == 0 */
  const uint16_t *w_o;             /* [H][Hq d] */
  const uint16_t *w_gate_up;       /* dense: [2 I][H], gate rows then up rows */
  const uint16_t *w_down;          /* dense: [H][I] */
  const uint16_t *w_router;        /* MoE: [E][H] */
  const uint16_t *w_exp_gate_up;   /* MoE: [E][2 Ie][H] */
  const uint16_t *w_exp_down;      /* MoE: [E][H][Ie] */
  const uint16_t *w_sh_gate_up;    /* MoE shared expert: [2 Is][H] */
  const uint16_t *w_sh_down;       /* MoE shared expert: [H][Is] */
  const uint16_t *w_sh_gate;       /* MoE shared-expert gate vector: [H] (when shared_gate) */
  const float *attn_sinks;         /* [Hq] one sink logit per query head, or NULL: it joins
                                      that head's softmax denominator and adds nothing to
                                      the output (decoder.rs AttnWeights::sinks) */
  const float *q_norm;             /* [d] per-head q norm gains (required when qk_norm) */
  const float *k_norm;             /* [d] per-head k norm gains (required when qk_norm) */
} decoder_layer_weights_t;

typedef struct {
  const uint16_t *embed;                  /* [V][H] */
  const float *final_norm;                /* [H] */
  const uint16_t *lm_head;                /* [V][H]; pass embed for tied embeddings */
  const decoder_layer_weights_t *layers;  /* HOST array [n_layers]; copied by decoder_init */
} decoder_weights_t;

/* Bytes of device workspace decoder_init needs for this config (KV cache,
 * RoPE table, activations and scratch), or 0 if the config is invalid.
 * pipeline.rs ForwardScratch: the forward pass's buffers are allocated once,
 * sized from the model, and reused by every steady-state step; here that
 * one allocation is the caller's (engine.zig Engine.init sizes its KV
 * cache and activation buffers from the config in the same way).  Pure
 * host arithmetic: nothing is launched or allocated. */
size_t decoder_workspace_bytes(const decoder_config_t *cfg);

/* Validate the config, record the borrowed weights, lay out the workspace
 * (256-byte aligned; its contents are overwritten), upload the RoPE table
 * and zero the KV cache.  stream is a hipStream_t (NULL = default stream).
 * On success *out owns host-side state only; free it with decoder_free.
 * engine.zig Engine.init: validate the config first, then build everything
 * a step needs from the borrowed layer weights, so that no later step has
 * to allocate.  Errors: DEC_E_INVALID (bad config, a required weight
 * pointer NULL), DEC_E_WORKSPACE (workspace NULL, misaligned or smaller
 * than decoder_workspace_bytes), DEC_E_HIP (a copy or launch of the set-up
 * failed; nothing is kept and *out stays NULL). */
int decoder_init(const decoder_config_t *cfg, const decoder_weights_t *weights,
                 void *d_workspace, size_t workspace_bytes, void *stream, decoder_t **out);

/* Forward n prompt tokens (host ids[n], 1 <= n <= max_chunk) of sequence
 * seq at positions start_pos .. start_pos+n-1; start_pos must equal the
 * sequence's current length (engine.zig Engine.prefill; pipeline.rs module
 * doc).  start_pos + n == max_seq is allowed; more is DEC_E_CONTEXT_OVERFLOW.
 * logits_mode: 0 no logits, 1 the last token's logits ([V] into d_logits),
 * 2 every token's logits ([n][V]).  d_logits may be NULL (then logits go to
 * internal scratch).  When logits are computed, the greedy next token of the
 * last row is kept for decode_step(tokens = NULL) and, if d_argmax is not
 * NULL, written to d_argmax[0] (int32); with logits_mode 2, d_argmax
 * receives every row's greedy token ([n] int32, lowest id on ties).
 * logits_mode 2 is also the multi-position verify of speculative decoding
 * (pipeline.rs Pipeline::generate_from_ids and forward_pair: the positions
 * of a drafted continuation go through one pass that streams each weight
 * matrix once, and row i's logits score the token after position
 * start_pos + i); kv_truncate rolls back the rows of rejected drafts. */
int prefill_chunk(decoder_t *dec, int32_t seq, const int32_t *ids, int32_t n,
                  int32_t start_pos, int32_t logits_mode, float *d_logits, int32_t *d_argmax);

/* One decode step for batch sequences (host seqs[batch], distinct): each
 * forwards one token at position len[seq] and appends it to its cache.
 * tokens: host [batch] ids, or NULL to feed each sequence's own previous
 * greedy token (kept on the device; no host round trip).  d_logits
 * ([batch][V] fp32) and d_argmax ([batch] int32) may each be NULL.
 * engine.zig Engine.forward: one decode step for a token at a position,
 * refused with a context-overflow error when the position has no cache row;
 * pipeline.rs module doc: decode rows of several sequences share one pass
 * over the weights, attention reads each sequence's own cache.  Errors:
 * DEC_E_INVALID (batch outside [1, max_batch], a seq out of range or
 * repeated, tokens NULL for a sequence with no previous greedy token),
 * DEC_E_TOKEN (an id outside [0, vocab)), DEC_E_CONTEXT_OVERFLOW (a
 * sequence already holds max_seq positions, or a paged pool has no page
 * left); nothing is launched on these.  DEC_E_HIP: a launch failed. */
int decode_step(decoder_t *dec, int32_t batch, const int32_t *seqs, const int32_t *tokens,
                float *d_logits, int32_t *d_argmax);

/* pipeline.rs Pipeline::generate_from_ids (its greedy loop: each step feeds
 * the previous step's argmax back in; decoder.rs folds the argmax into the
 * lm-head so only the token id leaves the device):
 * n_steps greedy decode steps of sequence seq (batch 1), each feeding the
 * previous step's greedy token, as decode_step(tokens = NULL) would; the n
 * generated ids go to d_tokens ([n_steps] int32, device).  One step is
 * captured into a HIP graph (positions read from device memory, attention
 * splits sized for the run's last position) and replayed n_steps times,
 * so the host does no work per step.  Captured on a stream of the
 * library's own; the caller's stream is synchronised first.  Needs a
 * previous greedy token (a decode_step, or a prefill_chunk with
 * logits_mode > 0, not followed by kv_truncate or kv_reset), len + n_steps
 * <= max_seq (DEC_E_CONTEXT_OVERFLOW otherwise, or when a paged pool lacks
 * the pages) and the node timers off; these are checked before anything
 * runs.  Synchronous: returns after the steps have run.  No per-step
 * logits.  d_tokens is borrowed, written only.  A DEC_E_HIP error after the
 * checks leaves the sequence's cache and greedy token undefined: reset it. */
int decode_run(decoder_t *dec, int32_t seq, int32_t n_steps, int32_t *d_tokens);

/* Forget sequence seq (-1: all sequences): its length becomes 0 and its KV
 * rows are zeroed (engine.zig Engine.reset: forget the KV cache to start a
 * new conversation).  A paged cache returns the sequence's pages to the
 * pool instead of zeroing them.  DEC_E_INVALID for seq outside
 * [-1, max_batch); DEC_E_HIP if the clearing launch fails. */
int kv_reset(decoder_t *dec, int32_t seq);

/* Roll sequence seq back to its first len cached positions
 * (0 <= len <= current length, else DEC_E_INVALID): the next prefill or
 * decode of seq writes at position len.  pipeline.rs
 * Pipeline::generate_from_ids: a rejected draft's KV entry is dropped
 * (truncate_last).  Host-side only: nothing is launched, and the rows past
 * len are never read again before they are rewritten.  decode_step with
 * tokens = NULL is refused for seq until a call with logits has run. */
int kv_truncate(decoder_t *dec, int32_t seq, int32_t len);

/* Install a KV-cache prefix for one layer of one sequence from device
 * buffers d_k, d_v, both bf16 [Hkv][len][d] (keys already rotated).  The
 * sequence's length becomes len once every layer has been loaded with the
 * same len (call in any layer order; the length is set on the last layer).
 * decoder.rs (its per-layer device-resident KV: a prefix restore uploads
 * host K/V rows into it).  A paged cache gives the sequence the pages len
 * needs at its first call (all or nothing) and keeps only those once every
 * layer is loaded.  DEC_E_INVALID: bad seq, layer or pointer, len < 0;
 * DEC_E_CONTEXT_OVERFLOW: len > max_seq, or the page pool lacks the pages. */
int kv_load(decoder_t *dec, int32_t seq, int32_t layer, const uint16_t *d_k,
            const uint16_t *d_v, int32_t len);

/* Current length (cached positions) of sequence seq, or -1 if seq is invalid.
 * decoder.rs: a prefill must start at the cache's current position count
 * (start_pos equal to cache.positions()); this reports that count. */
int32_t decoder_seq_len(const decoder_t *dec, int32_t seq);

/* Replace the stream all later calls launch on (hipStream_t).  Stream
 * plumbing only; no passage of the pages defines an operation here (their
 * engines run on one queue of their own).  When the stream changes, the
 * call first waits for the work already launched on the old one, so later
 * calls never overlap it (they share the decoder's buffers).  DEC_OK;
 * DEC_E_INVALID for NULL; DEC_E_HIP if that wait fails. */
int decoder_set_stream(decoder_t *dec, void *stream);

/* engine.zig Engine.deinit: release what init made.  Waits for the stream,
 * then frees the host state, pinned staging memory and events; the
 * caller's workspace and the borrowed weights stay the caller's.  NULL is a
 * no-op. */
void decoder_free(decoder_t *dec);
/* Static text for a DEC_* code ("unknown error" for others). */
const char *decoder_strerror(int code);
/* Text of the last failure on this decoder (empty if none), naming the
 * check or the HIP call and its error string: engine.zig prints why a
 * kernel build failed instead of a bare error code.  Valid until the next
 * call on the same decoder. */
const char *decoder_last_error(const decoder_t *dec);

#ifdef __cplusplus
}
#endif
#endif /* DECODER_H */
