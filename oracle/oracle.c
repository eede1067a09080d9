/*
 * oracle.c -- plain fp64 CPU oracle for one forward step of a decoder-only
 * GQA transformer (decode and chunked prefill, dense SwiGLU or routed MoE).
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU path; the only thing both sides
 * have in common is the seeded input generator (synth/), which holds none of
 * the decoder's arithmetic.
 *
 * Every quantity is evaluated in fp64.  Weights arrive as bf16 bit patterns
 * and are widened exactly; norm gains and biases arrive as fp32 and are
 * widened exactly.  Nothing is rounded between steps.  Loops follow the
 * definitions directly: every dot product is summed in index order, every
 * softmax is max-subtracted, and the only parallelism is OpenMP over
 * independent output elements (rows of a matrix-vector product, heads,
 * tokens), which does not change any sum.
 *
 * Sources (the three pages describe the same block; citations name the page
 * and the function or struct on it):
 *   engine.zig (midasdf/ANEDVD)       -- Engine.forward, Engine.prefill,
 *                                        rmsnormFlat / rmsnormColumn,
 *                                        ropeAndCache, the MoE route/accumulate
 *                                        loop and the shared-expert sigmoid gate.
 *   frink_models/decoder.rs            -- module doc (block order), AttnWeights
 *                                        (q/k/v/o shapes, bias before RoPE),
 *                                        MoeWeights (router, shared expert gate).
 *   cortiq_engine/pipeline.rs          -- module doc (prefill/decode contract),
 *                                        Pipeline::new (inverse-frequency table,
 *                                        1/sqrt(head_dim) scale), MoeFfn (softmax
 *                                        over all experts, top-k, optional renorm),
 *                                        lm_head_forward, embed_single.
 *
 * The KV cache is the one stored quantity whose precision the workloads fix
 * (a bf16 KV cache; engine.zig keeps its cache in f16): with kv_bf16 set,
 * keys (after RoPE) and values are rounded to bf16 (round to nearest even)
 * as they enter the cache, exactly where the method stores them, and every
 * later read sees the stored value.  All arithmetic stays fp64.
 *
 * Readings where the pages leave a step open (all listed in the design notes):
 *   RoPE pairs element i with element i + d/2 ("rope", not "ropeAdjacent"),
 *   with inverse frequency base^(-2i/d); GQA maps q head h to kv head
 *   floor(h * Hkv / Hq); top-k ties go to the lower expert index; argmax ties
 *   go to the lower token id.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- types -- */

typedef struct {
  int32_t hidden, n_layers, n_heads, n_kv_heads, head_dim;
  int32_t ffn_inter;                               /* dense SwiGLU width; 0 for MoE */
  int32_t n_experts, top_k, expert_inter, shared_inter, norm_topk_prob;
  int32_t vocab, qkv_bias;
  double rope_base, rms_eps;
  int32_t max_seq, n_seqs;
  int32_t kv_bf16;                                 /* 1: the KV cache stores bf16 values */
  int32_t sliding_window;                          /* 0: every earlier key; W > 0: the W most recent */
  double attn_softcap;                             /* 0: off; c > 0: score s -> c tanh(s / c) */
  int32_t qk_norm;                                 /* 1: RMSNorm of every q and k head before RoPE */
} orc_config_t;

typedef struct {
  const float *attn_norm, *ffn_norm;               /* [H] */
  const uint16_t *w_qkv;                           /* [(Hq+2Hkv)d][H]: q rows, k rows, v rows */
  const float *b_qkv;                              /* [(Hq+2Hkv)d] or NULL */
  const uint16_t *w_o;                             /* [H][Hq d] */
  const uint16_t *w_gate_up;                       /* [2I][H]: gate rows then up rows */
  const uint16_t *w_down;                          /* [H][I] */
  const uint16_t *w_router;                        /* [E][H] */
  const uint16_t *w_exp_gate_up;                   /* [E][2Ie][H] */
  const uint16_t *w_exp_down;                      /* [E][H][Ie] */
  const uint16_t *w_sh_gate_up;                    /* [2Is][H] */
  const uint16_t *w_sh_down;                       /* [H][Is] */
  const uint16_t *w_sh_gate;                       /* [H] or NULL */
  const float *attn_sinks;                         /* [Hq] sink logits, or NULL */
  const float *q_norm, *k_norm;                    /* [d] per-head norm gains (qk_norm) */
} orc_layer_t;

typedef struct {
  const uint16_t *embed;                           /* [V][H] */
  const float *final_norm;                         /* [H] */
  const uint16_t *lm_head;                         /* [V][H]; equals embed when tied */
  const orc_layer_t *layers;                       /* [n_layers] */
} orc_weights_t;

typedef struct {
  orc_config_t c;
  orc_weights_t w;
  orc_layer_t *layers;
  double *kc, *vc;                                 /* [seq][layer][pos][Hkv*d] */
  int32_t *len;                                    /* tokens already in each sequence's cache */
} orc_model_t;

enum { ORC_OK = 0, ORC_E_OVERFLOW = 1, ORC_E_INVALID = 2, ORC_E_TOKEN = 3, ORC_E_NOMEM = 4 };

/* ------------------------------------------------------------- helpers -- */

static inline double bf(uint16_t h) {            /* bf16 -> fp64, exact */
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round to the nearest bf16 value (8 significant bits), ties to even: the
 * value is scaled by a power of two so that its 8 significant bits are the
 * integer part, rounded with nearbyint (round-half-even in the default
 * rounding mode), and scaled back; both scalings are exact. */
double orc_round_bf16(double v) {
  if (v == 0.0 || !isfinite(v)) return v;
  int e;
  frexp(v, &e);                                  /* v = m 2^e, 0.5 <= |m| < 1 */
  double scale = ldexp(1.0, 8 - e);
  return nearbyint(v * scale) / scale;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------- primitives -- */

/* RMSNorm: out_i = x_i / sqrt(mean_j x_j^2 + eps) * g_i.
 * engine.zig, rmsnormFlat / rmsnormColumn: eps is added to the mean of
 * squares inside the square root, and the gain multiplies afterwards. */
void orc_rmsnorm(const double *x, const float *g, int n, double eps, double *out) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss / (double)n + eps);
  for (int i = 0; i < n; ++i) out[i] = x[i] * inv * (double)g[i];
}

/* Y[i][r] = sum_k W[r][k] X[i][k] for i < n tokens, W bf16 row-major [rows][cols].
 * The projections of engine.zig (1x1 convs: y = W x per column) and the
 * row-major [out][in] weight shapes of decoder.rs AttnWeights.  Each sum runs
 * over k in increasing order; tokens are handled four at a time only so one
 * widened weight feeds four independent sums. */
void orc_matmul(const uint16_t *W, int rows, int cols, const double *X, int n, double *Y) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    const uint16_t *wr = W + (size_t)r * cols;
    int i = 0;
    for (; i + 4 <= n; i += 4) {
      const double *x0 = X + (size_t)(i + 0) * cols, *x1 = X + (size_t)(i + 1) * cols;
      const double *x2 = X + (size_t)(i + 2) * cols, *x3 = X + (size_t)(i + 3) * cols;
      double s0 = 0, s1 = 0, s2 = 0, s3 = 0;
      for (int k = 0; k < cols; ++k) {
        double w = bf(wr[k]);
        s0 += w * x0[k];
        s1 += w * x1[k];
        s2 += w * x2[k];
        s3 += w * x3[k];
      }
      Y[(size_t)(i + 0) * rows + r] = s0;
      Y[(size_t)(i + 1) * rows + r] = s1;
      Y[(size_t)(i + 2) * rows + r] = s2;
      Y[(size_t)(i + 3) * rows + r] = s3;
    }
    for (; i < n; ++i) {
      const double *x0 = X + (size_t)i * cols;
      double s0 = 0;
      for (int k = 0; k < cols; ++k) s0 += bf(wr[k]) * x0[k];
      Y[(size_t)i * rows + r] = s0;
    }
  }
}

/* Single-vector form of orc_matmul. */
void orc_matvec(const uint16_t *W, int rows, int cols, const double *x, double *y) {
  orc_matmul(W, rows, cols, x, 1, y);
}

/* Rotary position embedding, in place, on nheads heads of width d at
 * position pos.  engine.zig ropeAndCache with rope_adjacent = false (the
 * "rope" pairing); pipeline.rs Pipeline::new (a head_dim/2 inverse-frequency
 * table).  Pair i is (v_i, v_{i+d/2}) and rotates by pos * base^(-2i/d). */
void orc_rope(double *v, int nheads, int d, long pos, double base) {
  int half = d / 2;
  for (int h = 0; h < nheads; ++h) {
    double *u = v + (size_t)h * d;
    for (int i = 0; i < half; ++i) {
      double theta = pow(base, -2.0 * (double)i / (double)d);
      double ang = (double)pos * theta;
      double c = cos(ang), s = sin(ang);
      double a = u[i], b = u[i + half];
      u[i] = a * c - b * s;
      u[i + half] = a * s + b * c;
    }
  }
}

/* Causal GQA attention for one query token over T cached positions.
 * engine.zig Engine.forward (cpu.attentionDecode over pos+1 rows) and
 * pipeline.rs Pipeline::new (scale 1/sqrt(head_dim)).  q: [Hq][d];
 * kc, vc: [T][Hkv*d] (row t holds every kv head of position t);
 * out: [Hq][d].  q head h reads kv head floor(h*Hkv/Hq).
 * Variants (engine.zig Engine.forward hands cpu.attentionDecode a logit
 * soft-cap and, on a sliding layer, a window; decoder.rs AttnWeights::sinks):
 *   window W > 0: only the W most recent positions (t > T - 1 - W) are keys;
 *   softcap c > 0: every scaled score s becomes c tanh(s / c);
 *   sinks (NULL: none): head h's sink logit z_h joins the softmax
 *   denominator as one more term and adds nothing to the output. */
void orc_attend(const double *q, const double *kc, const double *vc, int T, int Hq, int Hkv,
                int d, int window, double softcap, const float *sinks, double *out) {
  int kvd = Hkv * d;
  double scale = 1.0 / sqrt((double)d);
  int t0 = (window > 0 && T > window) ? T - window : 0;
  double *s = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  for (int h = 0; h < Hq; ++h) {
    int g = (int)((long)h * Hkv / Hq);
    const double *qh = q + (size_t)h * d;
    double m = -INFINITY;
    for (int t = t0; t < T; ++t) {
      const double *kt = kc + (size_t)t * kvd + (size_t)g * d;
      double acc = 0.0;
      for (int j = 0; j < d; ++j) acc += qh[j] * kt[j];
      s[t] = acc * scale;
      if (softcap > 0.0) s[t] = softcap * tanh(s[t] / softcap);
      if (s[t] > m) m = s[t];
    }
    double zs = sinks ? (double)sinks[h] : 0.0;
    if (sinks && zs > m) m = zs;
    double z = sinks ? exp(zs - m) : 0.0;
    for (int t = t0; t < T; ++t) {
      s[t] = exp(s[t] - m);
      z += s[t];
    }
    double *oh = out + (size_t)h * d;
    for (int j = 0; j < d; ++j) oh[j] = 0.0;
    for (int t = t0; t < T; ++t) {
      const double *vt = vc + (size_t)t * kvd + (size_t)g * d;
      double p = s[t] / z;
      for (int j = 0; j < d; ++j) oh[j] += p * vt[j];
    }
  }
  free(s);
}

/* silu(z) = z / (1 + e^-z).  pipeline.rs Act::Silu; engine.zig fused FFN
 * program (sigmoid, then two multiplies). */
double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* Logistic sigmoid, the shared-expert gate of engine.zig Engine.forward. */
double orc_sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* Router decision.  pipeline.rs MoeFfn: softmax over ALL expert logits,
 * then the k largest probabilities (distinct experts, engine.zig
 * expertWeightFor), optionally renormalised to sum to one.  Ties go to the
 * lower expert index (strict '>' scan in increasing index order).
 * probs (optional, [E]) receives the full softmax. */
void orc_route(const double *logits, int E, int k, int renorm, int32_t *idx, double *wts,
               double *probs) {
  double *p = (double *)malloc(sizeof(double) * (size_t)E);
  char *taken = (char *)calloc((size_t)E, 1);
  double m = -INFINITY;
  for (int e = 0; e < E; ++e) m = logits[e] > m ? logits[e] : m;
  double z = 0.0;
  for (int e = 0; e < E; ++e) {
    p[e] = exp(logits[e] - m);
    z += p[e];
  }
  for (int e = 0; e < E; ++e) p[e] /= z;
  double sel = 0.0;
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < E; ++e)
      if (!taken[e] && (best < 0 || p[e] > p[best])) best = e;
    taken[best] = 1;
    idx[j] = best;
    wts[j] = p[best];
    sel += p[best];
  }
  if (renorm)
    for (int j = 0; j < k; ++j) wts[j] /= sel;
  if (probs) memcpy(probs, p, sizeof(double) * (size_t)E);
  free(taken);
  free(p);
}

/* Greedy choice: index of the largest logit, lowest index on ties (the
 * strict '>' scans of engine.zig's MoE prefill test and pipeline.rs
 * ppl_ids). */
int32_t orc_argmax(const double *v, int n) {
  int32_t best = 0;
  for (int i = 1; i < n; ++i)
    if (v[i] > v[best]) best = i;
  return best;
}

/* SwiGLU FFN for n tokens: Y = W_d (silu(W_g B) * (W_u B)).
 * W_gu is [2I][H] with the gate rows first and the up rows after them
 * (engine.zig fused FFN program: gate conv, up conv, sigmoid, multiplies,
 * down conv). */
static void orc_swiglu(const uint16_t *W_gu, const uint16_t *W_d, int H, int I, const double *B,
                       int n, double *Y) {
  double *gu = (double *)malloc(sizeof(double) * (size_t)n * 2 * I);
  double *hh = (double *)malloc(sizeof(double) * (size_t)n * I);
  orc_matmul(W_gu, 2 * I, H, B, n, gu);
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < I; ++j) {
      double g = gu[(size_t)i * 2 * I + j], u = gu[(size_t)i * 2 * I + I + j];
      hh[(size_t)i * I + j] = orc_silu(g) * u;
    }
  orc_matmul(W_d, H, I, hh, n, Y);
  free(hh);
  free(gu);
}

/* ---------------------------------------------------------------- model -- */

orc_model_t *orc_create(const orc_config_t *c, const orc_weights_t *w) {
  orc_model_t *m = (orc_model_t *)calloc(1, sizeof(orc_model_t));
  if (!m) return NULL;
  m->c = *c;
  m->w = *w;
  m->layers = (orc_layer_t *)malloc(sizeof(orc_layer_t) * (size_t)c->n_layers);
  memcpy(m->layers, w->layers, sizeof(orc_layer_t) * (size_t)c->n_layers);
  m->w.layers = m->layers;
  size_t kvd = (size_t)c->n_kv_heads * c->head_dim;
  size_t per = (size_t)c->n_seqs * c->n_layers * (size_t)c->max_seq * kvd;
  m->kc = (double *)calloc(per, sizeof(double));
  m->vc = (double *)calloc(per, sizeof(double));
  m->len = (int32_t *)calloc((size_t)c->n_seqs, sizeof(int32_t));
  if (!m->kc || !m->vc || !m->len) {
    free(m->kc);
    free(m->vc);
    free(m->len);
    free(m->layers);
    free(m);
    return NULL;
  }
  return m;
}

void orc_free(orc_model_t *m) {
  if (!m) return;
  free(m->kc);
  free(m->vc);
  free(m->len);
  free(m->layers);
  free(m);
}

static double *kv_row(orc_model_t *m, double *base, int seq, int layer, int pos) {
  size_t kvd = (size_t)m->c.n_kv_heads * m->c.head_dim;
  return base + (((size_t)seq * m->c.n_layers + layer) * (size_t)m->c.max_seq + pos) * kvd;
}

/* Forget a sequence (seq = -1: every sequence).  engine.zig Engine.reset. */
void orc_reset(orc_model_t *m, int seq) {
  for (int s = 0; s < m->c.n_seqs; ++s) {
    if (seq >= 0 && s != seq) continue;
    size_t n = (size_t)m->c.n_layers * m->c.max_seq * m->c.n_kv_heads * m->c.head_dim;
    memset(kv_row(m, m->kc, s, 0, 0), 0, n * sizeof(double));
    memset(kv_row(m, m->vc, s, 0, 0), 0, n * sizeof(double));
    m->len[s] = 0;
  }
}

/* Install a cache prefix for one layer of one sequence: K and V are bf16
 * [Hkv][len][d].  The sequence's length becomes len (call for every layer
 * with the same len). */
int orc_kv_load(orc_model_t *m, int seq, int layer, const uint16_t *K, const uint16_t *V,
                int len) {
  if (seq < 0 || seq >= m->c.n_seqs || layer < 0 || layer >= m->c.n_layers) return ORC_E_INVALID;
  if (len < 0 || len > m->c.max_seq) return ORC_E_OVERFLOW;
  int Hkv = m->c.n_kv_heads, d = m->c.head_dim;
  for (int t = 0; t < len; ++t) {
    double *kr = kv_row(m, m->kc, seq, layer, t), *vr = kv_row(m, m->vc, seq, layer, t);
    for (int g = 0; g < Hkv; ++g)
      for (int j = 0; j < d; ++j) {
        size_t src = ((size_t)g * len + t) * d + j;
        kr[g * d + j] = bf(K[src]);
        vr[g * d + j] = bf(V[src]);
      }
  }
  m->len[seq] = len;
  return ORC_OK;
}

/* Weight quantisation (quantised weight streaming for decode): each row of
 * a bf16 matrix W [rows][K] becomes int8 codes q and one power-of-two scale
 * 2^e, with e the smallest integer for which 127 * 2^e covers the row's
 * largest magnitude a, and q_k = w_k / 2^e rounded to the nearest integer
 * (ties to even).  Every step is exact in fp64 (a bf16 value divided by a
 * power of two, then rounded), so the codes follow from the definition
 * alone.  The dequantised weight q_k * 2^e has at most 7 significant bits,
 * so it is itself a bf16 value; out receives those bf16 bit patterns and
 * e_out (optional) the exponents. */
void orc_quantize_rows(const uint16_t *W, int rows, int K, uint16_t *out, int32_t *e_out) {
  for (int r = 0; r < rows; ++r) {
    const uint16_t *w = W + (size_t)r * K;
    double a = 0.0;
    for (int k = 0; k < K; ++k) a = fmax(a, fabs(bf(w[k])));
    int e = 0;
    if (a > 0.0) {
      int p;
      double m = frexp(a, &p);          /* a = m 2^p, m in [0.5, 1) */
      e = (m <= 127.0 / 128.0) ? p - 7 : p - 6;
    }
    if (e_out) e_out[r] = e;
    for (int k = 0; k < K; ++k) {
      double q = nearbyint(ldexp(bf(w[k]), -e));  /* default rounding: to nearest, ties to even */
      double v = ldexp(q, e);
      float f = (float)v;                          /* exact: q 2^e fits bf16 */
      uint32_t u;
      memcpy(&u, &f, 4);
      out[(size_t)r * K + k] = (uint16_t)(u >> 16);
    }
  }
}

/* 4-bit weight quantisation (quantised weight streaming with 4-bit codes;
 * decoder.rs names packed 4-bit expert planes): every group of 32
 * consecutive weights of a row gets one power-of-two scale 2^e, with e the
 * smallest integer for which 7 * 2^e covers the group's largest magnitude a,
 * and codes q = w / 2^e rounded to the nearest integer (ties to even), so
 * |q| <= 7.  All steps are exact in fp64.  The dequantised q 2^e has at most
 * 3 significant bits, a bf16 value; out receives those bf16 bit patterns,
 * q_out (optional) the codes [rows][K] and e_out (optional) the exponents
 * [rows][K / 32].  K must be a multiple of 32.  An all-zero group takes e = 0. */
void orc_quantize_q4(const uint16_t *W, int rows, int K, uint16_t *out, int8_t *q_out, int32_t *e_out) {
  int groups = K / 32;
  for (int r = 0; r < rows; ++r)
    for (int gi = 0; gi < groups; ++gi) {
      const uint16_t *w = W + (size_t)r * K + (size_t)gi * 32;
      double a = 0.0;
      for (int j = 0; j < 32; ++j) a = fmax(a, fabs(bf(w[j])));
      int e = 0;
      if (a > 0.0) {
        int p;
        frexp(a, &p);                              /* a < 2^p, so 7 * 2^(p-2) > a */
        e = p - 2;
        while (7.0 * ldexp(1.0, e - 1) >= a) --e;  /* smallest e with 7 * 2^e >= a */
      }
      if (e_out) e_out[(size_t)r * groups + gi] = e;
      for (int j = 0; j < 32; ++j) {
        double q = nearbyint(ldexp(bf(w[j]), -e));  /* to nearest, ties to even */
        float f = (float)ldexp(q, e);                /* exact: 3 significant bits */
        uint32_t u;
        memcpy(&u, &f, 4);
        out[(size_t)r * K + (size_t)gi * 32 + j] = (uint16_t)(u >> 16);
        if (q_out) q_out[(size_t)r * K + (size_t)gi * 32 + j] = (int8_t)q;
      }
    }
}

/* Roll a sequence back to its first len positions (0 <= len <= current
 * length): the rows past len stop being part of it and are cleared, so the
 * state equals one that never held them.  pipeline.rs
 * Pipeline::generate_from_ids (a rejected draft's KV entry is dropped). */
int orc_truncate(orc_model_t *m, int seq, int len) {
  if (seq < 0 || seq >= m->c.n_seqs || len < 0 || len > m->len[seq]) return ORC_E_INVALID;
  size_t rows = (size_t)(m->len[seq] - len) * m->c.n_kv_heads * m->c.head_dim;
  for (int l = 0; l < m->c.n_layers; ++l) {
    memset(kv_row(m, m->kc, seq, l, len), 0, rows * sizeof(double));
    memset(kv_row(m, m->vc, seq, l, len), 0, rows * sizeof(double));
  }
  m->len[seq] = len;
  return ORC_OK;
}

int32_t orc_seq_len(const orc_model_t *m, int seq) { return m->len[seq]; }

/* Routed MoE FFN with shared expert for n tokens (B: normed inputs [n][H]).
 * engine.zig Engine.forward (router matmul over the normed FFN input, route,
 * accumulate p * expert(h) into a scratch, shared expert scaled by
 * sigmoid(gate . h)) and Engine.prefill (route every column first, then read
 * each chosen expert once for all the columns that chose it);
 * decoder.rs MoeWeights (router [E,H], shared_expert_gate [H]). */
static void orc_moe(const orc_model_t *m, const orc_layer_t *L, const double *B, int n,
                    double *F, int32_t *routes, double *probs, const int32_t *force) {
  int H = m->c.hidden, E = m->c.n_experts, k = m->c.top_k, Ie = m->c.expert_inter;
  int Is = m->c.shared_inter;
  double *logits = (double *)malloc(sizeof(double) * (size_t)n * E);
  int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)n * k);
  double *wts = (double *)malloc(sizeof(double) * (size_t)n * k);
  double *P = (double *)malloc(sizeof(double) * (size_t)E);
  orc_matmul(L->w_router, E, H, B, n, logits);
  for (int i = 0; i < n; ++i) {
    orc_route(logits + (size_t)i * E, E, k, m->c.norm_topk_prob, idx + (size_t)i * k,
              wts + (size_t)i * k, P);
    if (probs) memcpy(probs + (size_t)i * E, P, sizeof(double) * E);
    if (force) {
      /* teacher-forced expert choice: the given ids replace the top-k; each
       * keeps its own softmax probability as its weight (renormalised over
       * the given set when norm_topk_prob), exactly as if the router had
       * chosen it */
      double sum = 0.0;
      for (int j = 0; j < k; ++j) {
        int e = force[(size_t)i * k + j];
        idx[(size_t)i * k + j] = e;
        wts[(size_t)i * k + j] = P[e];
        sum += P[e];
      }
      if (m->c.norm_topk_prob)
        for (int j = 0; j < k; ++j) wts[(size_t)i * k + j] /= sum;
    }
  }
  free(P);
  if (routes) memcpy(routes, idx, sizeof(int32_t) * (size_t)n * k);
  memset(F, 0, sizeof(double) * (size_t)n * H);

  /* routed experts: each chosen expert is applied once to the tokens that chose it */
  int *cols = (int *)malloc(sizeof(int) * (size_t)n);
  double *wcol = (double *)malloc(sizeof(double) * (size_t)n);
  double *Bg = (double *)malloc(sizeof(double) * (size_t)n * H);
  double *Yg = (double *)malloc(sizeof(double) * (size_t)n * H);
  size_t gu_sz = (size_t)2 * Ie * H, d_sz = (size_t)H * Ie;
  for (int e = 0; e < E; ++e) {
    int cnt = 0;
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < k; ++j)
        if (idx[(size_t)i * k + j] == e) {
          cols[cnt] = i;
          wcol[cnt] = wts[(size_t)i * k + j];
          ++cnt;
        }
    if (!cnt) continue;
    for (int c = 0; c < cnt; ++c) memcpy(Bg + (size_t)c * H, B + (size_t)cols[c] * H, sizeof(double) * H);
    orc_swiglu(L->w_exp_gate_up + (size_t)e * gu_sz, L->w_exp_down + (size_t)e * d_sz, H, Ie, Bg,
               cnt, Yg);
    for (int c = 0; c < cnt; ++c)
      for (int r = 0; r < H; ++r) F[(size_t)cols[c] * H + r] += wcol[c] * Yg[(size_t)c * H + r];
  }
  /* shared expert, scaled by sigmoid(w_sg . b) when the gate vector exists */
  if (Is > 0) {
    orc_swiglu(L->w_sh_gate_up, L->w_sh_down, H, Is, B, n, Yg);
    for (int i = 0; i < n; ++i) {
      double sc = 1.0;
      if (L->w_sh_gate) {
        double g = 0.0;
        for (int r = 0; r < H; ++r) g += bf(L->w_sh_gate[r]) * B[(size_t)i * H + r];
        sc = orc_sigmoid(g);
      }
      for (int r = 0; r < H; ++r) F[(size_t)i * H + r] += sc * Yg[(size_t)i * H + r];
    }
  }
  free(Yg);
  free(Bg);
  free(wcol);
  free(cols);
  free(wts);
  free(idx);
  free(logits);
}

/* Forward n tokens of one sequence starting at start_pos (which must equal
 * the sequence's current length), layer by layer over the whole chunk.
 * Every token is forwarded exactly once and enters the cache exactly once
 * (pipeline.rs module doc); engine.zig Engine.prefill / Engine.forward give
 * the per-layer order: RMSNorm, QKV (+bias), RoPE and cache append,
 * attention, o_proj and residual, RMSNorm, FFN and residual; then the final
 * RMSNorm and the lm-head (pipeline.rs lm_head_forward).
 *
 * logits_mode: 0 none, 1 the last token only (logits: [V]), 2 every token
 * (logits: [n][V]).  routes ([L][n][k]) and router_probs ([L][n][E]) are
 * optional MoE records.  force_routes ([L][n][k], optional) teacher-forces
 * the expert choice: where two expert sets are both correct (a near-tie of
 * the k-th expert), the oracle follows the given one, as a teacher-forced
 * decode follows a given token.  x_trace ([L+1][n][H], optional) receives the
 * residual stream after the embedding and after every layer. */
int orc_forward(orc_model_t *m, int seq, const int32_t *ids, int n, int start_pos,
                int logits_mode, double *logits, int32_t *routes, double *router_probs,
                double *x_trace, const int32_t *force_routes) {
  const orc_config_t *c = &m->c;
  if (seq < 0 || seq >= c->n_seqs || n <= 0) return ORC_E_INVALID;
  if (start_pos != m->len[seq]) return ORC_E_INVALID;
  if ((long)start_pos + n > c->max_seq) return ORC_E_OVERFLOW;
  for (int i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= c->vocab) return ORC_E_TOKEN;
  /* forced expert ids must be k distinct experts per (layer, token) */
  if (force_routes && c->n_experts > 0) {
    int k = c->top_k;
    for (size_t r = 0; r < (size_t)c->n_layers * n; ++r)
      for (int j = 0; j < k; ++j) {
        int e = force_routes[r * k + j];
        if (e < 0 || e >= c->n_experts) return ORC_E_INVALID;
        for (int j2 = 0; j2 < j; ++j2)
          if (force_routes[r * k + j2] == e) return ORC_E_INVALID;
      }
  }

  int H = c->hidden, Hq = c->n_heads, Hkv = c->n_kv_heads, d = c->head_dim;
  int qd = Hq * d, kvd = Hkv * d, nqkv = qd + 2 * kvd;
  size_t nh = (size_t)n * H;
  double *X = (double *)malloc(sizeof(double) * nh);
  double *A = (double *)malloc(sizeof(double) * nh);
  double *Y = (double *)malloc(sizeof(double) * nh);
  double *QKV = (double *)malloc(sizeof(double) * (size_t)n * nqkv);
  double *O = (double *)malloc(sizeof(double) * (size_t)n * qd);
  if (!X || !A || !Y || !QKV || !O) return ORC_E_NOMEM;

  /* embedding gather, scale 1 (pipeline.rs embed_single; engine.zig
   * Engine.forward with embed_scale 1) */
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < H; ++j) X[(size_t)i * H + j] = bf(m->w.embed[(size_t)ids[i] * H + j]);
  if (x_trace) memcpy(x_trace, X, sizeof(double) * nh);

  for (int l = 0; l < c->n_layers; ++l) {
    const orc_layer_t *L = &m->layers[l];
    for (int i = 0; i < n; ++i) orc_rmsnorm(X + (size_t)i * H, L->attn_norm, H, c->rms_eps, A + (size_t)i * H);
    orc_matmul(L->w_qkv, nqkv, H, A, n, QKV);
    if (c->qkv_bias && L->b_qkv)            /* bias before RoPE (decoder.rs AttnWeights) */
      for (int i = 0; i < n; ++i)
        for (int r = 0; r < nqkv; ++r) QKV[(size_t)i * nqkv + r] += (double)L->b_qkv[r];
    for (int i = 0; i < n; ++i) {
      double *q = QKV + (size_t)i * nqkv, *k = q + qd, *v = k + kvd;
      long pos = (long)start_pos + i;
      if (c->qk_norm) {                       /* engine.zig applyHeadNorm: per head, before RoPE */
        for (int h = 0; h < Hq; ++h) orc_rmsnorm(q + (size_t)h * d, L->q_norm, d, c->rms_eps, q + (size_t)h * d);
        for (int h = 0; h < Hkv; ++h) orc_rmsnorm(k + (size_t)h * d, L->k_norm, d, c->rms_eps, k + (size_t)h * d);
      }
      orc_rope(q, Hq, d, pos, c->rope_base);
      orc_rope(k, Hkv, d, pos, c->rope_base);
      double *kr = kv_row(m, m->kc, seq, l, (int)pos), *vr = kv_row(m, m->vc, seq, l, (int)pos);
      for (int j = 0; j < kvd; ++j) {
        kr[j] = c->kv_bf16 ? orc_round_bf16(k[j]) : k[j];
        vr[j] = c->kv_bf16 ? orc_round_bf16(v[j]) : v[j];
      }
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < n; ++i) {
      int T = start_pos + i + 1;              /* causal: keys 0 .. start_pos+i */
      orc_attend(QKV + (size_t)i * nqkv, kv_row(m, m->kc, seq, l, 0), kv_row(m, m->vc, seq, l, 0), T,
                 Hq, Hkv, d, c->sliding_window, c->attn_softcap, L->attn_sinks, O + (size_t)i * qd);
    }
    orc_matmul(L->w_o, H, qd, O, n, Y);
    for (size_t j = 0; j < nh; ++j) X[j] += Y[j];
    for (int i = 0; i < n; ++i) orc_rmsnorm(X + (size_t)i * H, L->ffn_norm, H, c->rms_eps, A + (size_t)i * H);
    if (c->n_experts > 0)
      orc_moe(m, L, A, n, Y, routes ? routes + (size_t)l * n * c->top_k : NULL,
              router_probs ? router_probs + (size_t)l * n * c->n_experts : NULL,
              force_routes ? force_routes + (size_t)l * n * c->top_k : NULL);
    else
      orc_swiglu(L->w_gate_up, L->w_down, H, c->ffn_inter, A, n, Y);
    for (size_t j = 0; j < nh; ++j) X[j] += Y[j];
    if (x_trace) memcpy(x_trace + (size_t)(l + 1) * nh, X, sizeof(double) * nh);
  }
  m->len[seq] = start_pos + n;

  if (logits_mode == 1 || logits_mode == 2) {
    int first = logits_mode == 1 ? n - 1 : 0, cnt = n - first;
    for (int i = 0; i < cnt; ++i)
      orc_rmsnorm(X + (size_t)(first + i) * H, m->w.final_norm, H, c->rms_eps, A + (size_t)i * H);
    orc_matmul(m->w.lm_head, c->vocab, H, A, cnt, logits);
  }
  free(O);
  free(QKV);
  free(Y);
  free(A);
  free(X);
  return ORC_OK;
}
