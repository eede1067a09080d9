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

/* out[r] = bf16(x[r] / sqrt(mean(x[r]^2) + eps) * g) for r < rows
 * (engine.zig rmsnormColumn).  x fp32 [rows][H], g fp32 [H], out bf16 [rows][H]. */
int dec_diag_rmsnorm(const float *d_x, const float *d_g, int32_t rows, int32_t H, double eps,
                     uint16_t *d_out, void *stream);

/* Run only the first `layers` layers in later calls (-1: all of them); the
 * final norm and lm-head still run (engine.zig Engine.stopAfterLayer). */
int decoder_debug_layer_limit(decoder_t *dec, int32_t layers);

/* Copy the residual stream x (fp32 [rows][H]) left by the last prefill_chunk
 * or decode_step (row i = token i of the chunk, or batch entry i) to d_out. */
int decoder_debug_read_x(decoder_t *dec, float *d_out, int32_t rows);

/* Copy the MoE expert choices of the last call, int32 [n_layers][rows][top_k]
 * in router order, to d_out. */
int decoder_debug_read_routes(decoder_t *dec, int32_t *d_out, int32_t rows);

#ifdef __cplusplus
}
#endif
#endif /* DECODER_DIAG_H */
