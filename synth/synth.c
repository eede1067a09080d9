/*
 * Seeded synthetic input generator (host side).
 *
 * This module produces inputs only: weights, biases, prompts and KV-cache
 * fills.  It contains none of the decoder's arithmetic.  Both the fp64
 * oracle and the GPU harness draw their inputs from it, so the two sides see
 * bit-identical bf16 weights.
 *
 * Definitions (each element is independent of every other, so any range can
 * be produced in parallel or in pieces):
 *   SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 *   generators", OOPSLA 2014): the i-th output (i = 0, 1, ...) of a stream
 *   started from state s is mix(s + (i + 1) * 0x9E3779B97F4A7C15), where
 *   mix(z) = z' ^ (z' >> 31) with z' from the two xor-shift-multiply rounds
 *   (>>30, *0xBF58476D1CE4E5B9, >>27, *0x94D049BB133111EB).
 *   Uniforms: u1 = ((z >> 11) + 0.5) * 2^-53 (never 0), u2 = (z >> 11) * 2^-53.
 *   Normal element j: Box-Muller cosine branch over outputs 2j and 2j+1,
 *   n = sqrt(-2 ln u1) * cos(2 pi u2), scaled by sigma in fp64, rounded to
 *   fp32, then to bf16 with round-to-nearest-even.
 *   Token j: ((output_j >> 32) * vocab) >> 32.
 *   Tensor seed: output 0 of the stream started at base ^ (layer << 20) ^ id.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_splitmix64_at(uint64_t state, uint64_t i) {
  return sm64_mix(state + (i + 1) * SM64_GAMMA);
}

uint64_t synth_tensor_seed(uint64_t base, uint32_t layer, uint32_t tensor_id) {
  return synth_splitmix64_at(base ^ ((uint64_t)layer << 20) ^ (uint64_t)tensor_id, 0);
}

static inline double sm64_normal(uint64_t seed, uint64_t j) {
  uint64_t z1 = synth_splitmix64_at(seed, 2 * j);
  uint64_t z2 = synth_splitmix64_at(seed, 2 * j + 1);
  double u1 = ((double)(z1 >> 11) + 0.5) * 0x1.0p-53;
  double u2 = (double)(z2 >> 11) * 0x1.0p-53;
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

uint16_t synth_f32_to_bf16(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  if ((b & 0x7f800000u) == 0x7f800000u) return (uint16_t)((b >> 16) | ((b & 0xffffu) ? 0x40u : 0u));
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

/* out[i] = bf16(fp32(sigma * normal(seed, offset + i))), i in [0, n). */
void synth_normal_bf16(uint16_t *out, uint64_t n, uint64_t seed, double sigma, uint64_t offset) {
  long long nn = (long long)n;
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < nn; ++i) {
    float f = (float)(sigma * sm64_normal(seed, offset + (uint64_t)i));
    out[i] = synth_f32_to_bf16(f);
  }
}

/* Same values as synth_normal_bf16, widened back to fp32 (exact). */
void synth_normal_bf16_as_f32(float *out, uint64_t n, uint64_t seed, double sigma, uint64_t offset) {
  long long nn = (long long)n;
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < nn; ++i) {
    float f = (float)(sigma * sm64_normal(seed, offset + (uint64_t)i));
    uint32_t b = (uint32_t)synth_f32_to_bf16(f) << 16;
    memcpy(&out[i], &b, 4);
  }
}

/* Uniform token ids in [0, vocab). */
void synth_tokens(int32_t *out, uint64_t n, uint64_t seed, uint32_t vocab) {
  for (uint64_t i = 0; i < n; ++i) {
    uint64_t z = synth_splitmix64_at(seed, i);
    out[i] = (int32_t)(((z >> 32) * (uint64_t)vocab) >> 32);
  }
}
