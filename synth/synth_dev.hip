// Seeded synthetic input generator (device side), for inputs too large to
// build on the host in reasonable time (tens of GB of KV-cache fill or
// weights).  Same definitions as synth.c: SplitMix64 counter stream,
// Box-Muller cosine branch in fp64, fp32 then bf16 round-to-nearest-even.
// Device libm may differ from the host's in the last fp64 ulp, which flips a
// bf16 rounding only for values within ~2^-45 of a rounding boundary; the
// tests compare both generators on a sample.  Holds none of the decoder's
// arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

__device__ __forceinline__ uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint16_t to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__global__ void synth_normal_bf16_kernel(uint16_t *out, uint64_t n, uint64_t seed,
                                         double sigma, uint64_t offset) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    uint64_t j = offset + i;
    uint64_t z1 = sm64_mix(seed + (2 * j + 1) * SM64_GAMMA);
    uint64_t z2 = sm64_mix(seed + (2 * j + 2) * SM64_GAMMA);
    double u1 = ((double)(z1 >> 11) + 0.5) * 0x1.0p-53;
    double u2 = (double)(z2 >> 11) * 0x1.0p-53;
    double v = sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
    out[i] = to_bf16_rne((float)(sigma * v));
  }
}

extern "C" int synth_dev_normal_bf16(void *d_out, uint64_t n, uint64_t seed, double sigma,
                                     uint64_t offset, void *stream) {
  if (n == 0) return 0;
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(synth_normal_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, (uint16_t *)d_out, n, seed, sigma, offset);
  return (int)hipGetLastError();
}
