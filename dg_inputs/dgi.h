/* dgi.h — seeded synthetic-input generator shared by the GPU path's tests/bench
 * and the CPU oracle's tests.
 *
 * This header holds NO arithmetic of the block-diffusion method.  It only turns
 * (seed, stream, index) into reproducible numbers used as *inputs*: weights,
 * prompt tokens, hidden states, KV-cache contents.  The method's own random
 * draws (canvas initialisation and re-randomisation) use Philox4x32-10, which
 * the oracle and the HIP library each implement separately; this generator is
 * a different algorithm on purpose so that the two never share a code path.
 *
 * Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used in counter mode:
 *     bits(seed, stream, i) = mix(mix(seed ^ stream*GOLDEN) + (i+1)*GOLDEN)
 * where mix is the SplitMix64 output finaliser.
 *
 * Normal-like values: the 64 bits are cut into four 16-bit uniforms
 * u0..u3 in [0, 65535]; s = 2*(u0+u1+u2+u3) - 4*65535 is an odd integer with
 * mean 0 and standard deviation 2*sqrt(4*(65536^2-1)/12) ~= 75674.4 (an
 * Irwin-Hall sum of four uniforms).  The value is (float)s * scale, where the
 * caller passes scale = sigma / 75674.4 as an fp32 number.  Every step is exact
 * integer arithmetic followed by one correctly rounded fp32 multiply, so the
 * host and the device produce bit-identical values; bf16 storage is then the
 * round-to-nearest-even truncation below, also bit-identical.
 *
 * Uniform integers in [0, n): ((bits >> 32) * n) >> 32 (multiply-shift).
 */
#ifndef DGI_H
#define DGI_H

#include <stdint.h>

#if defined(__HIPCC__)
#define DGI_FN static inline __host__ __device__
#else
#define DGI_FN static inline
#endif

#define DGI_GOLDEN 0x9E3779B97F4A7C15ULL
/* Standard deviation of s = 2*(u0+u1+u2+u3) - 4*65535 for u uniform on 0..65535. */
#define DGI_SUM4_STD 75674.38473

DGI_FN uint64_t dgi_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

DGI_FN uint64_t dgi_bits(uint64_t seed, uint64_t stream, uint64_t i) {
  uint64_t base = dgi_mix(seed ^ (stream * DGI_GOLDEN));
  return dgi_mix(base + (i + 1ULL) * DGI_GOLDEN);
}

DGI_FN float dgi_normal(uint64_t seed, uint64_t stream, uint64_t i, float scale) {
  uint64_t b = dgi_bits(seed, stream, i);
  int32_t u0 = (int32_t)(b & 0xFFFFu);
  int32_t u1 = (int32_t)((b >> 16) & 0xFFFFu);
  int32_t u2 = (int32_t)((b >> 32) & 0xFFFFu);
  int32_t u3 = (int32_t)((b >> 48) & 0xFFFFu);
  int32_t s = 2 * (u0 + u1 + u2 + u3) - 4 * 65535;
  return (float)s * scale;
}

DGI_FN int32_t dgi_uniform_int(uint64_t seed, uint64_t stream, uint64_t i, uint32_t n) {
  uint64_t b = dgi_bits(seed, stream, i);
  return (int32_t)(((b >> 32) * (uint64_t)n) >> 32);
}

/* fp32 -> bf16 bits, round to nearest even (NaN kept quiet). */
DGI_FN uint16_t dgi_f32_to_bf16(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  uint32_t u = v.u;
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

#endif /* DGI_H */
