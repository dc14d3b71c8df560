/* Host fill routines of the seeded input generator (see dgi.h).  Built with gcc
 * into libdgi_host.so; OpenMP spreads large fills over the host cores. */
#include <stddef.h>
#include <stdint.h>
#include "dgi.h"

void dgi_host_normal_f32(float* out, int64_t n, uint64_t seed, uint64_t stream, float scale) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = dgi_normal(seed, stream, (uint64_t)i, scale);
}

void dgi_host_normal_bf16(uint16_t* out, int64_t n, uint64_t seed, uint64_t stream, float scale) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = dgi_f32_to_bf16(dgi_normal(seed, stream, (uint64_t)i, scale));
}

void dgi_host_uniform_i32(int32_t* out, int64_t n, uint64_t seed, uint64_t stream, uint32_t bound) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = dgi_uniform_int(seed, stream, (uint64_t)i, bound);
}

/* Offset variants: values for indices [first, first+n) of the stream, so that a
 * large tensor can be produced slice by slice with the same result. */
void dgi_host_normal_bf16_range(uint16_t* out, int64_t first, int64_t n, uint64_t seed, uint64_t stream,
                                float scale) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = dgi_f32_to_bf16(dgi_normal(seed, stream, (uint64_t)(first + i), scale));
}

void dgi_host_normal_f32_range(float* out, int64_t first, int64_t n, uint64_t seed, uint64_t stream,
                               float scale) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = dgi_normal(seed, stream, (uint64_t)(first + i), scale);
}
