// Device fill routines of the seeded input generator (see dgi.h).  Built with
// hipcc into libdgi_dev.so.  Same arithmetic as gen_host.c, from the same
// header, so device-filled tensors are bit-identical to host-filled ones.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "dgi.h"

namespace {

__global__ void k_normal_f32(float* out, int64_t n, uint64_t seed, uint64_t stream, float scale) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = dgi_normal(seed, stream, (uint64_t)i, scale);
}

__global__ void k_normal_bf16(uint16_t* out, int64_t n, uint64_t seed, uint64_t stream, float scale) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = dgi_f32_to_bf16(dgi_normal(seed, stream, (uint64_t)i, scale));
}

__global__ void k_uniform_i32(int32_t* out, int64_t n, uint64_t seed, uint64_t stream, uint32_t bound) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = dgi_uniform_int(seed, stream, (uint64_t)i, bound);
}

int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

extern "C" {

int dgi_dev_normal_f32(float* out, int64_t n, uint64_t seed, uint64_t stream, float scale, void* stream_h) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_normal_f32, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream_h, out, n, seed, stream,
                     scale);
  return (int)hipGetLastError();
}

int dgi_dev_normal_bf16(uint16_t* out, int64_t n, uint64_t seed, uint64_t stream, float scale, void* stream_h) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_normal_bf16, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream_h, out, n, seed, stream,
                     scale);
  return (int)hipGetLastError();
}

int dgi_dev_uniform_i32(int32_t* out, int64_t n, uint64_t seed, uint64_t stream, uint32_t bound, void* stream_h) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_uniform_i32, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream_h, out, n, seed, stream,
                     bound);
  return (int)hipGetLastError();
}

}  // extern "C"
