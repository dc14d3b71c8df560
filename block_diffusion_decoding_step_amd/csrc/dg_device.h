// dg_device.h — gfx950 (CDNA4) device primitives shared by the libdg kernels.
//
// Matrix-core convention (v_mfma_f32_16x16x32_bf16 and v_mfma_f32_16x16x4_f32):
//   A fragment: lane l holds row (l & 15) and 8 consecutive K elements at
//               k0 + 8*(l >> 4) .. +8 (one 16-byte load for bf16, two for fp32)
//   B fragment: lane l holds column (l & 15), same 8 K elements
//   C tile    : lane l holds column (l & 15), rows 4*(l >> 4) + r, r = 0..3
// A 32-wide K step is one bf16 MFMA, or eight fp32 MFMAs that each take the
// j-th of the lane's 8 elements (the K order inside a step is a permutation
// applied identically to A and B, so the sum is unchanged).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }
__device__ __forceinline__ int wave_id() { return (int)(threadIdx.x >> 6); }

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // round to nearest even

// ---------------------------------------------------------------- fragments
template <typename T>
struct Frag;

template <>
struct Frag<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const bf16x8*>(p); }
  // streaming (non-temporal) load: data read once should not displace reused data in the caches
  __device__ __forceinline__ void load_nt(const bf16* p) {
    v = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
  }
  __device__ __forceinline__ void zero() {
    u32x4 z = {0u, 0u, 0u, 0u};
    v = __builtin_bit_cast(bf16x8, z);
  }
  __device__ __forceinline__ void set(int j, float x) { v[j] = (bf16)x; }
  __device__ __forceinline__ float get(int j) const { return (float)v[j]; }
};

template <>
struct Frag<float> {
  f32x4 lo, hi;
  __device__ __forceinline__ void load(const float* p) {
    lo = *reinterpret_cast<const f32x4*>(p);
    hi = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ void load_nt(const float* p) {
    lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
  }
  __device__ __forceinline__ void zero() {
    lo = f32x4{0.f, 0.f, 0.f, 0.f};
    hi = lo;
  }
  __device__ __forceinline__ void set(int j, float x) {
    if (j < 4) lo[j] = x; else hi[j - 4] = x;
  }
  __device__ __forceinline__ float get(int j) const { return j < 4 ? lo[j] : hi[j - 4]; }
};

// FP8 (OCP E4M3) operand of two consecutive 32-wide K steps: one 16-byte load per lane, whose two 8-byte halves
// are the lane's elements of the two steps (the FP8 pair-tiled layout).  E4M3 values are exact in bf16, so the
// pair decodes without rounding into two bf16 fragments for the bf16 matrix core.
struct Frag8x2 {
  u32x4 v;
  __device__ __forceinline__ void load(const uint8_t* p) { v = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void load_nt(const uint8_t* p) {
    v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  // half h (0: first K step, 1: second) as a bf16 fragment
  __device__ __forceinline__ Frag<bf16> half(int h) const;
};

// eight E4M3 codes (bytes of w in order, the low byte first) as a bf16 fragment; exact, since every E4M3
// value is a bf16 value
__device__ __forceinline__ Frag<bf16> fp8x8_to_bf16(u32x2 w) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
  Frag<bf16> f;
  f.v = bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return f;
}
__device__ __forceinline__ Frag<bf16> Frag8x2::half(int h) const {
  return fp8x8_to_bf16(h ? u32x2{v[2], v[3]} : u32x2{v[0], v[1]});
}

// acc += A(16 x 32) * B(32 x 16) for one 32-wide K step
__device__ __forceinline__ void mma(f32x4& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[j], b.lo[j], acc, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[j], b.hi[j], acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------- 8-wide vector IO
template <typename T>
struct Vec8;
template <>
struct Vec8<bf16> {
  static __device__ __forceinline__ void load(const bf16* p, float* out) {
    bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = (float)v[j];
  }
  static __device__ __forceinline__ void store(bf16* p, const float* in) {
    bf16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (bf16)in[j];
    *reinterpret_cast<bf16x8*>(p) = v;
  }
};
template <>
struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* out) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) { out[j] = a[j]; out[j + 4] = b[j]; }
  }
  static __device__ __forceinline__ void store(float* p, const float* in) {
    *reinterpret_cast<f32x4*>(p) = f32x4{in[0], in[1], in[2], in[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{in[4], in[5], in[6], in[7]};
  }
};

// ---------------------------------------------------------------- Philox4x32-10
// Counter-based generator of Salmon, Moraes, Dror and Shaw ("Parallel Random Numbers: As Easy
// as 1, 2, 3", SC'11): ten rounds; each round forms the 64-bit products of counter words 0 and 2
// with two fixed multipliers, moves their low halves to words 3 and 1 and xors their high halves
// with words 1 / 3 and the key; the key advances by two Weyl constants between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    const uint64_t p0 = (uint64_t)M0 * c0;
    const uint64_t p1 = (uint64_t)M1 * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  return uint4{c0, c1, c2, c3};
}

// 64-bit integer min / max as plain compares (the generic min/max overloads may go through double)
__device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }
__device__ __forceinline__ int64_t imax64(int64_t a, int64_t b) { return a > b ? a : b; }

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Remap a linear workgroup id so that each of the 8 XCDs (dispatched round-robin
// by workgroup id) receives one contiguous range of logical tiles; tiles that
// share operands then share an L2.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int nx = 8;
  int per = total / nx, rem = total % nx;
  int x = b % nx, i = b / nx;
  // XCD x owns per + (x < rem) tiles starting at x*per + min(x, rem)
  int start = x * per + (x < rem ? x : rem);
  int cnt = per + (x < rem ? 1 : 0);
  return i < cnt ? start + i : b;  // b beyond the balanced split keeps its own id
}

}  // namespace dg
