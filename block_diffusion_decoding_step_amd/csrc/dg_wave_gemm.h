// dg_wave_gemm.h — one wave's share of a K-contiguous GEMM on the gfx950 matrix core.
#pragma once

#include "dg_device.h"

namespace dg {

// Fragment-tiled matrices: 16-row x 32-column blocks of kFragElems elements.
constexpr int kFragElems = 512;

// Element (r, c) of a fragment-tiled [rows, K] matrix (K a multiple of 32, rows padded to 16): the
// 16-row x 32-column block (r/16, c/32) is one contiguous fragment in the matrix cores' operand order.
__device__ __forceinline__ int64_t tiled_offset(int64_t r, int c, int K) {
  return ((r >> 4) * (K >> 5) + (c >> 5)) * (int64_t)kFragElems + ((r & 15) + 16 * ((c & 31) >> 3)) * 8 + (c & 7);
}

// Pointer to this lane's part of fragment (row tile rt, K step s) of a tiled matrix with ks K steps.
template <typename T>
__device__ __forceinline__ const T* tiled_frag(const T* base, int64_t rt, int ks, int s) {
  return base + ((rt * ks + s) * kFragElems + (int64_t)lane_id() * 8);
}

// ---------------------------------------------------------------- wave GEMM core
// acc[mt][nt] += sum_k A[row(mt)][k] * B[col(nt)][k] over ksteps 32-wide steps.
// ap[mt] / bp[nt] point at this lane's first fragment; consecutive K steps are sa
// (A) and sb (B) elements apart: 32 for a row-major operand, 512 for a
// fragment-tiled one (one contiguous 16x32 fragment per step).
// Software pipeline with a ring of DEPTH register buffers and no branches in the
// steady state: step s + DEPTH is loaded into the buffer step s just used, at an
// index clamped to the last step (the few clamped reloads at the end are never
// consumed), so the compiler can wait for exactly the oldest loads in flight.
template <bool STREAM, typename T>
__device__ __forceinline__ void frag_load(Frag<T>& f, const T* p) {
  if constexpr (STREAM) f.load_nt(p); else f.load(p);
}

// The first DEPTH steps of each operand (the pipeline's fill), issued separately so that a caller
// can start the B loads before the A addresses are known.
template <typename T, int NT, int DEPTH, bool STREAM>
__device__ __forceinline__ void wave_gemm_fill(Frag<T> (&f)[DEPTH][NT], const T* const (&p)[NT], int ksteps, int stride) {
  const int last = ksteps - 1;
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) frag_load<STREAM>(f[d][nt], p[nt] + (int64_t)stride * min(d, last));
}

// The steady state and the tail, on rings already filled by wave_gemm_fill.
template <typename T, int MT, int NT, int DEPTH, bool SA, bool SB>
__device__ __forceinline__ void wave_gemm_run(f32x4 (&acc)[MT][NT], Frag<T> (&fa)[DEPTH][MT], Frag<T> (&fb)[DEPTH][NT],
                                              const T* const (&ap)[MT], const T* const (&bp)[NT], int ksteps, int sa,
                                              int sb) {
  const int last = ksteps - 1;
  int s0 = 0;
  for (; s0 + DEPTH <= ksteps; s0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) mma(acc[mt][nt], fa[d][mt], fb[d][nt]);
      const int sn = min(s0 + DEPTH + d, last);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) frag_load<SA>(fa[d][mt], ap[mt] + (int64_t)sa * sn);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) frag_load<SB>(fb[d][nt], bp[nt] + (int64_t)sb * sn);
    }
  }
  const int rem = ksteps - s0;  // steps s0 .. ksteps-1 sit in buffers 0 .. rem-1
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (d < rem) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) mma(acc[mt][nt], fa[d][mt], fb[d][nt]);
    }
}

// SA / SB: operand read once per launch (weights), loaded non-temporally.
template <typename T, int MT, int NT, int DEPTH, bool SA = false, bool SB = false>
__device__ __forceinline__ void wave_gemm(f32x4 (&acc)[MT][NT], const T* const (&ap)[MT], const T* const (&bp)[NT],
                                          int ksteps, int sa = 32, int sb = 32) {
  Frag<T> fa[DEPTH][MT];
  Frag<T> fb[DEPTH][NT];
  wave_gemm_fill<T, MT, DEPTH, SA>(fa, ap, ksteps, sa);
  wave_gemm_fill<T, NT, DEPTH, SB>(fb, bp, ksteps, sb);
  wave_gemm_run<T, MT, NT, DEPTH, SA, SB>(acc, fa, fb, ap, bp, ksteps, sa, sb);
}

// ---------------------------------------------------------------- FP8 B operand (routed experts)
// acc[mt][nt] += sum_k A[row(mt)][k] * B[col(nt)][k] over npairs pairs of 32-wide K steps, with A in bf16 (ap:
// this lane's first fragment, consecutive K steps sa elements apart) and B in the FP8 pair-tiled layout (bp:
// this lane's first 16 bytes, consecutive pairs sb bytes apart; decoded to bf16 in registers).  Same ring
// discipline as wave_gemm: DEPTH pairs of loads in flight, clamped reloads at the end, no branches in the
// steady state.
template <int NT, int DEPTH, bool STREAM>
__device__ __forceinline__ void wave_gemm_f8_fill(Frag8x2 (&f)[DEPTH][NT], const uint8_t* const (&p)[NT], int npairs,
                                                  int stride) {
  const int last = npairs - 1;
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if constexpr (STREAM) f[d][nt].load_nt(p[nt] + (int64_t)stride * min(d, last));
      else f[d][nt].load(p[nt] + (int64_t)stride * min(d, last));
    }
}

template <int MT, int DEPTH>
__device__ __forceinline__ void wave_gemm_f8_fill_a(Frag<bf16> (&f)[DEPTH][2][MT], const bf16* const (&p)[MT],
                                                    int npairs, int sa) {
  const int last = npairs - 1;
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) f[d][h][mt].load(p[mt] + (int64_t)sa * (2 * min(d, last) + h));
}

template <int MT, int NT, int DEPTH, bool SB>
__device__ __forceinline__ void wave_gemm_f8_run(f32x4 (&acc)[MT][NT], Frag<bf16> (&fa)[DEPTH][2][MT],
                                                 Frag8x2 (&fb)[DEPTH][NT], const bf16* const (&ap)[MT],
                                                 const uint8_t* const (&bp)[NT], int npairs, int sa, int sb) {
  const int last = npairs - 1;
  int s0 = 0;
  for (; s0 + DEPTH <= npairs; s0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const Frag<bf16> b0 = fb[d][nt].half(0), b1 = fb[d][nt].half(1);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          mma(acc[mt][nt], fa[d][0][mt], b0);
          mma(acc[mt][nt], fa[d][1][mt], b1);
        }
      }
      const int sn = min(s0 + DEPTH + d, last);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) fa[d][h][mt].load(ap[mt] + (int64_t)sa * (2 * sn + h));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if constexpr (SB) fb[d][nt].load_nt(bp[nt] + (int64_t)sb * sn);
        else fb[d][nt].load(bp[nt] + (int64_t)sb * sn);
      }
    }
  }
  const int rem = npairs - s0;
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (d < rem) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const Frag<bf16> b0 = fb[d][nt].half(0), b1 = fb[d][nt].half(1);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          mma(acc[mt][nt], fa[d][0][mt], b0);
          mma(acc[mt][nt], fa[d][1][mt], b1);
        }
      }
    }
}

}  // namespace dg
