// k_gemm.hip — matrix-core GEMMs of the denoising pass (gfx950, 64-wide waves).
//
// Every GEMM here has the form C[M, N] = A[M, K] * B[N, K]^T with both operands
// K-contiguous (activations [tokens, in] and weights [out, in]).  At batch 1 the
// token count is small (256 canvas slots; ~16 tokens per routed expert), so the
// weights are streamed from HBM once and the activations come from L2/L1.  A
// wave owns MT 16-row tiles by NT 16-column tiles over the full K range and
// reads its fragments straight from global memory into registers, keeping
// DEPTH K-steps of loads in flight (a register ring) to cover HBM latency.
//
// Kernels
//   k_gemm_dense  : dense projections (QKV with a scatter into Q / KV cache,
//                   O-projection + residual, shared-expert SwiGLU and down
//                   projection, fp32 router logits)
//   k_moe_gate_up : routed experts, H = silu(X_e Wg^T) * (X_e Wu^T) per expert
//   k_moe_down    : routed experts, Y = H We_down^T per expert
// The routed kernels walk a device-side list of (expert, first pair, rows <= kMoeTileRows)
// tiles written by the permutation kernel, so the host never reads routing.
#include "dg_device.h"
#include "dg_kernels.h"

namespace dg {

// ---------------------------------------------------------------- wave GEMM core
// acc[mt][nt] += sum_k A[row(mt)][k] * B[col(nt)][k] over ksteps 32-wide steps.
// ap[mt] / bp[nt] point at this lane's row start plus its 8*(lane>>4) K offset.
template <typename T, int MT, int NT, int DEPTH>
__device__ __forceinline__ void wave_gemm(f32x4 (&acc)[MT][NT], const T* const (&ap)[MT], const T* const (&bp)[NT],
                                          int ksteps, int mt_active) {
  Frag<T> fa[DEPTH][MT];
  Frag<T> fb[DEPTH][NT];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    if (d < ksteps) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (mt < mt_active) fa[d][mt].load(ap[mt] + 32 * d);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) fb[d][nt].load(bp[nt] + 32 * d);
    }
  }
  for (int s0 = 0; s0 < ksteps; s0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int s = s0 + d;
      if (s < ksteps) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          if (mt < mt_active) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) mma(acc[mt][nt], fa[d][mt], fb[d][nt]);
          }
        const int sn = s + DEPTH;
        if (sn < ksteps) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            if (mt < mt_active) fa[d][mt].load(ap[mt] + 32 * sn);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) fb[d][nt].load(bp[nt] + 32 * sn);
        }
      }
    }
  }
}

template <typename T>
struct Depth;
template <>
struct Depth<bf16> { static constexpr int v = 8; };
template <>
struct Depth<float> { static constexpr int v = 2; };

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// ---------------------------------------------------------------- dense GEMM
// Workgroup = 4 waves = (16*MT) rows x (64*NT) columns; wave w owns columns
// [n0 + 16*NT*w, +16*NT).  SwiGLU: the output column c pairs B row c (gate) with
// B row F + c (up), NT = 1 column tile per wave and two B streams.
template <typename T, int MT, int NT, GemmEpi EPI>
__global__ __launch_bounds__(256) void k_gemm_dense(GemmArgs a) {
  constexpr bool SW = EPI == GemmEpi::SwiGLU;
  constexpr int NB = SW ? 2 : NT;  // B streams per wave
  const int lane = lane_id(), w = wave_id();
  const int row16 = lane & 15, kq = (lane >> 4) * 8;
  const int n_mtiles = (a.M + 16 * MT - 1) / (16 * MT);
  const int n_ntiles = (a.N + 64 * NT - 1) / (64 * NT);
  const int t = xcd_remap(blockIdx.x, n_mtiles * n_ntiles);
  const int mtile = t % n_mtiles, ntile = t / n_mtiles;
  const int m0 = mtile * 16 * MT;
  const int nw0 = ntile * 64 * NT + w * 16 * NT;  // first output column of this wave
  if (nw0 >= a.N) return;
  const int mt_active = min(MT, (a.M - m0 + 15) / 16);

  const T* A = (const T*)a.A;
  const T* B = (const T*)a.B;
  const T* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int r = min(m0 + 16 * mt + row16, a.M - 1);
    ap[mt] = A + (int64_t)r * a.lda + kq;
  }
  const T* bp[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    int c = SW ? nw0 + row16 + (nb ? a.N : 0) : nw0 + 16 * nb + row16;
    int cmax = SW ? 2 * a.N - 1 : a.N - 1;
    bp[nb] = B + (int64_t)min(c, cmax) * a.ldb + kq;
  }
  f32x4 acc[MT][NB];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mt][nb] = zero4();
  wave_gemm<T, MT, NB, Depth<T>::v>(acc, ap, bp, a.K / 32, mt_active);

  // epilogue: lane holds column (lane & 15) and rows 4*(lane>>4) + r of each tile
  const int rq = (lane >> 4) * 4;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt >= mt_active) continue;
#pragma unroll
    for (int nt = 0; nt < (SW ? 1 : NT); ++nt) {
      const int n = nw0 + 16 * nt + row16;
      if (n >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * mt + rq + r;
        if (m >= a.M) continue;
        float v = acc[mt][nt][r];
        if constexpr (EPI == GemmEpi::Store) {
          ((T*)a.C)[(int64_t)m * a.ldc + n] = from_f32<T>(v);
        } else if constexpr (EPI == GemmEpi::StoreF32) {
          ((float*)a.C)[(int64_t)m * a.ldc + n] = v;
        } else if constexpr (EPI == GemmEpi::Resid) {
          T* c = (T*)a.C + (int64_t)m * a.ldc + n;
          *c = from_f32<T>(to_f32(*c) + v);
        } else if constexpr (EPI == GemmEpi::SwiGLU) {
          ((T*)a.C)[(int64_t)m * a.ldc + n] = from_f32<T>(silu(v) * acc[mt][1][r]);
        } else {  // QKV scatter
          const int dh = a.head_dim;
          const int hq = a.n_heads, hkv = a.n_kv_heads;
          if (n < hq * dh) {
            int h = n / dh, c = n % dh;
            ((T*)a.q)[((int64_t)h * a.q_rows + m) * dh + c] = from_f32<T>(v);
          } else if (n < (hq + hkv) * dh) {
            int h = (n - hq * dh) / dh, c = (n - hq * dh) % dh;
            ((T*)a.kc)[((int64_t)h * a.cap + a.pos0 + m) * dh + c] = from_f32<T>(v);
          } else {
            int h = (n - (hq + hkv) * dh) / dh, c = (n - (hq + hkv) * dh) % dh;
            ((T*)a.vc)[((int64_t)h * dh + c) * a.cap + a.pos0 + m] = from_f32<T>(v);
          }
        }
      }
    }
  }
}

template <typename T>
hipError_t launch_gemm(GemmEpi epi, const GemmArgs& a, hipStream_t s) {
  constexpr int MT = 4;
  auto grid_for = [&](int nt) {
    int mt = (a.M + 16 * MT - 1) / (16 * MT);
    int ntl = (a.N + 64 * nt - 1) / (64 * nt);
    return dim3(mt * ntl);
  };
  switch (epi) {
    case GemmEpi::Store:
      hipLaunchKernelGGL((k_gemm_dense<T, MT, 1, GemmEpi::Store>), grid_for(1), dim3(256), 0, s, a);
      break;
    case GemmEpi::StoreF32:
      hipLaunchKernelGGL((k_gemm_dense<T, MT, 1, GemmEpi::StoreF32>), grid_for(1), dim3(256), 0, s, a);
      break;
    case GemmEpi::Resid:
      hipLaunchKernelGGL((k_gemm_dense<T, MT, 1, GemmEpi::Resid>), grid_for(1), dim3(256), 0, s, a);
      break;
    case GemmEpi::QKV:
      hipLaunchKernelGGL((k_gemm_dense<T, MT, 1, GemmEpi::QKV>), grid_for(1), dim3(256), 0, s, a);
      break;
    case GemmEpi::SwiGLU:
      hipLaunchKernelGGL((k_gemm_dense<T, MT, 1, GemmEpi::SwiGLU>), grid_for(1), dim3(256), 0, s, a);
      break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- routed experts
// grid = (column tiles, max tiles).  Tile (e, p0, rows): pairs p0 .. p0+rows-1 all
// routed to expert e.  gate_up: wave owns H columns [c0, c0+16) and reads gate
// rows c0.. and up rows F+c0.. of expert e; A rows are the routed tokens' rows.
template <typename T>
__global__ __launch_bounds__(256) void k_moe_gate_up(MoeArgs a) {
  constexpr int MT = kMoeTileRows / 16;
  const int tile_i = blockIdx.y;
  if (tile_i >= *a.n_tiles) return;
  const int4 tile = a.tiles[tile_i];
  const int e = tile.x, p0 = tile.y, rows = tile.z;
  const int lane = lane_id(), w = wave_id();
  const int row16 = lane & 15, kq = (lane >> 4) * 8;
  const int c0 = blockIdx.x * 64 + w * 16;
  if (c0 >= a.F) return;
  const int mt_active = (rows + 15) / 16;
  const T* X = (const T*)a.X;
  const T* W = (const T*)a.W + (int64_t)e * 2 * a.F * a.d;
  const T* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int r = min(16 * mt + row16, rows - 1);
    int tok = a.perm[p0 + r];
    ap[mt] = X + (int64_t)tok * a.d + kq;
  }
  const T* bp[2] = {W + (int64_t)(c0 + row16) * a.d + kq, W + (int64_t)(a.F + c0 + row16) * a.d + kq};
  f32x4 acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) { acc[mt][0] = zero4(); acc[mt][1] = zero4(); }
  wave_gemm<T, MT, 2, Depth<T>::v>(acc, ap, bp, a.d / 32, mt_active);
  T* H = (T*)a.out;
  const int rq = (lane >> 4) * 4;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt >= mt_active) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int rr = 16 * mt + rq + r;
      if (rr < rows) H[(int64_t)(p0 + rr) * a.F + c0 + row16] = from_f32<T>(silu(acc[mt][0][r]) * acc[mt][1][r]);
    }
  }
}

// down: wave owns output columns [c0, c0+32) (two tiles) of expert e's [d][F] matrix.
template <typename T>
__global__ __launch_bounds__(256) void k_moe_down(MoeArgs a) {
  constexpr int MT = kMoeTileRows / 16, NT = 2;
  const int tile_i = blockIdx.y;
  if (tile_i >= *a.n_tiles) return;
  const int4 tile = a.tiles[tile_i];
  const int e = tile.x, p0 = tile.y, rows = tile.z;
  const int lane = lane_id(), w = wave_id();
  const int row16 = lane & 15, kq = (lane >> 4) * 8;
  const int c0 = blockIdx.x * 128 + w * 32;
  if (c0 >= a.d) return;
  const int mt_active = (rows + 15) / 16;
  const T* H = (const T*)a.X;
  const T* W = (const T*)a.W + (int64_t)e * a.d * a.F;
  const T* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int r = min(16 * mt + row16, rows - 1);
    ap[mt] = H + (int64_t)(p0 + r) * a.F + kq;
  }
  const T* bp[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) bp[nt] = W + (int64_t)min(c0 + 16 * nt + row16, a.d - 1) * a.F + kq;
  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = zero4();
  wave_gemm<T, MT, NT, Depth<T>::v>(acc, ap, bp, a.F / 32, mt_active);
  T* Y = (T*)a.out;
  const int rq = (lane >> 4) * 4;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt >= mt_active) continue;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      int c = c0 + 16 * nt + row16;
      if (c >= a.d) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int rr = 16 * mt + rq + r;
        if (rr < rows) Y[(int64_t)(p0 + rr) * a.d + c] = from_f32<T>(acc[mt][nt][r]);
      }
    }
  }
}

template <typename T>
hipError_t launch_moe_gate_up(const MoeArgs& a, hipStream_t s) {
  dim3 grid((a.F + 63) / 64, a.max_tiles);
  hipLaunchKernelGGL(k_moe_gate_up<T>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}
template <typename T>
hipError_t launch_moe_down(const MoeArgs& a, hipStream_t s) {
  dim3 grid((a.d + 127) / 128, a.max_tiles);
  hipLaunchKernelGGL(k_moe_down<T>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_gemm<float>(GemmEpi, const GemmArgs&, hipStream_t);
template hipError_t launch_gemm<bf16>(GemmEpi, const GemmArgs&, hipStream_t);
template hipError_t launch_moe_gate_up<float>(const MoeArgs&, hipStream_t);
template hipError_t launch_moe_gate_up<bf16>(const MoeArgs&, hipStream_t);
template hipError_t launch_moe_down<float>(const MoeArgs&, hipStream_t);
template hipError_t launch_moe_down<bf16>(const MoeArgs&, hipStream_t);

}  // namespace dg
