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
//                   projection)
//   k_moe_gate_up : routed experts, H = silu(X_e Wg^T) * (X_e Wu^T) per expert
//   k_moe_down    : routed experts, Y = H We_down^T per expert
// The routed kernels walk a device-side list of (expert, first pair, rows <= kMoeTileRows)
// tiles written by the routing kernels, so the host never reads routing.
#include <hip/hip_ext.h>

#include "dg_device.h"
#include "dg_kernels.h"
#include "dg_wave_gemm.h"

namespace dg {

template <typename T>
struct Depth;
template <>
struct Depth<bf16> {
  static constexpr int v = 2;     // dense tiles (4 A + 4 B fragments per step)
  static constexpr int moe1 = 4;  // routed experts, one 16-row M-tile
  static constexpr int moe2 = 3;  // routed experts, two 16-row M-tiles
  static constexpr int moe4 = 2;  // routed experts, three or four 16-row M-tiles (wide tiles)
  static constexpr int down = 6;  // routed down projection (K = ffn width, short), one or two M-tiles
};
template <>
struct Depth<float> {
  static constexpr int v = 1;
  static constexpr int moe1 = 1;
  static constexpr int moe2 = 1;
  static constexpr int moe4 = 1;
  static constexpr int down = 1;
};

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// ---------------------------------------------------------------- dense GEMM
// Workgroup tile = (16*MT) rows x (16*NT) columns; the NW waves split the K range
// NW ways (each wave reads a distinct share of both operands, so nothing is
// loaded twice inside a workgroup) and their partial tiles are summed through
// LDS in fixed wave order.  Tiles are ordered so that the row tiles sharing a
// weight tile run on one XCD and share its L2.  SwiGLU: output column c pairs
// B row c (gate) with B row N + c (up); the first NT/2 column tiles are gate
// rows and the last NT/2 the matching up rows, so the tile covers 8*NT outputs.
template <typename T, int MT, int NT, GemmEpi EPI, int DEPTH = Depth<T>::v, bool A_TILED = false, int NW = 4>
__global__ __launch_bounds__(64 * NW, 8 / NW) void k_gemm_dense(GemmArgs a) {
  constexpr bool SW = EPI == GemmEpi::SwiGLU;
  constexpr int OUTC = SW ? 8 * NT : 16 * NT;  // output columns per tile
  __shared__ f32x4 red[NW][MT * NT][64];
  const int lane = lane_id(), w = wave_id();
  const int row16 = lane & 15, kq = (lane >> 4) * 8;
  const int n_mtiles = (a.M + 16 * MT - 1) / (16 * MT);
  const int n_ntiles = (a.N + OUTC - 1) / OUTC;
  const int t = xcd_remap(blockIdx.x, n_mtiles * n_ntiles);
  const int mtile = t % n_mtiles, ntile = t / n_mtiles;
  const int m0 = mtile * 16 * MT;
  const int c0 = ntile * OUTC;  // first output column of the tile
  const int ks = a.K / 32, q = (ks + NW - 1) / NW;
  const int sb = min(w * q, ks), se = min(sb + q, ks);

  const T* A = (const T*)a.A;
  const T* B = (const T*)a.B;
  const T* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if constexpr (A_TILED) {
      ap[mt] = tiled_frag(A, min(m0 / 16 + mt, (a.M + 15) / 16 - 1), ks, sb);
    } else {
      const int r = min(m0 + 16 * mt + row16, a.M - 1);
      ap[mt] = A + (int64_t)r * a.lda + 32 * sb + kq;
    }
  }
  // weights are fragment-tiled: one row tile per 16 output columns
  const int last_rt = (a.N + 15) / 16 - 1;
  const T* bp[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int rt;
    if constexpr (SW) {
      const int ct = min(c0 / 16 + nt % (NT / 2), last_rt);
      rt = nt < NT / 2 ? ct : a.N / 16 + ct;
    } else {
      rt = min(c0 / 16 + nt, last_rt);
    }
    bp[nt] = tiled_frag(B, rt, ks, sb);
  }
  // Resid: this wave's residual inputs are requested before the K loop, so the epilogue does not wait
  // for them (the residual rows were last written long before and are usually no longer cached)
  const int rq = (lane >> 4) * 4;
  constexpr int OT = SW ? MT * NT / 2 : MT * NT;  // output tiles
  constexpr int OPW = (OT + NW - 1) / NW;          // per wave: tiles w, w + NW, ...
  float cres[OPW][4];
  if constexpr (EPI == GemmEpi::Resid) {
#pragma unroll
    for (int k = 0; k < OPW; ++k) {
      const int o = w + NW * k, mt = (o % OT) / NT, nt = o % NT;
      const int n = min(c0 + 16 * nt + row16, a.N - 1);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = min(m0 + 16 * mt + rq + r, a.M - 1);
        cres[k][r] = to_f32(((const T*)a.C)[(int64_t)m * a.ldc + n]);
      }
    }
  }
  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = zero4();
  if (se > sb) wave_gemm<T, MT, NT, DEPTH>(acc, ap, bp, se - sb, A_TILED ? kFragElems : 32, kFragElems);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) red[w][mt * NT + nt][lane] = acc[mt][nt];
  __syncthreads();

  // epilogue: wave w finishes output tiles w, w+NW, ...; lane holds column (lane & 15),
  // rows 4*(lane>>4) + r of each 16x16 tile
#pragma unroll
  for (int k = 0; k < OPW; ++k) {
    const int o = w + NW * k;
    if (o >= OT) break;
    const int mt = o / (SW ? NT / 2 : NT), nt = o % (SW ? NT / 2 : NT);
    f32x4 v = red[0][mt * NT + nt][lane];
#pragma unroll
    for (int x = 1; x < NW; ++x) v += red[x][mt * NT + nt][lane];
    f32x4 u = zero4();
    if constexpr (SW) {
      const int ut = mt * NT + nt + NT / 2;
      u = red[0][ut][lane];
#pragma unroll
      for (int x = 1; x < NW; ++x) u += red[x][ut][lane];
    }
    const int n = c0 + 16 * nt + row16;
    if (n >= a.N) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 16 * mt + rq + r;
      if (m >= a.M) continue;
      const float x = v[r];
      if constexpr (EPI == GemmEpi::Store) {
        ((T*)a.C)[(int64_t)m * a.ldc + n] = from_f32<T>(x);
      } else if constexpr (EPI == GemmEpi::Resid) {
        ((T*)a.C)[(int64_t)m * a.ldc + n] = from_f32<T>(cres[k][r] + x);
      } else if constexpr (EPI == GemmEpi::SwiGLU) {
        ((T*)a.C)[tiled_offset(m, n, a.N)] = from_f32<T>(silu(x) * u[r]);
      } else {  // QKV scatter: queries [h][m][dh], keys [h][pos][dh], values [h][dh][pos]
        const int dh = a.head_dim;
        const int hq = a.n_heads, hkv = a.n_kv_heads;
        if (n < hq * dh) {
          const int h = n / dh, c = n % dh;
          ((T*)a.q)[((int64_t)h * a.q_rows + m) * dh + c] = from_f32<T>(x);
        } else if (n < (hq + hkv) * dh) {
          const int h = (n - hq * dh) / dh, c = (n - hq * dh) % dh;
          ((T*)a.kc)[((int64_t)h * a.cap + a.pos0 + m) * dh + c] = from_f32<T>(x);
        } else {
          const int h = (n - (hq + hkv) * dh) / dh, c = (n - (hq + hkv) * dh) % dh;
          ((T*)a.vc)[((int64_t)h * dh + c) * a.cap + a.pos0 + m] = from_f32<T>(x);
        }
      }
    }
  }
}

template <typename T, int MT, int NT, GemmEpi EPI, int DEPTH = Depth<T>::v, int NW = 4>
static void launch_dense_t(const GemmArgs& a, hipStream_t s, hipEvent_t done) {
  constexpr int OUTC = EPI == GemmEpi::SwiGLU ? 8 * NT : 16 * NT;
  const int tiles = ((a.M + 16 * MT - 1) / (16 * MT)) * ((a.N + OUTC - 1) / OUTC);
  if (a.a_tiled)
    hipExtLaunchKernelGGL((k_gemm_dense<T, MT, NT, EPI, DEPTH, true, NW>), dim3(tiles), dim3(64 * NW), 0, s, nullptr, done,
                          0, a);
  else
    hipExtLaunchKernelGGL((k_gemm_dense<T, MT, NT, EPI, DEPTH, false, NW>), dim3(tiles), dim3(64 * NW), 0, s, nullptr,
                          done, 0, a);
}

// 64x64 tiles when the output is wide (K split over 8 waves and 3 steps in flight, except the SwiGLU
// pairs, which fill the chip with 4 waves, also 3 steps in flight for bf16); 16x32 tiles for narrow
// outputs (d_model < 512)
template <typename T, GemmEpi EPI>
static void launch_dense_pick(const GemmArgs& a, hipStream_t s, hipEvent_t done) {
  constexpr int D3 = sizeof(T) == 2 ? 3 : 1;
  if (a.N >= 512) {
    if constexpr (EPI == GemmEpi::SwiGLU)
      launch_dense_t<T, 4, 4, EPI, D3>(a, s, done);
    else
      launch_dense_t<T, 4, 4, EPI, D3, 8>(a, s, done);
  } else {
    launch_dense_t<T, 1, 2, EPI>(a, s, done);
  }
}

template <typename T>
hipError_t launch_gemm(GemmEpi epi, const GemmArgs& a, hipStream_t s, hipEvent_t done) {
  switch (epi) {
    case GemmEpi::Store: launch_dense_pick<T, GemmEpi::Store>(a, s, done); break;
    case GemmEpi::Resid: launch_dense_pick<T, GemmEpi::Resid>(a, s, done); break;
    case GemmEpi::QKV: launch_dense_pick<T, GemmEpi::QKV>(a, s, done); break;
    case GemmEpi::SwiGLU: launch_dense_pick<T, GemmEpi::SwiGLU>(a, s, done); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- routed experts
// Tile (e, p0, rows, n): pairs p0 .. p0+rows-1 all routed to expert e (rows <= 32, so one or two
// 16-row M-tiles); n = tiles of expert e.  The weights of an expert with one tile are read once and
// streamed with non-temporal loads; those of an expert with several tiles are loaded normally, so
// its other tiles can find them in the caches.
//
// gate_up: a workgroup owns 64 H columns of expert e, i.e. 4 gate and the 4
// matching up 16-row weight tiles; its 4 waves split K = d_model four ways, so
// every weight byte and every token-row byte is loaded exactly once per
// workgroup.  Partial tiles are summed through LDS (one 16-row M-tile per round)
// and the SwiGLU product is formed on the sum.
template <typename T, int MT, bool NTL>
__device__ __forceinline__ void moe_gate_up_body(const MoeArgs& a, f32x4 (*red)[8][64], int e, int p0, int rows,
                                                 int c0) {
  constexpr int NT = 8;
  const int lane = lane_id(), w = wave_id();
  const int row16 = lane & 15, kq = (lane >> 4) * 8;
  const int ks = a.d / 32, q = (ks + 3) / 4;
  const int sb = min(w * q, ks), se = min(sb + q, ks);
  const T* X = (const T*)a.X;
  const T* W = (const T*)a.W + (int64_t)e * 2 * a.F * a.d;
  // the weight loads need only the tile: they are issued before the row gather's indices arrive
  constexpr int D = MT == 1 ? Depth<T>::moe1 : MT == 2 ? Depth<T>::moe2 : Depth<T>::moe4;
  const T* bp[NT];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ct = min(c0 / 16 + j, a.F / 16 - 1);
    bp[j] = tiled_frag(W, ct, ks, sb);
    bp[4 + j] = tiled_frag(W, a.F / 16 + ct, ks, sb);
  }
  Frag<T> fb[D][NT];
  if (se > sb) wave_gemm_fill<T, NT, D, NTL>(fb, bp, se - sb, kFragElems);
  const T* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = min(16 * mt + row16, rows - 1);
    ap[mt] = X + (int64_t)a.perm[p0 + r] * a.d + 32 * sb + kq;
  }
  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = zero4();
  if (se > sb) {
    Frag<T> fa[D][MT];
    wave_gemm_fill<T, MT, D, false>(fa, ap, se - sb, 32);
    wave_gemm_run<T, MT, NT, D, false, NTL>(acc, fa, fb, ap, bp, se - sb, 32, kFragElems);
  }
  T* H = (T*)a.out;
  const int rq = (lane >> 4) * 4;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt) __syncthreads();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) red[w][nt][lane] = acc[mt][nt];
    __syncthreads();
    const int c = c0 + 16 * w + row16;  // wave w finishes gate tile w with up tile 4 + w
    const f32x4 g = red[0][w][lane] + red[1][w][lane] + red[2][w][lane] + red[3][w][lane];
    const f32x4 u = red[0][4 + w][lane] + red[1][4 + w][lane] + red[2][4 + w][lane] + red[3][4 + w][lane];
    if (c < a.F) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = 16 * mt + rq + r;
        if (rr < rows) H[(int64_t)(p0 + rr) * a.F + c] = from_f32<T>(silu(g[r]) * u[r]);
      }
    }
  }
}

// Routed-expert grids are 1-D: 8 * ceil(max_tiles / 8) * ncols workgroups.  The work units (tile,
// column block) are ordered expert by expert; within an expert, column block by column block, and
// within a column block, the expert's tiles.  Workgroup b runs on XCD b % 8 (round-robin dispatch) and
// XCD x takes the x-th of eight equal contiguous runs of that order (n_tiles is the device-side,
// data-dependent tile count).  So the workgroups of one tile share its activation rows in one L2, and
// the tiles of an expert routed more than 32 pairs read each weight block at about the same time on
// one XCD, where the second read hits the first one's L2 lines.
__device__ __forceinline__ bool moe_unit(const MoeArgs& a, int ncols, int n_tiles, int4& tile, int& col) {
  const int b = (int)blockIdx.x, x = b & 7, i = b >> 3;
  const int units = ncols * n_tiles, per = units / 8, rem = units % 8;
  if (i >= per + (x < rem ? 1 : 0)) return false;
  const int u = x * per + min(x, rem) + i;
  const int4 t = a.tiles[u / ncols];  // a tile of the unit's expert
  const int te = t.w & 255, j = (t.w >> 8) & 255, last = t.w >> 16;
  const int r = u - ncols * (u / ncols - j);  // unit index within the expert's ncols * te units
  const int jj = r % te;
  col = r / te;
  tile = make_int4(t.x, t.y + (jj - j) * a.tile_rows, jj == te - 1 ? last : a.tile_rows, te);
  return true;
}
static inline int moe_grid(int max_tiles, int ncols) { return 8 * ((max_tiles + 7) / 8) * ncols; }

template <typename T>
__global__ __launch_bounds__(256, 2) void k_moe_gate_up(MoeArgs a) {
  __shared__ f32x4 red[4][8][64];
  int4 tile;
  int col;
  if (!moe_unit(a, (a.F + 63) / 64, min(*a.n_tiles, a.max_tiles), tile, col)) return;
  const int c0 = col * 64;
  if (tile.w > 1) {  // weights re-read by the expert's other tiles: keep them cacheable
    if (tile.z > 16) moe_gate_up_body<T, 2, false>(a, red, tile.x, tile.y, tile.z, c0);
    else moe_gate_up_body<T, 1, false>(a, red, tile.x, tile.y, tile.z, c0);
  } else {  // weights read once: streamed (non-temporal)
    if (tile.z > 16) moe_gate_up_body<T, 2, true>(a, red, tile.x, tile.y, tile.z, c0);
    else moe_gate_up_body<T, 1, true>(a, red, tile.x, tile.y, tile.z, c0);
  }
}

// wide tiles (up to 64 rows): a separate kernel, so that the 32-row kernel keeps its register budget
template <typename T>
__global__ __launch_bounds__(256, 2) void k_moe_gate_up_wide(MoeArgs a) {
  __shared__ f32x4 red[4][8][64];
  int4 tile;
  int col;
  if (!moe_unit(a, (a.F + 63) / 64, min(*a.n_tiles, a.max_tiles), tile, col)) return;
  const int c0 = col * 64;
  if (tile.w > 1) {
    if (tile.z > 32) moe_gate_up_body<T, 4, false>(a, red, tile.x, tile.y, tile.z, c0);
    else if (tile.z > 16) moe_gate_up_body<T, 2, false>(a, red, tile.x, tile.y, tile.z, c0);
    else moe_gate_up_body<T, 1, false>(a, red, tile.x, tile.y, tile.z, c0);
  } else {
    if (tile.z > 32) moe_gate_up_body<T, 4, true>(a, red, tile.x, tile.y, tile.z, c0);
    else if (tile.z > 16) moe_gate_up_body<T, 2, true>(a, red, tile.x, tile.y, tile.z, c0);
    else moe_gate_up_body<T, 1, true>(a, red, tile.x, tile.y, tile.z, c0);
  }
}

// down: wave owns output columns [c0, c0+64) (four tiles) of expert e's [d][F]
// matrix over the full K = F; a workgroup covers 256 columns.
template <typename T, int MT, bool NTL>
__device__ __forceinline__ void moe_down_body(const MoeArgs& a, int e, int p0, int rows, int c0) {
  constexpr int NT = 4;
  const int lane = lane_id();
  const int row16 = lane & 15, kq = (lane >> 4) * 8;
  const T* H = (const T*)a.X;
  const T* W = (const T*)a.W + (int64_t)e * a.d * a.F;
  const T* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = min(16 * mt + row16, rows - 1);
    ap[mt] = H + (int64_t)(p0 + r) * a.F + kq;
  }
  const int ks = a.F / 32;
  const T* bp[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) bp[nt] = tiled_frag(W, min(c0 / 16 + nt, a.d / 16 - 1), ks, 0);
  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = zero4();
  wave_gemm<T, MT, NT, (MT <= 2 ? Depth<T>::down : Depth<T>::moe1), false, NTL>(acc, ap, bp, ks, 32, kFragElems);
  T* Y = (T*)a.out;
  const int rq = (lane >> 4) * 4;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int c = c0 + 16 * nt + row16;
      if (c >= a.d) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = 16 * mt + rq + r;
        if (rr < rows) Y[(int64_t)(p0 + rr) * a.d + c] = from_f32<T>(acc[mt][nt][r]);
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_moe_down(MoeArgs a) {
  int4 tile;
  int col;
  if (!moe_unit(a, (a.d + 255) / 256, min(*a.n_tiles, a.max_tiles), tile, col)) return;
  const int c0 = col * 256 + wave_id() * 64;
  if (c0 >= a.d) return;
  if (tile.w > 1) {
    if (tile.z > 16) moe_down_body<T, 2, false>(a, tile.x, tile.y, tile.z, c0);
    else moe_down_body<T, 1, false>(a, tile.x, tile.y, tile.z, c0);
  } else {
    if (tile.z > 16) moe_down_body<T, 2, true>(a, tile.x, tile.y, tile.z, c0);
    else moe_down_body<T, 1, true>(a, tile.x, tile.y, tile.z, c0);
  }
}

// wide tiles; held to two waves per SIMD (the four-fragment path would otherwise take the register file)
template <typename T>
__global__ __launch_bounds__(256, 2) void k_moe_down_wide(MoeArgs a) {
  int4 tile;
  int col;
  if (!moe_unit(a, (a.d + 255) / 256, min(*a.n_tiles, a.max_tiles), tile, col)) return;
  const int c0 = col * 256 + wave_id() * 64;
  if (c0 >= a.d) return;
  if (tile.w > 1) {
    if (tile.z > 32) moe_down_body<T, 4, false>(a, tile.x, tile.y, tile.z, c0);
    else if (tile.z > 16) moe_down_body<T, 2, false>(a, tile.x, tile.y, tile.z, c0);
    else moe_down_body<T, 1, false>(a, tile.x, tile.y, tile.z, c0);
  } else {
    if (tile.z > 32) moe_down_body<T, 4, true>(a, tile.x, tile.y, tile.z, c0);
    else if (tile.z > 16) moe_down_body<T, 2, true>(a, tile.x, tile.y, tile.z, c0);
    else moe_down_body<T, 1, true>(a, tile.x, tile.y, tile.z, c0);
  }
}

// ---------------------------------------------------------------- routed experts, FP8 weights
// The same work units and reductions as above with the expert weights in OCP E4M3 (FP8 pair-tiled layout, one
// float scale per output channel): each 16-byte weight load covers two K steps and is decoded to bf16 in
// registers for the bf16 matrix core; the scale of a channel multiplies its fp32 sum before the SwiGLU (gate and
// up channels each their own) or before the store (down).  Activations stay bf16.  Half the weight bytes of the
// bf16 kernels, which are bound by exactly those bytes.
// Pairs of K steps in flight (A/B/A timing of the full FP8 loop: (2, 1, 1) 8.53 ms per pass against 8.64-8.84
// for (3, 2, 3); deeper rings were slower, the down projection's occupancy covers its latency better).
struct DepthF8 {
  static constexpr int moe1 = 2;  // one 16-row M-tile
  static constexpr int moe2 = 1;  // two M-tiles
  static constexpr int moe4 = 1;  // three or four M-tiles (wide tiles)
  static constexpr int down = 1;
};

template <int MT, bool NTL>
__device__ __forceinline__ void moe_gate_up_body_f8(const MoeArgs& a, f32x4 (*red)[8][64], int e, int p0, int rows,
                                                    int c0) {
  constexpr int NT = 8;
  const int lane = lane_id(), w = wave_id();
  const int row16 = lane & 15, kq = (lane >> 4) * 8;
  const int np = a.d / 64, q = (np + 3) / 4;
  const int pb = min(w * q, np), pe = min(pb + q, np);
  const bf16* X = (const bf16*)a.X;
  const uint8_t* W = (const uint8_t*)a.W + (int64_t)e * 2 * a.F * a.d;
  constexpr int D = MT == 1 ? DepthF8::moe1 : MT == 2 ? DepthF8::moe2 : DepthF8::moe4;
  const uint8_t* bp[NT];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ct = min(c0 / 16 + j, a.F / 16 - 1);
    bp[j] = W + ((int64_t)ct * np + pb) * 1024 + lane * 16;
    bp[4 + j] = W + ((int64_t)(a.F / 16 + ct) * np + pb) * 1024 + lane * 16;
  }
  Frag8x2 fb[D][NT];
  if (pe > pb) wave_gemm_f8_fill<NT, D, NTL>(fb, bp, pe - pb, 1024);
  const bf16* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = min(16 * mt + row16, rows - 1);
    ap[mt] = X + (int64_t)a.perm[p0 + r] * a.d + 64 * pb + kq;
  }
  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = zero4();
  if (pe > pb) {
    Frag<bf16> fa[D][2][MT];
    wave_gemm_f8_fill_a<MT, D>(fa, ap, pe - pb, 32);
    wave_gemm_f8_run<MT, NT, D, NTL>(acc, fa, fb, ap, bp, pe - pb, 32, 1024);
  }
  bf16* H = (bf16*)a.out;
  const int rq = (lane >> 4) * 4;
  const int c = c0 + 16 * w + row16;  // wave w finishes gate tile w with up tile 4 + w
  const float sg = a.scale[(int64_t)e * 2 * a.F + min(c, a.F - 1)];
  const float su = a.scale[(int64_t)e * 2 * a.F + a.F + min(c, a.F - 1)];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt) __syncthreads();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) red[w][nt][lane] = acc[mt][nt];
    __syncthreads();
    const f32x4 g = red[0][w][lane] + red[1][w][lane] + red[2][w][lane] + red[3][w][lane];
    const f32x4 u = red[0][4 + w][lane] + red[1][4 + w][lane] + red[2][4 + w][lane] + red[3][4 + w][lane];
    if (c < a.F) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = 16 * mt + rq + r;
        if (rr < rows) H[(int64_t)(p0 + rr) * a.F + c] = from_f32<bf16>(silu(sg * g[r]) * (su * u[r]));
      }
    }
  }
}

__global__ __launch_bounds__(256, 2) void k_moe_gate_up_f8(MoeArgs a) {
  __shared__ f32x4 red[4][8][64];
  int4 tile;
  int col;
  if (!moe_unit(a, (a.F + 63) / 64, min(*a.n_tiles, a.max_tiles), tile, col)) return;
  const int c0 = col * 64;
  if (tile.w > 1) {
    if (tile.z > 16) moe_gate_up_body_f8<2, false>(a, red, tile.x, tile.y, tile.z, c0);
    else moe_gate_up_body_f8<1, false>(a, red, tile.x, tile.y, tile.z, c0);
  } else {
    if (tile.z > 16) moe_gate_up_body_f8<2, true>(a, red, tile.x, tile.y, tile.z, c0);
    else moe_gate_up_body_f8<1, true>(a, red, tile.x, tile.y, tile.z, c0);
  }
}

__global__ __launch_bounds__(256, 2) void k_moe_gate_up_f8_wide(MoeArgs a) {
  __shared__ f32x4 red[4][8][64];
  int4 tile;
  int col;
  if (!moe_unit(a, (a.F + 63) / 64, min(*a.n_tiles, a.max_tiles), tile, col)) return;
  const int c0 = col * 64;
  if (tile.w > 1) {
    if (tile.z > 32) moe_gate_up_body_f8<4, false>(a, red, tile.x, tile.y, tile.z, c0);
    else if (tile.z > 16) moe_gate_up_body_f8<2, false>(a, red, tile.x, tile.y, tile.z, c0);
    else moe_gate_up_body_f8<1, false>(a, red, tile.x, tile.y, tile.z, c0);
  } else {
    if (tile.z > 32) moe_gate_up_body_f8<4, true>(a, red, tile.x, tile.y, tile.z, c0);
    else if (tile.z > 16) moe_gate_up_body_f8<2, true>(a, red, tile.x, tile.y, tile.z, c0);
    else moe_gate_up_body_f8<1, true>(a, red, tile.x, tile.y, tile.z, c0);
  }
}

template <int MT, bool NTL>
__device__ __forceinline__ void moe_down_body_f8(const MoeArgs& a, int e, int p0, int rows, int c0) {
  constexpr int NT = 4;
  const int lane = lane_id();
  const int row16 = lane & 15, kq = (lane >> 4) * 8;
  const bf16* H = (const bf16*)a.X;
  const uint8_t* W = (const uint8_t*)a.W + (int64_t)e * a.d * a.F;
  const bf16* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = min(16 * mt + row16, rows - 1);
    ap[mt] = H + (int64_t)(p0 + r) * a.F + kq;
  }
  const int np = a.F / 64;
  const uint8_t* bp[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) bp[nt] = W + (int64_t)min(c0 / 16 + nt, a.d / 16 - 1) * np * 1024 + lane * 16;
  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = zero4();
  constexpr int D = MT <= 2 ? DepthF8::down : DepthF8::moe4;
  Frag8x2 fb[D][NT];
  Frag<bf16> fa[D][2][MT];
  wave_gemm_f8_fill<NT, D, NTL>(fb, bp, np, 1024);
  wave_gemm_f8_fill_a<MT, D>(fa, ap, np, 32);
  wave_gemm_f8_run<MT, NT, D, NTL>(acc, fa, fb, ap, bp, np, 32, 1024);
  bf16* Y = (bf16*)a.out;
  const int rq = (lane >> 4) * 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int c = c0 + 16 * nt + row16;
    if (c >= a.d) continue;
    const float sc = a.scale[(int64_t)e * a.d + c];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = 16 * mt + rq + r;
        if (rr < rows) Y[(int64_t)(p0 + rr) * a.d + c] = from_f32<bf16>(sc * acc[mt][nt][r]);
      }
  }
}

__global__ __launch_bounds__(256) void k_moe_down_f8(MoeArgs a) {
  int4 tile;
  int col;
  if (!moe_unit(a, (a.d + 255) / 256, min(*a.n_tiles, a.max_tiles), tile, col)) return;
  const int c0 = col * 256 + wave_id() * 64;
  if (c0 >= a.d) return;
  if (tile.w > 1) {
    if (tile.z > 16) moe_down_body_f8<2, false>(a, tile.x, tile.y, tile.z, c0);
    else moe_down_body_f8<1, false>(a, tile.x, tile.y, tile.z, c0);
  } else {
    if (tile.z > 16) moe_down_body_f8<2, true>(a, tile.x, tile.y, tile.z, c0);
    else moe_down_body_f8<1, true>(a, tile.x, tile.y, tile.z, c0);
  }
}

__global__ __launch_bounds__(256, 2) void k_moe_down_f8_wide(MoeArgs a) {
  int4 tile;
  int col;
  if (!moe_unit(a, (a.d + 255) / 256, min(*a.n_tiles, a.max_tiles), tile, col)) return;
  const int c0 = col * 256 + wave_id() * 64;
  if (c0 >= a.d) return;
  if (tile.w > 1) {
    if (tile.z > 32) moe_down_body_f8<4, false>(a, tile.x, tile.y, tile.z, c0);
    else if (tile.z > 16) moe_down_body_f8<2, false>(a, tile.x, tile.y, tile.z, c0);
    else moe_down_body_f8<1, false>(a, tile.x, tile.y, tile.z, c0);
  } else {
    if (tile.z > 32) moe_down_body_f8<4, true>(a, tile.x, tile.y, tile.z, c0);
    else if (tile.z > 16) moe_down_body_f8<2, true>(a, tile.x, tile.y, tile.z, c0);
    else moe_down_body_f8<1, true>(a, tile.x, tile.y, tile.z, c0);
  }
}

hipError_t launch_moe_gate_up_f8(const MoeArgs& a, hipStream_t s) {
  const dim3 grid(moe_grid(a.max_tiles, (a.F + 63) / 64));
  if (a.tile_rows > kMoeTileRows)
    hipLaunchKernelGGL(k_moe_gate_up_f8_wide, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_moe_gate_up_f8, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_moe_down_f8(const MoeArgs& a, hipStream_t s) {
  const dim3 grid(moe_grid(a.max_tiles, (a.d + 255) / 256));
  if (a.tile_rows > kMoeTileRows)
    hipLaunchKernelGGL(k_moe_down_f8_wide, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_moe_down_f8, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_moe_gate_up(const MoeArgs& a, hipStream_t s) {
  const dim3 grid(moe_grid(a.max_tiles, (a.F + 63) / 64));
  if (a.tile_rows > kMoeTileRows)
    hipLaunchKernelGGL(k_moe_gate_up_wide<T>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_moe_gate_up<T>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}
template <typename T>
hipError_t launch_moe_down(const MoeArgs& a, hipStream_t s) {
  const dim3 grid(moe_grid(a.max_tiles, (a.d + 255) / 256));
  if (a.tile_rows > kMoeTileRows)
    hipLaunchKernelGGL(k_moe_down_wide<T>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_moe_down<T>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_gemm<float>(GemmEpi, const GemmArgs&, hipStream_t, hipEvent_t);
template hipError_t launch_gemm<bf16>(GemmEpi, const GemmArgs&, hipStream_t, hipEvent_t);
template hipError_t launch_moe_gate_up<float>(const MoeArgs&, hipStream_t);
template hipError_t launch_moe_gate_up<bf16>(const MoeArgs&, hipStream_t);
template hipError_t launch_moe_down<float>(const MoeArgs&, hipStream_t);
template hipError_t launch_moe_down<bf16>(const MoeArgs&, hipStream_t);

}  // namespace dg
