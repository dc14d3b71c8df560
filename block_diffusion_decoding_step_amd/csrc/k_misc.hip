// k_misc.hip — the memory-light stages of a denoising pass:
//   embedding gather, RMSNorm, MoE routing (FFN norm + router logits + top-k, then softmax and the
//   token->expert order),
//   MoE combine + residual, stop check and the Philox canvas update.
// Page tags: [P2] "DiffusionGemma 26B: How Google's Text Diffusion Model Generates
// Tokens in Parallel"; [P5] "When to use a diffusion LLM: I compared DiffusionGemma
// and Gemma 4".
#include <hip/hip_ext.h>

#include <algorithm>

#include "dg_device.h"
#include "dg_kernels.h"
#include "dg_wave_gemm.h"

namespace dg {

// ============================================================== embedding
// X[m, :] = E[tok[m], :] with E fragment-tiled; tokens outside [0, V) are clamped
// into range.  Thread i copies the 8 elements (K step i/4, quarter i%4) of its row.
template <typename T>
__global__ __launch_bounds__(256) void k_embed(const int32_t* __restrict__ tok, const T* __restrict__ E,
                                               T* __restrict__ X, int M, int d, int V) {
  const int m = blockIdx.x;
  if (m >= M) return;
  int t = tok[m];
  t = t < 0 ? 0 : (t >= V ? V - 1 : t);
  const int ks = d / 32;
  const T* tile = E + (int64_t)(t >> 4) * ks * 512;
  for (int i = threadIdx.x; i < d / 8; i += blockDim.x) {
    const int s = i >> 2, q = i & 3;
    float v[8];
    Vec8<T>::load(tile + ((int64_t)s * 512 + ((t & 15) + 16 * q) * 8), v);
    Vec8<T>::store(X + (int64_t)m * d + 8 * i, v);
  }
}

// X[m, :] = bf16(code * s) for an E4M3 embedding in the FP8 pair-tiled layout (dg.h, dg_quantize_e4m3) with
// one float scale per vocabulary row: the 8 codes of columns 8i .. 8i+7 are 8 contiguous bytes of the row's
// 64-column block, decoded exactly to bf16 (every E4M3 value is a bf16 value), widened, scaled in fp32 and
// rounded to bf16.  Tokens outside [0, V) are clamped into range.
__global__ __launch_bounds__(256) void k_embed_f8(const int32_t* __restrict__ tok, const uint8_t* __restrict__ E,
                                                  const float* __restrict__ scale, bf16* __restrict__ X, int M, int d,
                                                  int V) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const int m = blockIdx.x;
  if (m >= M) return;
  int t = tok[m];
  t = t < 0 ? 0 : (t >= V ? V - 1 : t);
  const float s = scale[t];
  const uint8_t* tile = E + (int64_t)(t >> 4) * (d / 64) * 1024;
  for (int i = threadIdx.x; i < d / 8; i += blockDim.x) {
    const int c = 8 * i;
    const uint2 w = *reinterpret_cast<const uint2*>(tile + (c >> 6) * 1024 + ((t & 15) + 16 * ((c & 31) >> 3)) * 16 +
                                                    ((c & 63) >> 5) * 8);
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false);
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true);
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false);
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true);
    float v[8] = {(float)p0[0], (float)p0[1], (float)p1[0], (float)p1[1],
                  (float)p2[0], (float)p2[1], (float)p3[0], (float)p3[1]};
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] *= s;
    Vec8<bf16>::store(X + (int64_t)m * d + c, v);
  }
}

// ============================================================== weight packing
// Row-major [rows, cols] -> fragment-tiled (see dg.h); thread i writes 8 elements:
// fragment i/64 (row tile, K step) and lane i%64 of it.
template <typename T>
__global__ __launch_bounds__(256) void k_pack(const T* __restrict__ src, T* __restrict__ dst, int64_t batch,
                                              int64_t rows, int64_t cols, int64_t rows_p) {
  const int64_t ks = cols / 32;
  const int64_t per = rows_p / 16 * ks * 64;  // 8-element chunks per matrix
  const int64_t total = batch * per;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t b = i / per, rem = i % per;
    const int lane = (int)(rem & 63);
    const int64_t frag = rem >> 6;
    const int64_t s = frag % ks, rt = frag / ks;
    const int64_t r = rt * 16 + (lane & 15), c = s * 32 + (lane >> 4) * 8;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (r < rows) Vec8<T>::load(src + (b * rows + r) * cols + c, v);
    Vec8<T>::store(dst + b * rows_p * cols + rem * 8, v);
  }
}

// ============================================================== FP8 (OCP E4M3) weight quantisation
// Per-row (output channel) scale s = amax / 448 in fp32 (1 for an all-zero row); each weight w becomes the
// E4M3 code of w / s rounded to nearest, ties to the even mantissa, magnitudes beyond 448 saturated.  E4M3 is
// the OCP 8-bit float with 4 exponent bits (bias 7) and 3 mantissa bits, subnormals 0.mmm * 2^-6 and no
// infinities (0x7F / 0xFF are NaN, 448 the largest finite value).
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u, mag = u & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return sign | 0x7Fu;                      // NaN
  const float a = __uint_as_float(mag);
  if (a >= 448.f) return sign | 0x7Eu;                             // saturate
  if (a < 0.015625f) return sign | (uint32_t)(int)rintf(a * 512.f);  // subnormal spacing 2^-9 (8 -> 2^-6)
  int e = (int)((mag >> 23) & 0xFF) - 127 + 7;                     // biased E4M3 exponent, 1 .. 15
  uint32_t keep = (mag >> 20) & 7u, rest = mag & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
  if (keep == 8u) { keep = 0u; ++e; }
  if (e > 15 || (e == 15 && keep == 7u)) return sign | 0x7Eu;
  return sign | ((uint32_t)e << 3) | keep;
}

// amax of each row of `batch` row-major [rows, cols] bf16 matrices -> scale; one wave per row
__global__ __launch_bounds__(256) void k_e4m3_scales(const bf16* __restrict__ src, float* __restrict__ scale,
                                                     int64_t n_rows, int64_t cols) {
  const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
  if (row >= n_rows) return;
  const bf16* p = src + row * cols;
  float m = 0.f;
  for (int64_t c = lane_id(); c < cols; c += 64) m = fmaxf(m, fabsf((float)p[c]));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (lane_id() == 0) scale[row] = m > 0.f ? m / 448.f : 1.f;
}

// codes in the FP8 pair-tiled layout: 16-row x 64-column blocks of 1024 bytes; lane l's 16 bytes hold row
// (l & 15), columns 8 (l >> 4) .. +8 of the block's first 32-wide half, then the same of its second half
// (one 16-byte load gives a lane its A/B fragment elements of two consecutive 32-wide K steps); padded rows 0
__global__ __launch_bounds__(256) void k_e4m3_pack(const bf16* __restrict__ src, const float* __restrict__ scale,
                                                   uint8_t* __restrict__ dst, int64_t batch, int64_t rows,
                                                   int64_t cols, int64_t rows_p) {
  const int64_t kp = cols / 64;
  const int64_t per = rows_p / 16 * kp * 64;  // 16-byte lane chunks per matrix
  const int64_t total = batch * per;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t b = i / per, rem = i % per;
    const int lane = (int)(rem & 63);
    const int64_t blk = rem >> 6;
    const int64_t pk = blk % kp, rt = blk / kp;
    const int64_t r = rt * 16 + (lane & 15), c = pk * 64 + (lane >> 4) * 8;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (r < rows) {
      const bf16* row = src + (b * rows + r) * cols;
      const float sc = scale[b * rows + r];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t q = e4m3_rne((float)row[c + 32 * h + j] / sc);
          w[2 * h + j / 4] |= q << (8 * (j % 4));
        }
    }
    *reinterpret_cast<uint4*>(dst + (b * rows_p * cols) + rem * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ============================================================== RMSNorm
// Y = X / sqrt(mean(X^2) + eps) * g, fp32 statistics.  One workgroup per row, one thread per 8
// consecutive columns (blockDim = 64 * ceil(d / 512)); the sum of squares is reduced in a fixed
// order (within each wave, then across waves in wave order), shared with the combine kernel's fused
// normalisation below so that both give bit-identical rows.  Written row-major to Y and / or
// fragment-tiled to Yt (the layout the matrix-core GEMMs read their A operand in).
__device__ __forceinline__ float row_sum_sq(float ss) {
  __shared__ float part[16];
  ss = wave_sum(ss);
  if (lane_id() == 0) part[wave_id()] = ss;
  __syncthreads();
  float t = 0.f;
  const int nw = (int)(blockDim.x >> 6);
  for (int i = 0; i < nw; ++i) t += part[i];
  return t;
}

template <typename T>
__device__ __forceinline__ void store_norm_row(const float (&v)[8], float r, const T* __restrict__ g, int c, int row,
                                               int d, T* __restrict__ Y, T* __restrict__ Yt) {
  float gv[8], o[8];
  Vec8<T>::load(g + c, gv);
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = v[j] * r * gv[j];
  if (Y) Vec8<T>::store(Y + (int64_t)row * d + c, o);
  if (Yt) Vec8<T>::store(Yt + tiled_offset(row, c, d), o);
}

template <typename T>
__global__ __launch_bounds__(1024) void k_rmsnorm(const T* __restrict__ X, const T* __restrict__ g,
                                                  T* __restrict__ Y, T* __restrict__ Yt, int M, int d, float eps) {
  const int row = blockIdx.x;
  const int c = threadIdx.x * 8;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  if (c < d) {
    Vec8<T>::load(X + (int64_t)row * d + c, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += v[j] * v[j];
  }
  ss = row_sum_sq(ss);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  if (c < d) store_norm_row<T>(v, r, g, c, row, d, Y, Yt);
}

// ============================================================== routing
// Everything between the FFN RMSNorm and the routed experts, in two launches: the fp32 router
// logits, top-k with ties to the lower expert id and a softmax over the k chosen ([P2] "Architecture
// Details": 8 of 128 experts active per token, plus one shared expert that is always applied), and
// the order of the (token, choice) pairs by (expert, token) that the grouped expert GEMMs walk, with
// their list of (expert, first pair, rows <= kMoeTileRows, tiles of the expert) work tiles.
//
// k_route_logits<T, NT>: workgroup (row tile rt, expert slice es) of a ceil(M/16) x ES grid (ES <= 2
// slices of 16*NT experts), 8 waves that split K = d eight ways; no workgroup waits for another.
//  1. the 16 FFN-normalised rows (fragment-tiled) against the slice's NT router weight tiles, DB K
//     steps of loads in flight; partial tiles summed in wave order through LDS: the slice's logits;
//  2. per row, the slice's k best, best first, by k rounds of an arg-max across one 16-lane row (DPP
//     lane exchanges).
// k_route_order (one workgroup): per row, the k best of the slices' sorted candidates (ranked across
// the two lists by four threads) and the softmax weights; an LDS mask of 64 tokens per (expert, 64-token chunk), built with atomic ORs, gives
// every pair's rank among its expert's pairs as a prefix count, so the order is (expert, token).
constexpr int kRouteWaves = 8;
template <typename T>
struct RouteDepth;
template <>
struct RouteDepth<bf16> {
  static constexpr int b = 6;  // K steps of loads in flight (of 11 per wave at d = 2816)
};
template <>
struct RouteDepth<float> {
  static constexpr int b = 1;
};
__host__ __device__ inline int route_tiles(int E) { return E <= 128 ? 4 : 8; }  // 16-expert tiles per workgroup: two slices at most

// the better of two (logit, expert) candidates: larger logit, then lower expert id
__device__ __forceinline__ bool route_better(float v, int e, float bv, int be) {
  return v > bv || (v == bv && e < be);
}
// the same order over candidates that may be empty (expert -1, below every other), as one unsigned
// 64-bit key (larger key = better candidate): the logit's bits mapped
// monotonically to an unsigned word (-0 taken as +0, so equal logits tie), then the inverted expert
// id; an empty candidate is 0, below every other
__device__ __forceinline__ unsigned long long route_key(float v, int e) {
  uint32_t u = __float_as_uint(v + 0.0f);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return e < 0 ? 0ull : ((unsigned long long)u << 32) | (uint32_t)(0x7fffffff - e);
}
// arg-max step across a 16-lane row: exchange with the lane the DPP control names
template <int CTRL>
__device__ __forceinline__ void route_argmax_step(float& bv, int& be) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bv), CTRL, 0xF, 0xF, false));
  const int oe = __builtin_amdgcn_update_dpp(0, be, CTRL, 0xF, 0xF, false);
  if (route_better(ov, oe, bv, be)) { bv = ov; be = oe; }
}
// every lane of each 16-lane row ends with the row's best: swap neighbours (quad_perm 1,0,3,2), pairs
// (quad_perm 2,3,0,1), then the mirror inside each half row and inside the row (each pairs two groups
// that already agree)
__device__ __forceinline__ void route_argmax16(float& bv, int& be) {
  route_argmax_step<0xB1>(bv, be);
  route_argmax_step<0x4E>(bv, be);
  route_argmax_step<0x141>(bv, be);
  route_argmax_step<0x140>(bv, be);
}

template <typename T, int NT>
__global__ __launch_bounds__(64 * kRouteWaves) void k_route_logits(RouteArgs a) {
  constexpr int NW = kRouteWaves, DB = RouteDepth<T>::b, EPW = 16 * NT;
  __shared__ f32x4 red[NW][NT][64];
  __shared__ float lg[16][EPW];
  const int lane = lane_id(), w = wave_id();
  const int M = a.M, d = a.d, E = a.E, k = a.k;
  const int ES = (E + EPW - 1) / EPW;
  const int rt = (int)blockIdx.x / ES, es = (int)blockIdx.x % ES;
  const int ks = d / 32, qw = (ks + NW - 1) / NW;
  const int sb = min(w * qw, ks), se = min(sb + qw, ks);
  const int row16 = lane & 15;

  // 1. this wave's share of K for the tile's 16 rows and the slice's NT expert tiles
  const T* ap[1] = {tiled_frag((const T*)a.Xt, rt, ks, sb)};
  const T* bp[NT];
  {
    const int last_ct = (E + 15) / 16 - 1;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bp[nt] = tiled_frag((const T*)a.Wr, min(es * NT + nt, last_ct), ks, sb);
  }
  f32x4 acc[1][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[0][nt] = zero4();
  if (se > sb) wave_gemm<T, 1, NT, DB>(acc, ap, bp, se - sb, kFragElems, kFragElems);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) red[w][nt][lane] = acc[0][nt];
  __syncthreads();

  // 2. the slice's logits, then its k best per row
  for (int nt = w; nt < NT; nt += NW) {
    f32x4 v = red[0][nt][lane];
#pragma unroll
    for (int x = 1; x < NW; ++x) v += red[x][nt][lane];
    const int c = 16 * nt + (lane & 15), e = EPW * es + c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * (lane >> 4) + i, tt = 16 * rt + row;
      lg[row][c] = v[i] != v[i] ? -INFINITY : v[i];  // a NaN logit counts as -inf
      if (e < E && tt < M) a.logits[(int64_t)tt * E + e] = v[i];
    }
  }
  __syncthreads();
  if (w >= 4) return;
  const int row = 4 * w + (lane >> 4), tt = 16 * rt + row;
  if (tt >= M) return;  // a whole 16-lane row leaves together
  const int valid = min(EPW, E - EPW * es);  // experts of this slice
  float v[NT];
  bool used[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int c = row16 + 16 * i;
    v[i] = lg[row][c];
    used[i] = c >= valid;
  }
  float* cv = a.cand_v + ((int64_t)tt * ES + es) * k;
  int32_t* ce = a.cand_e + ((int64_t)tt * ES + es) * k;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NT; ++i)
      if (!used[i] && route_better(v[i], row16 + 16 * i, bv, be)) { bv = v[i]; be = row16 + 16 * i; }
    route_argmax16(bv, be);
#pragma unroll
    for (int i = 0; i < NT; ++i)
      if (be == row16 + 16 * i) used[i] = true;
    if (row16 == 0) {  // fewer experts than k in this slice: the rest are empty (-1), never chosen
      cv[j] = bv;
      ce[j] = be < valid ? EPW * es + be : -1;
    }
  }
}

template <int KMAX>  // k <= KMAX
__global__ __launch_bounds__(1024) void k_route_order(RouteArgs a) {
  constexpr int CPT = KMAX / 2;  // candidates a thread owns: half of one slice's list
  __shared__ unsigned long long masks[kRouteMasks];  // [E][chunks]: bit b of (e, c) set when token 64c + b routes to e
  __shared__ int32_t pre[kRouteMasks];               // [E][chunks]: pairs of e in earlier chunks
  __shared__ uint8_t sel_s[kRouteMaxRows * 16];      // [M][k] chosen experts, best first
  __shared__ int32_t off_s[257];
  __shared__ int32_t wsum_n[4], wsum_t[4];
  const int tid = (int)threadIdx.x, lane = lane_id(), w = wave_id();
  const int M = a.M, E = a.E, k = a.k;
  const int ES = (E + 16 * route_tiles(E) - 1) / (16 * route_tiles(E));
  const int chunks = (M + 63) >> 6;
  for (int i = tid; i < E * chunks; i += 1024) masks[i] = 0ull;
  __syncthreads();

  // 1. four threads per row: thread (row, L, H) owns places H*CPT .. H*CPT + CPT-1 of slice L's sorted
  //    list; a candidate's rank among both lists is its place plus the other list's candidates that
  //    beat it.  Softmax over the k best in fp32, shifted by the best logit; the quad adds its four
  //    partial sums pairwise, so all four hold the same total.
  const int L = (tid >> 1) & 1, H = tid & 1;
  for (int t0 = 0; t0 < M; t0 += 256) {
    const int t = t0 + (tid >> 2);
    if (t >= M) break;  // a quad shares its row
    const float* cv = a.cand_v + (int64_t)t * ES * k;
    const int32_t* ce = a.cand_e + (int64_t)t * ES * k;
    // every load is unconditional, at an index clamped into the row's lists, so that all of them are in
    // flight at once; entries outside the lists are replaced by empty candidates afterwards
    const int Lo = min(L, ES - 1), Lx = min(1 - L, ES - 1);
    float ov[CPT], xv[KMAX];
    int oe[CPT], xe[KMAX];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int pc = min(H * CPT + i, k - 1);
      ov[i] = cv[Lo * k + pc];
      oe[i] = ce[Lo * k + pc];
    }
#pragma unroll
    for (int o = 0; o < KMAX; ++o) {
      const int oc = min(o, k - 1);
      xv[o] = cv[Lx * k + oc];
      xe[o] = ce[Lx * k + oc];
    }
    const float hv = cv[Lo * k];  // head of this thread's list (the other list's head is xv[0])
    const int he = ce[Lo * k];
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      if (!(L < ES && H * CPT + i < k)) { ov[i] = -INFINITY; oe[i] = -1; }
#pragma unroll
    for (int o = 0; o < KMAX; ++o)
      if (!(1 - L < ES && o < k)) { xv[o] = -INFINITY; xe[o] = -1; }
    // the row's best logit (the better head), the same on all four threads of the row
    unsigned long long xk[KMAX];
#pragma unroll
    for (int o = 0; o < KMAX; ++o) xk[o] = route_key(xv[o], xe[o]);
    const float mx = xk[0] > route_key(hv, he) ? xv[0] : hv;
    int rk[CPT];
    float ex[CPT], s = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      rk[i] = H * CPT + i;
      const unsigned long long ok = route_key(ov[i], oe[i]);
#pragma unroll
      for (int o = 0; o < KMAX; ++o) rk[i] += xk[o] > ok;
      if (oe[i] < 0) rk[i] = k;  // empty: not chosen
      ex[i] = 0.f;
      if (rk[i] < k) {
        ex[i] = expf(ov[i] - mx);
        s += ex[i];
      }
    }
    s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0xB1, 0xF, 0xF, false));
    s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x4E, 0xF, 0xF, false));
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      if (rk[i] < k) {
        const int64_t p = (int64_t)t * k + rk[i];
        a.idx[p] = oe[i];
        a.w[p] = ex[i] / s;
        sel_s[p] = (uint8_t)oe[i];
        atomicOr(&masks[oe[i] * chunks + (t >> 6)], 1ull << (t & 63));  // ds_or_b64
      }
  }
  __syncthreads();

  // 2. per expert: pairs in earlier chunks, total; exclusive scans over experts of pairs and tiles
  int n_e = 0;
  if (tid < E) {
    for (int c = 0; c < chunks; ++c) {
      pre[tid * chunks + c] = n_e;
      n_e += __popcll(masks[tid * chunks + c]);
    }
    a.counts[tid] = n_e;
  }
  const int tr = a.tile_rows;
  const int t_e = (n_e + tr - 1) / tr;
  int inc_n = n_e, inc_t = t_e;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int yn = __shfl_up(inc_n, o, 64), yt = __shfl_up(inc_t, o, 64);
    if (lane >= o) { inc_n += yn; inc_t += yt; }
  }
  if (tid < 256 && lane == 63) { wsum_n[w] = inc_n; wsum_t[w] = inc_t; }
  __syncthreads();
  if (tid < E) {
    int base_n = 0, base_t = 0;
    for (int x = 0; x < w; ++x) { base_n += wsum_n[x]; base_t += wsum_t[x]; }
    const int off = base_n + inc_n - n_e, toff = base_t + inc_t - t_e;
    off_s[tid] = off;
    a.offsets[tid] = off;
    for (int i = 0; i < t_e; ++i)
      a.tiles[toff + i] = make_int4(tid, off + i * tr, min(tr, n_e - i * tr), moe_pack_tile_w(t_e, i, n_e - (t_e - 1) * tr));
    if (tid == E - 1) {
      a.offsets[E] = off + n_e;
      *a.n_tiles = toff + t_e;
    }
  }
  __syncthreads();

  // 3. every pair's slot: its expert's offset + pairs of the expert in earlier chunks + earlier tokens
  //    of the expert in its own chunk
  for (int p = tid; p < M * k; p += 1024) {
    const int t = p / k, c = t >> 6, b = t & 63, e = sel_s[p];
    const unsigned long long below = b ? (~0ull) >> (64 - b) : 0ull;
    const int qs = off_s[e] + pre[e * chunks + c] + __popcll(masks[e * chunks + c] & below);
    a.pos[p] = qs;
    a.perm[qs] = t;
  }
}

// ============================================================== combine + residual (+ next RMSNorm)
// X[t] = X[t] + Ys[t] + sum_j w[t,j] * Yp[pos[t,j]], in fp32, j in fixed order, stored in the storage
// type.  With g != null the same kernel also forms the RMSNorm of the stored row with gain g (the next
// layer's attention norm, or the final norm before the head) and writes it to Yn, fragment-tiled
// (yn_tiled) or row-major, with k_rmsnorm's exact reduction order (bit-identical to normalising the
// stored X separately).  One workgroup per row, one thread per 8 columns.
template <typename T>
__global__ __launch_bounds__(1024) void k_moe_combine(T* __restrict__ X, const T* __restrict__ Ys,
                                                      const T* __restrict__ Yp, const int32_t* __restrict__ pos,
                                                      const float* __restrict__ w, int M, int d, int k,
                                                      const T* __restrict__ g, T* __restrict__ Yn, int yn_tiled,
                                                      float eps) {
  const int row = blockIdx.x;
  const int c = threadIdx.x * 8;
  int pj[16];
  float wj[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    pj[j] = j < k ? pos[(int64_t)row * k + j] : 0;
    wj[j] = j < k ? w[(int64_t)row * k + j] : 0.f;
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  if (c < d) {
    T* x = X + (int64_t)row * d + c;
    float v[8];
    Vec8<T>::load(x, acc);
    Vec8<T>::load(Ys + (int64_t)row * d + c, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += v[q];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < k) {
        Vec8<T>::load(Yp + (int64_t)pj[j] * d + c, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += wj[j] * v[q];
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      acc[q] = to_f32(from_f32<T>(acc[q]));  // the stored value
      ss += acc[q] * acc[q];
    }
    Vec8<T>::store(x, acc);
  }
  if (!g) return;  // uniform over the workgroup
  ss = row_sum_sq(ss);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  if (c < d) store_norm_row<T>(acc, r, g, c, row, d, yn_tiled ? nullptr : Yn, yn_tiled ? Yn : nullptr);
}

// ============================================================== stop check
// [P2] "How Diffusion Changes the Equation": stop when the mean canvas entropy is
// under a threshold or when predictions are unchanged over two consecutive
// passes, at most 48 passes; [P5] "How block diffusion works": the mean covers
// every slot.  With and_rule the early stop needs both at once ([P2] "Architecture
// Details": the recommended sampler).  With lock, a locked slot's prediction is
// replaced by its canvas token first (pred is rewritten).  One workgroup; S <= 1024.
__global__ __launch_bounds__(1024) void k_stop_check(const float* __restrict__ ent, int32_t* __restrict__ pred,
                                                     int32_t* __restrict__ prev, const int32_t* __restrict__ canvas,
                                                     const uint8_t* __restrict__ lock, int S, int step,
                                                     StopParams sp, dg_block_status* __restrict__ out) {
  __shared__ float part[1024];
  __shared__ int diff, bad;
  int i = threadIdx.x;
  if (i == 0) { diff = 0; bad = 0; }
  __syncthreads();
  float e = 0.f;
  int32_t p = 0;
  if (i < S) {
    e = ent[i];
    if (!(e >= 0.f && e <= sp.ln_vocab * 1.0001f + 1e-5f)) atomicOr(&bad, 1);
    p = pred[i];
    if (lock && lock[i]) {
      p = canvas[i];
      pred[i] = p;
    }
    if (p != prev[i]) atomicOr(&diff, 1);
  }
  part[i] = e;
  __syncthreads();
  for (int s = blockDim.x >> 1; s > 0; s >>= 1) {  // fixed pairwise tree
    if (i < s) part[i] += part[i + s];
    __syncthreads();
  }
  if (i < S) prev[i] = p;
  if (i == 0) {
    float mean = part[0] / (float)S;
    const bool low = mean < sp.threshold, stable = step >= 2 && !diff;
    int reason = 0;
    if (sp.fixed_steps > 0) {
      reason = step >= sp.fixed_steps ? DG_STOP_FIXED : 0;
    } else if (sp.and_rule ? (low && stable) : low) {
      reason = sp.and_rule ? DG_STOP_SETTLED : DG_STOP_ENTROPY;
    } else if (!sp.and_rule && stable) {
      reason = DG_STOP_STABLE;
    } else if (step >= sp.max_steps) {
      reason = DG_STOP_CAP;
    }
    out->steps = step;
    out->reason = reason;
    out->mean_entropy = mean;
    out->flags = bad ? DG_WARN_NUMERIC : 0u;
  }
}

// ============================================================== canvas update (Philox)
// [P5] "How block diffusion works": each pass keeps the slots the model is most
// confident about and re-randomises the rest; the canvas starts as random tokens.
// The key is the confidence, or minus the entropy (rank_entropy: lowest entropy
// first, [P2] "Architecture Details"); NaN ranks as -inf.  With lock (non-null),
// locked slots rank first, stay kept and keep their canvas token.  One workgroup
// of S threads (S <= 1024); rank_i counts slots that precede slot i in (key
// descending, slot ascending) order.  lock and keep_mask may alias (each thread
// reads its own entry before the barrier and writes it after).
__global__ __launch_bounds__(1024) void k_canvas_update(const int32_t* __restrict__ pred,
                                                        const float* __restrict__ conf, const float* ent,
                                                        int rank_entropy, const uint8_t* lock, int S, int keep,
                                                        uint32_t k0, uint32_t k1, uint32_t block, uint32_t step,
                                                        uint32_t V, int32_t* __restrict__ canvas, uint8_t* keep_mask) {
  __shared__ float key[1024];
  int i = threadIdx.x;
  const bool locked = lock && i < S && lock[i];
  if (keep > 0 && i < S) {
    float c = rank_entropy ? -ent[i] : conf[i];
    c = (c != c) ? -INFINITY : c;
    key[i] = locked ? INFINITY : c;
  }
  __syncthreads();
  if (i >= S) return;
  bool kept = false;
  if (keep >= S) {
    kept = true;
  } else if (keep > 0) {
    float ki = key[i];
    int rank = 0;
    for (int j = 0; j < S; ++j) {
      float kj = key[j];
      rank += (kj > ki || (kj == ki && j < i)) ? 1 : 0;
    }
    kept = rank < keep;
  }
  kept = kept || locked;
  int32_t out;
  if (locked) {
    out = canvas[i];
  } else if (kept) {
    out = pred[i];
  } else {
    const uint32_t w0 = philox4x32_10((uint32_t)i, step, block, 0u, k0, k1).x;
    out = (int32_t)(((uint64_t)w0 * V) >> 32);
  }
  canvas[i] = out;
  if (keep_mask) keep_mask[i] = kept ? 1 : 0;
}

// ============================================================== batched calls: cache scatter
// One thread per element; keys [h][pos][dh] and values [h][dh][pos], so both copies walk their
// innermost index fastest.
template <typename T>
__global__ __launch_bounds__(256) void k_kv_scatter(KvScatterArgs a) {
  const int dh = a.head_dim;
  const int64_t n = (int64_t)a.n_kv_heads * a.rows * dh;
  const T* ks = (const T*)a.ks;
  const T* vs = (const T*)a.vs;
  T* kd = (T*)a.kc;
  T* vd = (T*)a.vc;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % dh);
    const int64_t hr = i / dh;
    const int r = (int)(hr % a.rows), h = (int)(hr / a.rows);
    kd[((int64_t)h * a.cap + a.pos0 + r) * dh + c] = ks[((int64_t)h * a.M + a.row0 + r) * dh + c];
    const int r2 = (int)(i % a.rows);
    const int64_t hc = i / a.rows;  // h * dh + column
    vd[hc * a.cap + a.pos0 + r2] = vs[hc * a.M + a.row0 + r2];
  }
}

// ============================================================== launchers
template <typename T>
hipError_t launch_kv_scatter(const KvScatterArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.n_kv_heads * a.rows * a.head_dim;
  if (n <= 0) return hipSuccess;
  const int64_t g = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_kv_scatter<T>, dim3((unsigned)g), dim3(256), 0, s, a);
  return hipGetLastError();
}
template hipError_t launch_kv_scatter<float>(const KvScatterArgs&, hipStream_t);
template hipError_t launch_kv_scatter<bf16>(const KvScatterArgs&, hipStream_t);
hipError_t launch_embed_f8(const int32_t* tok, const uint8_t* E, const float* scale, bf16* X, int M, int d, int V,
                           hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_embed_f8, dim3(M), dim3(256), 0, s, tok, E, scale, X, M, d, V);
  return hipGetLastError();
}
template <typename T>
hipError_t launch_embed(const int32_t* tok, const T* E, T* X, int M, int d, int V, hipStream_t s) {
  hipLaunchKernelGGL(k_embed<T>, dim3(M), dim3(256), 0, s, tok, E, X, M, d, V);
  return hipGetLastError();
}
template <typename T>
hipError_t launch_pack(const T* src, T* dst, int64_t batch, int64_t rows, int64_t cols, hipStream_t s) {
  const int64_t rows_p = (rows + 15) / 16 * 16;
  const int64_t chunks = batch * rows_p / 16 * (cols / 32) * 64;
  int64_t g = (chunks + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(k_pack<T>, dim3((unsigned)g), dim3(256), 0, s, src, dst, batch, rows, cols, rows_p);
  return hipGetLastError();
}
hipError_t launch_quantize_e4m3(const bf16* src, uint8_t* dst, float* scale, int64_t batch, int64_t rows, int64_t cols,
                                hipStream_t s) {
  const int64_t n_rows = batch * rows;
  hipLaunchKernelGGL(k_e4m3_scales, dim3((unsigned)((n_rows + 3) / 4)), dim3(256), 0, s, src, scale, n_rows, cols);
  const int64_t rows_p = (rows + 15) / 16 * 16;
  const int64_t chunks = batch * rows_p / 16 * (cols / 64) * 64;
  int64_t g = (chunks + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(k_e4m3_pack, dim3((unsigned)g), dim3(256), 0, s, src, scale, dst, batch, rows, cols, rows_p);
  return hipGetLastError();
}
static inline int row_threads(int d) { return 64 * ((d + 511) / 512); }

template <typename T>
hipError_t launch_rmsnorm(const T* X, const T* g, T* Y, T* Yt, int M, int d, float eps, hipStream_t s, hipEvent_t done) {
  if (done)  // the event completes with the kernel itself (no separate marker in the stream)
    hipExtLaunchKernelGGL(k_rmsnorm<T>, dim3(M), dim3(row_threads(d)), 0, s, nullptr, done, 0, X, g, Y, Yt, M, d, eps);
  else
    hipLaunchKernelGGL(k_rmsnorm<T>, dim3(M), dim3(row_threads(d)), 0, s, X, g, Y, Yt, M, d, eps);
  return hipGetLastError();
}
template <typename T>
hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  // the ordering workgroup's LDS holds kRouteMaxRows rows and one mask per (expert, 64-token chunk)
  if (a.M > kRouteMaxRows || a.E * ((a.M + 63) / 64) > kRouteMasks || a.E > 256 || a.k > 16)
    return hipErrorInvalidValue;
  const int nt = route_tiles(a.E), slices = (a.E + 16 * nt - 1) / (16 * nt);
  const dim3 grid(((a.M + 15) / 16) * slices), block(64 * kRouteWaves);
  if (nt == 4)
    hipLaunchKernelGGL((k_route_logits<T, 4>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((k_route_logits<T, 8>), grid, block, 0, s, a);
  if (a.k <= 8)
    hipLaunchKernelGGL(k_route_order<8>, dim3(1), dim3(1024), 0, s, a);
  else
    hipLaunchKernelGGL(k_route_order<16>, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}
template <typename T>
hipError_t launch_moe_combine(T* X, const T* Ys, const T* Yp, const int32_t* pos, const float* w, int M, int d,
                              int k, const T* g, T* Yn, int yn_tiled, float eps, hipStream_t s) {
  hipLaunchKernelGGL(k_moe_combine<T>, dim3(M), dim3(row_threads(d)), 0, s, X, Ys, Yp, pos, w, M, d, k, g, Yn,
                     yn_tiled, eps);
  return hipGetLastError();
}
hipError_t launch_stop_check(const float* ent, int32_t* pred, int32_t* prev, const int32_t* canvas,
                             const uint8_t* lock, int S, int step, StopParams sp, dg_block_status* out,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_stop_check, dim3(1), dim3(1024), 0, s, ent, pred, prev, canvas, lock, S, step, sp, out);
  return hipGetLastError();
}
hipError_t launch_canvas_update(const CanvasArgs& a, hipStream_t s) {
  int threads = ((a.S + 63) / 64) * 64;
  hipLaunchKernelGGL(k_canvas_update, dim3(1), dim3(threads), 0, s, a.pred, a.conf, a.ent, a.rank_entropy, a.lock,
                     a.S, a.keep, (uint32_t)a.seed, (uint32_t)(a.seed >> 32), a.block, a.step, a.V, a.canvas,
                     a.keep_mask);
  return hipGetLastError();
}

template hipError_t launch_embed<float>(const int32_t*, const float*, float*, int, int, int, hipStream_t);
template hipError_t launch_pack<float>(const float*, float*, int64_t, int64_t, int64_t, hipStream_t);
template hipError_t launch_pack<bf16>(const bf16*, bf16*, int64_t, int64_t, int64_t, hipStream_t);
template hipError_t launch_embed<bf16>(const int32_t*, const bf16*, bf16*, int, int, int, hipStream_t);
template hipError_t launch_rmsnorm<float>(const float*, const float*, float*, float*, int, int, float, hipStream_t, hipEvent_t);
template hipError_t launch_rmsnorm<bf16>(const bf16*, const bf16*, bf16*, bf16*, int, int, float, hipStream_t, hipEvent_t);
template hipError_t launch_route<float>(const RouteArgs&, hipStream_t);
template hipError_t launch_route<bf16>(const RouteArgs&, hipStream_t);
template hipError_t launch_moe_combine<float>(float*, const float*, const float*, const int32_t*, const float*, int,
                                                      int, int, const float*, float*, int, float, hipStream_t);
template hipError_t launch_moe_combine<bf16>(bf16*, const bf16*, const bf16*, const int32_t*, const float*, int,
                                                     int, int, const bf16*, bf16*, int, float, hipStream_t);

}  // namespace dg
