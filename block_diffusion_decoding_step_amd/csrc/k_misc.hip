// k_misc.hip — the memory-light stages of a denoising pass:
//   embedding gather, RMSNorm, MoE routing (top-k + token->expert permutation),
//   MoE combine + residual, stop check and the Philox canvas update.
// Page tags: [P2] "DiffusionGemma 26B: How Google's Text Diffusion Model Generates
// Tokens in Parallel"; [P5] "When to use a diffusion LLM: I compared DiffusionGemma
// and Gemma 4".
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

// ============================================================== router top-k
// One wave per token.  Top-k of the fp32 router logits, ties to the lower expert
// id, then softmax over the k chosen ([P2] "Architecture Details": 8 of 128
// experts active per token, plus one shared expert that is always applied).
__global__ __launch_bounds__(256) void k_router_topk(const float* __restrict__ logits, int M, int E, int k,
                                                     int32_t* __restrict__ idx, float* __restrict__ w) {
  int t = blockIdx.x * 4 + wave_id();
  if (t >= M) return;
  int l = lane_id();
  const float* r = logits + (int64_t)t * E;
  float v[4];
  bool used[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = l + 64 * i;
    const float x = e < E ? r[e] : -INFINITY;
    v[i] = x != x ? -INFINITY : x;  // a NaN logit counts as -inf, so a valid expert is always chosen
    used[i] = e >= E;
  }
  float sel_v[16];
  int sel_e[16];
  for (int j = 0; j < k; ++j) {
    // lane-local best among unused entries: larger value, then lower id
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = l + 64 * i;
      if (!used[i] && (v[i] > bv || (v[i] == bv && e < be))) { bv = v[i]; be = e; }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      float ov = __shfl_xor(bv, o, 64);
      int oe = __shfl_xor(be, o, 64);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (l + 64 * i == be) used[i] = true;
    sel_v[j] = bv;
    sel_e[j] = be;
  }
  if (l == 0) {
    float mx = sel_v[0];
    float s = 0.f, ex[16];
    for (int j = 0; j < k; ++j) { ex[j] = expf(sel_v[j] - mx); s += ex[j]; }
    for (int j = 0; j < k; ++j) {
      idx[(int64_t)t * k + j] = sel_e[j];
      w[(int64_t)t * k + j] = ex[j] / s;
    }
  }
}

// ============================================================== token -> expert permutation
// Pairs (token t, choice j) are ordered by (expert, token).  Built with wavefront
// ballots: for expert e and a 64-token chunk c, ballot(token routes to e) gives a
// 64-bit mask whose popcount is the chunk's count and whose prefix popcount is a
// pair's rank inside the chunk.  All integer, deterministic.  Also emits the list
// of (expert, first pair, rows <= kMoeTileRows) work tiles of the grouped expert GEMMs.
// Launch: one workgroup of 1024 threads.  Limits (checked by the host, see
// moe_max_rows): M <= 2048, M * ceil(E/32) <= 8192, E * ceil(M/64) <= 4096.

__global__ __launch_bounds__(1024) void k_moe_permute(const int32_t* __restrict__ idx, int M, int E, int k,
                                                      int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ perm, int32_t* __restrict__ pos,
                                                      int4* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
  __shared__ uint32_t bits[kPermBitWords];  // [M][ceil(E/32)] token -> expert bitmap
  __shared__ uint64_t masks[kPermMasks];    // [E][chunks] ballot masks
  __shared__ int32_t pre[kPermMasks];       // [E][chunks] chunk counts, then chunk prefixes
  __shared__ int32_t off_s[257];
  const int words = (E + 31) >> 5;
  const int chunks = (M + 63) >> 6;
  const int tid = threadIdx.x;
  for (int i = tid; i < M * words; i += blockDim.x) bits[i] = 0u;
  __syncthreads();
  for (int p = tid; p < M * k; p += blockDim.x) {
    int t = p / k;
    int e = idx[p];
    atomicOr(&bits[t * words + (e >> 5)], 1u << (e & 31));
  }
  __syncthreads();
  const int nwaves = blockDim.x >> 6;
  const int l = lane_id();
  for (int ec = wave_id(); ec < E * chunks; ec += nwaves) {
    int e = ec / chunks, c = ec % chunks;
    int t = c * 64 + l;
    bool hit = t < M && ((bits[t * words + (e >> 5)] >> (e & 31)) & 1u);
    uint64_t m = __ballot(hit);
    if (l == 0) {
      masks[ec] = m;
      pre[ec] = __popcll(m);
    }
  }
  __syncthreads();
  // per-expert totals and chunk prefixes (thread e walks its expert's chunks)
  int n_e = 0;
  if (tid < E) {
    for (int c = 0; c < chunks; ++c) {
      const int n = pre[tid * chunks + c];
      pre[tid * chunks + c] = n_e;
      n_e += n;
    }
    counts[tid] = n_e;
  }
  // exclusive scans over experts of (pairs, tiles): wave prefix sums, then wave totals (E <= 256)
  const int t_e = (n_e + kMoeTileRows - 1) / kMoeTileRows;
  int inc_n = n_e, inc_t = t_e;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int yn = __shfl_up(inc_n, o, 64), yt = __shfl_up(inc_t, o, 64);
    if (l >= o) { inc_n += yn; inc_t += yt; }
  }
  __shared__ int wsum_n[4], wsum_t[4];
  if (tid < 256 && l == 63) { wsum_n[tid >> 6] = inc_n; wsum_t[tid >> 6] = inc_t; }
  __syncthreads();
  if (tid < E) {
    int base_n = 0, base_t = 0;
    for (int wv = 0; wv < (tid >> 6); ++wv) { base_n += wsum_n[wv]; base_t += wsum_t[wv]; }
    const int off = base_n + inc_n - n_e, toff = base_t + inc_t - t_e;
    off_s[tid] = off;
    offsets[tid] = off;
    for (int i = 0; i < t_e; ++i)
      tiles[toff + i] = make_int4(tid, off + i * kMoeTileRows, min(kMoeTileRows, n_e - i * kMoeTileRows), 0);
    if (tid == E - 1) {
      offsets[E] = off + n_e;
      *n_tiles = toff + t_e;
    }
  }
  __syncthreads();
  for (int p = tid; p < M * k; p += blockDim.x) {
    int t = p / k;
    int e = idx[p];
    int c = t >> 6, b = t & 63;
    uint64_t below = b ? (masks[e * chunks + c] & ((~0ull) >> (64 - b))) : 0ull;
    int q = off_s[e] + pre[e * chunks + c] + __popcll(below);
    pos[p] = q;
    perm[q] = t;
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
// every slot.  One workgroup; S <= 1024.
__global__ __launch_bounds__(1024) void k_stop_check(const float* __restrict__ ent, const int32_t* __restrict__ pred,
                                                     int32_t* __restrict__ prev, int S, int step,
                                                     StopParams sp, dg_block_status* __restrict__ out) {
  __shared__ float part[1024];
  __shared__ int diff, bad;
  int i = threadIdx.x;
  if (i == 0) { diff = 0; bad = 0; }
  __syncthreads();
  float e = 0.f;
  if (i < S) {
    e = ent[i];
    if (!(e >= 0.f && e <= sp.ln_vocab * 1.0001f + 1e-5f)) atomicOr(&bad, 1);
    if (pred[i] != prev[i]) atomicOr(&diff, 1);
  }
  part[i] = e;
  __syncthreads();
  for (int s = blockDim.x >> 1; s > 0; s >>= 1) {  // fixed pairwise tree
    if (i < s) part[i] += part[i + s];
    __syncthreads();
  }
  if (i < S) prev[i] = pred[i];
  if (i == 0) {
    float mean = part[0] / (float)S;
    int reason = 0;
    if (sp.fixed_steps > 0) {
      reason = step >= sp.fixed_steps ? 4 : 0;
    } else if (mean < sp.threshold) {
      reason = 1;
    } else if (step >= 2 && !diff) {
      reason = 2;
    } else if (step >= sp.max_steps) {
      reason = 3;
    }
    out->steps = step;
    out->reason = reason;
    out->mean_entropy = mean;
    out->flags = bad ? DG_WARN_NUMERIC : 0u;
  }
}

// ============================================================== canvas update (Philox)
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds; each round takes
// the 64-bit products of counter words 0 and 2 with two fixed multipliers, swaps
// in their low halves and xors their high halves with words 1/3 and the key;
// the key advances by two Weyl constants between rounds.
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    uint64_t p0 = (uint64_t)M0 * c0;
    uint64_t p1 = (uint64_t)M1 * c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  return c0;
}

// [P5] "How block diffusion works": each pass keeps the slots the model is most
// confident about and re-randomises the rest; the canvas starts as random tokens.
// One workgroup of S threads (S <= 1024).  rank_i counts slots that precede slot i
// in (conf descending, slot ascending) order; NaN ranks as -inf.
__global__ __launch_bounds__(1024) void k_canvas_update(const int32_t* __restrict__ pred,
                                                        const float* __restrict__ conf, int S, int keep,
                                                        uint32_t k0, uint32_t k1, uint32_t block, uint32_t step,
                                                        uint32_t V, int32_t* __restrict__ canvas,
                                                        uint8_t* __restrict__ keep_mask) {
  __shared__ float key[1024];
  int i = threadIdx.x;
  if (keep > 0 && i < S) {
    float c = conf[i];
    key[i] = (c != c) ? -INFINITY : c;
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
  int32_t out;
  if (kept) {
    out = pred[i];
  } else {
    uint32_t w0 = philox_word0((uint32_t)i, step, block, 0u, k0, k1);
    out = (int32_t)(((uint64_t)w0 * V) >> 32);
  }
  canvas[i] = out;
  if (keep_mask) keep_mask[i] = kept ? 1 : 0;
}

// ============================================================== launchers
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
static inline int row_threads(int d) { return 64 * ((d + 511) / 512); }

template <typename T>
hipError_t launch_rmsnorm(const T* X, const T* g, T* Y, T* Yt, int M, int d, float eps, hipStream_t s) {
  hipLaunchKernelGGL(k_rmsnorm<T>, dim3(M), dim3(row_threads(d)), 0, s, X, g, Y, Yt, M, d, eps);
  return hipGetLastError();
}
hipError_t launch_router_topk(const float* logits, int M, int E, int k, int32_t* idx, float* w, hipStream_t s) {
  hipLaunchKernelGGL(k_router_topk, dim3((M + 3) / 4), dim3(256), 0, s, logits, M, E, k, idx, w);
  return hipGetLastError();
}
hipError_t launch_moe_permute(const int32_t* idx, int M, int E, int k, int32_t* counts, int32_t* offsets,
                              int32_t* perm, int32_t* pos, int4* tiles, int32_t* n_tiles, hipStream_t s) {
  hipLaunchKernelGGL(k_moe_permute, dim3(1), dim3(1024), 0, s, idx, M, E, k, counts, offsets, perm, pos, tiles,
                     n_tiles);
  return hipGetLastError();
}
template <typename T>
hipError_t launch_moe_combine(T* X, const T* Ys, const T* Yp, const int32_t* pos, const float* w, int M, int d,
                              int k, const T* g, T* Yn, int yn_tiled, float eps, hipStream_t s) {
  hipLaunchKernelGGL(k_moe_combine<T>, dim3(M), dim3(row_threads(d)), 0, s, X, Ys, Yp, pos, w, M, d, k, g, Yn,
                     yn_tiled, eps);
  return hipGetLastError();
}
hipError_t launch_stop_check(const float* ent, const int32_t* pred, int32_t* prev, int S, int step, StopParams sp,
                             dg_block_status* out, hipStream_t s) {
  hipLaunchKernelGGL(k_stop_check, dim3(1), dim3(1024), 0, s, ent, pred, prev, S, step, sp, out);
  return hipGetLastError();
}
hipError_t launch_canvas_update(const int32_t* pred, const float* conf, int S, int keep, uint64_t seed,
                                uint32_t block, uint32_t step, uint32_t V, int32_t* canvas, uint8_t* keep_mask,
                                hipStream_t s) {
  int threads = ((S + 63) / 64) * 64;
  hipLaunchKernelGGL(k_canvas_update, dim3(1), dim3(threads), 0, s, pred, conf, S, keep, (uint32_t)seed,
                     (uint32_t)(seed >> 32), block, step, V, canvas, keep_mask);
  return hipGetLastError();
}

template hipError_t launch_embed<float>(const int32_t*, const float*, float*, int, int, int, hipStream_t);
template hipError_t launch_pack<float>(const float*, float*, int64_t, int64_t, int64_t, hipStream_t);
template hipError_t launch_pack<bf16>(const bf16*, bf16*, int64_t, int64_t, int64_t, hipStream_t);
template hipError_t launch_embed<bf16>(const int32_t*, const bf16*, bf16*, int, int, int, hipStream_t);
template hipError_t launch_rmsnorm<float>(const float*, const float*, float*, float*, int, int, float, hipStream_t);
template hipError_t launch_rmsnorm<bf16>(const bf16*, const bf16*, bf16*, bf16*, int, int, float, hipStream_t);
template hipError_t launch_moe_combine<float>(float*, const float*, const float*, const int32_t*, const float*, int,
                                                      int, int, const float*, float*, int, float, hipStream_t);
template hipError_t launch_moe_combine<bf16>(bf16*, const bf16*, const bf16*, const int32_t*, const float*, int,
                                                     int, int, const bf16*, bf16*, int, float, hipStream_t);

}  // namespace dg
