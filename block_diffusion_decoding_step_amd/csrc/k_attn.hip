// k_attn.hip — canvas attention over the KV cache (gfx950 matrix cores).
//
// [P2] "DiffusionGemma 26B: How Google's Text Diffusion Model Generates Tokens in
// Parallel", "How Diffusion Changes the Equation": inside the block every position
// attends to every other (no mask); [P5] "When to use a diffusion LLM",
// "How block diffusion works": the canvas also reads the cached prompt.  Causal mode
// (query i sees keys up to its own position) serves prompt prefill and block commit.
//
// Design
//   * One wave = 16 query rows x HG query heads of one KV head (GQA packing: the
//     HG heads share every K/V fragment) x one split of the key range.
//   * S^T = K Q^T on the matrix core, so each lane ends up holding 8 consecutive
//     keys of ONE query (its lane & 15): the online softmax needs only two xor
//     shuffles, and the probabilities are already in the B-operand layout of
//     O^T = V^T P^T.  The value cache is stored [dh][position], so the A operand
//     of that product is a contiguous 16-byte load per lane.  No LDS, no
//     transposes; probabilities stay in registers.  For bf16 storage each
//     probability is split into a bf16 high part and a bf16 remainder and P V
//     takes two matrix-core products, so P keeps ~16 significant bits instead of
//     8 (rounding P to bf16 alone shifts the attention output by ~0.1%, enough to
//     move a visible fraction of bf16 hidden states by one unit in the last place).
//   * Scores use base-2 exponentials with log2(e)/sqrt(Dh) folded into the scale.
//   * Splits write unnormalised partials (O, running max, running sum); a merge
//     kernel combines them in fixed split order (deterministic) and normalises.
#include "dg_device.h"
#include "dg_kernels.h"

namespace dg {

template <typename T, int DH, int HG>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a) {
  constexpr int KS = DH / 32;   // 32-wide K steps over the head dimension
  constexpr bool kExactP = sizeof(T) == 4;  // fp32 storage holds P exactly
  constexpr int MTD = DH / 16;  // 16-row tiles of O^T along the head dimension
  const int lane = lane_id(), row16 = lane & 15, quad = lane >> 4;
  const int G = a.n_heads / a.n_kv_heads;
  const int hsub = G / HG;                      // head sub-groups per KV head
  const int n_rt = (a.q_rows + 15) / 16;        // query row tiles
  const int tasks = a.n_kv_heads * hsub * a.n_split * n_rt;
  const int n_wg = (tasks + 3) / 4;
  const int task = xcd_remap(blockIdx.x, n_wg) * 4 + wave_id();
  if (task >= tasks) return;
  const int rt = task % n_rt;
  int rest = task / n_rt;
  const int split = rest % a.n_split;
  rest /= a.n_split;
  const int hs = rest % hsub;
  const int g = rest / hsub;
  const int r0 = rt * 16;
  const int mq = r0 + row16;                     // this lane's query row
  const int mq_ld = min(mq, a.q_rows - 1);

  const int64_t n_chunks = (a.n_keys + 31) / 32;
  const int64_t per = (n_chunks + a.n_split - 1) / a.n_split;
  int64_t c_begin = split * per;
  int64_t c_end = min(n_chunks, c_begin + per);
  if (a.causal) {
    int64_t last_pos = a.q_pos0 + min(r0 + 15, a.q_rows - 1);  // furthest key any row of the tile sees
    c_end = min(c_end, last_pos / 32 + 1);
  }
  const int64_t my_pos = a.q_pos0 + mq;

  const T* Q = (const T*)a.q;
  const T* K = (const T*)a.kc + (int64_t)g * a.cap * DH;
  const T* Vt = (const T*)a.vc + (int64_t)g * DH * a.cap;

  Frag<T> qf[HG][KS];
#pragma unroll
  for (int j = 0; j < HG; ++j) {
    const int h = g * G + hs * HG + j;
    const T* qrow = Q + ((int64_t)h * a.q_rows + mq_ld) * DH + quad * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[j][ks].load(qrow + 32 * ks);
  }
  const float scale = 1.4426950408889634f / sqrtf((float)DH);

  float m_run[HG], l_run[HG];
  f32x4 o[HG][MTD];
#pragma unroll
  for (int j = 0; j < HG; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
#pragma unroll
    for (int mt = 0; mt < MTD; ++mt) o[j][mt] = zero4();
  }
  // A-operand row of S^T tile i for this lane: key kbase + 8*(row16/4) + 4*i + row16%4,
  // so that C register r of tile i on this lane is key kbase + 8*quad + 4*i + r.
  const int krow = 8 * (row16 >> 2) + (row16 & 3);

  for (int64_t c = c_begin; c < c_end; ++c) {
    const int64_t kbase = c * 32;
    Frag<T> kf[2][KS];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const T* kr = K + (kbase + krow + 4 * i) * DH + quad * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[i][ks].load(kr + 32 * ks);
    }
    Frag<T> vf[MTD];
#pragma unroll
    for (int mt = 0; mt < MTD; ++mt) vf[mt].load(Vt + (int64_t)(16 * mt + row16) * a.cap + kbase + quad * 8);
    if (kbase + 32 > a.n_keys) {  // zero values past the last key (memory there may hold anything)
#pragma unroll
      for (int mt = 0; mt < MTD; ++mt)
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (kbase + quad * 8 + t >= a.n_keys) vf[mt].set(t, 0.f);
    }
#pragma unroll
    for (int j = 0; j < HG; ++j) {
      f32x4 s[2] = {zero4(), zero4()};
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) mma(s[i], kf[i][ks], qf[j][ks]);
      float sc[8];
      bool ok[8];
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int64_t key = kbase + quad * 8 + t;
        ok[t] = key < a.n_keys && (!a.causal || key <= my_pos);
        sc[t] = s[t >> 2][t & 3] * scale;
        if (ok[t]) mx = fmaxf(mx, sc[t]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[j], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m_run[j] - m_use);
      Frag<T> pf, pl;
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        float p = ok[t] ? exp2f(sc[t] - m_use) : 0.f;
        psum += p;
        pf.set(t, p);
        if constexpr (!kExactP) pl.set(t, p - pf.get(t));
      }
      l_run[j] = l_run[j] * alpha + psum;
      m_run[j] = m_new;
#pragma unroll
      for (int mt = 0; mt < MTD; ++mt) {
        o[j][mt] *= alpha;
        mma(o[j][mt], vf[mt], pf);
        if constexpr (!kExactP) mma(o[j][mt], vf[mt], pl);
      }
    }
  }

  // partials: O^T tile register r of tile mt on this lane = (query mq, dh 16*mt + 4*quad + r)
#pragma unroll
  for (int j = 0; j < HG; ++j) {
    float l_tot = l_run[j];
    l_tot += __shfl_xor(l_tot, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if (mq < a.q_rows) {
      const int h = g * G + hs * HG + j;
      const int64_t row = ((int64_t)split * a.n_heads + h) * a.q_rows + mq;
      float* op = a.o_part + row * DH + quad * 4;
#pragma unroll
      for (int mt = 0; mt < MTD; ++mt) *reinterpret_cast<f32x4*>(op + 16 * mt) = o[j][mt];
      if (quad == 0) {
        a.ml_part[row * 2] = m_run[j];
        a.ml_part[row * 2 + 1] = l_tot;
      }
    }
  }
}

// Merge split partials in split order and normalise: one thread per (row, head, 8 dh).
template <typename T, int DH>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  const int per_row = DH / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.q_rows * a.n_heads * per_row;
  if (i >= total) return;
  const int c = (int)(i % per_row) * 8;
  const int64_t hm = i / per_row;
  const int h = (int)(hm % a.n_heads);
  const int m = (int)(hm / a.n_heads);
  float mx = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) {
    const int64_t row = ((int64_t)s * a.n_heads + h) * a.q_rows + m;
    mx = fmaxf(mx, a.ml_part[row * 2]);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int s = 0; s < a.n_split; ++s) {
    const int64_t row = ((int64_t)s * a.n_heads + h) * a.q_rows + m;
    const float ms = a.ml_part[row * 2];
    if (ms == -INFINITY) continue;
    const float f = exp2f(ms - mx);
    L += a.ml_part[row * 2 + 1] * f;
    const float* op = a.o_part + row * DH + c;
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] += op[t] * f;
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] *= inv;
  Vec8<T>::store((T*)a.o + (int64_t)m * a.n_heads * DH + h * DH + c, acc);
}

int attention_splits(int64_t n_keys, int q_rows, int n_heads, int n_kv_heads, int causal, int max_split) {
  (void)causal;
  const int64_t n_chunks = (n_keys + 31) / 32;
  const int base = n_kv_heads * ((q_rows + 15) / 16) * (n_heads / n_kv_heads >= 2 ? n_heads / n_kv_heads / 2 : 1);
  int s = (2048 + base - 1) / base;
  if (s > max_split) s = max_split;
  int64_t by_chunks = n_chunks / 4;  // at least 4 chunks (128 keys) per split
  if (s > by_chunks) s = (int)by_chunks;
  if (s < 1) s = 1;
  return s;
}

template <typename T, int DH, int HG>
static void launch_attn_t(const AttnArgs& a, hipStream_t s) {
  const int G = a.n_heads / a.n_kv_heads;
  const int tasks = a.n_kv_heads * (G / HG) * a.n_split * ((a.q_rows + 15) / 16);
  hipLaunchKernelGGL((k_attn<T, DH, HG>), dim3((tasks + 3) / 4), dim3(256), 0, s, a);
}

template <typename T>
hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const int G = a.n_heads / a.n_kv_heads;
  const bool pair = G % 2 == 0;
  if (a.head_dim == 128) {
    if (pair) launch_attn_t<T, 128, 2>(a, s); else launch_attn_t<T, 128, 1>(a, s);
  } else {
    if (pair) launch_attn_t<T, 64, 2>(a, s); else launch_attn_t<T, 64, 1>(a, s);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_attention_merge(const AttnArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.q_rows * a.n_heads * (a.head_dim / 8);
  dim3 grid((unsigned)((total + 255) / 256));
  if (a.head_dim == 128)
    hipLaunchKernelGGL((k_attn_merge<T, 128>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_attn_merge<T, 64>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_attention<float>(const AttnArgs&, hipStream_t);
template hipError_t launch_attention<bf16>(const AttnArgs&, hipStream_t);
template hipError_t launch_attention_merge<float>(const AttnArgs&, hipStream_t);
template hipError_t launch_attention_merge<bf16>(const AttnArgs&, hipStream_t);

}  // namespace dg
