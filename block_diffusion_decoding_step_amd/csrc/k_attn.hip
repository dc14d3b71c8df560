// k_attn.hip — canvas attention over the KV cache (gfx950 matrix cores).
//
// [P2] "DiffusionGemma 26B: How Google's Text Diffusion Model Generates Tokens in
// Parallel", "How Diffusion Changes the Equation": inside the block every position
// attends to every other (no mask); [P5] "When to use a diffusion LLM",
// "How block diffusion works": the canvas also reads the cached prompt.  Causal mode
// (query i sees keys up to its own position) serves prompt prefill and block commit.
//
// Design
//   * A workgroup of 8 waves takes 256 (head, query) rows of ONE KV head -- every
//     query head of the GQA group reads the same keys -- and one split of the key
//     range.  Each wave owns 32 consecutive queries of one head (two 16-row tiles).
//   * The key range is walked in chunks of 64 keys.  Each chunk's K and V
//     fragments are copied once from global memory straight into LDS (no register
//     staging), double-buffered so that the copy of the next chunk is in flight
//     while this one is computed, and read by all 8 waves: K/V leave L2 once per
//     workgroup.  In LDS every fragment is stored in the matrix core's operand order
//     (one contiguous 16-byte read per lane, no bank conflicts).
//   * S^T = K Q^T on the matrix core, with the key rows of each K fragment
//     permuted so that each lane ends up holding 8 consecutive keys of ONE query
//     (its lane & 15), already in the B-operand layout of O^T = V^T P^T.  The value
//     cache is stored [dh][position], so V^T fragments are contiguous 16-byte rows.
//     For bf16 storage each probability is split into a bf16 high part and a bf16
//     remainder and P V takes two matrix-core products, so P keeps ~16 significant
//     bits instead of 8 (rounding P to bf16 alone perturbs the attention output by
//     ~0.1%, enough to flip downstream bf16 roundings and routing decisions).
//   * Online softmax in base 2 with log2(e)/sqrt(Dh) folded into one FMA per score,
//     against a lazily updated reference max: the exact row max (two shuffles) and
//     the rescale of O are only computed when some probability would exceed 2^8.
//   * Splits write unnormalised partials (O, reference max, sum); a merge kernel
//     combines them in fixed split order (deterministic) and normalises.
#include "dg_device.h"
#include "dg_kernels.h"
#include "dg_wave_gemm.h"

namespace dg {

constexpr int kAttnWaves = 8;     // waves per workgroup
constexpr int kAttnQT = 2;        // 16-query tiles per wave
constexpr int kAttnRows = 16 * kAttnQT;  // (head, query) rows per wave
constexpr int kAttnChunk = 64;    // keys per LDS stage (two 32-key steps)
constexpr bool kAttnSplitP = true;   // bf16 P as high + remainder parts (two products)
constexpr uint32_t kAttnLazyBits = 0x43800000u;  // 256.0f: probabilities stay below 2^8 of the reference

typedef __attribute__((address_space(3))) void lds_void;

template <typename T, int DH, int NW = kAttnWaves, int SUBS_ = 4>
struct AttnCfg {
  static constexpr int SUBS = (sizeof(T) == 4 && DH == 128) ? (SUBS_ < 2 ? SUBS_ : 2) : SUBS_;  // 32-key steps per chunk
  static constexpr int CHUNK = 32 * SUBS;
  static constexpr int KF = DH / 32;                 // K fragments per 16-key tile (32-wide dh steps)
  static constexpr int MTD = DH / 16;                // 16-row dh tiles of O^T
  static constexpr int NKF = SUBS * 2 * KF;          // K fragments per chunk (2 key tiles per step)
  static constexpr int NVF = SUBS * MTD;             // V^T fragments per chunk
  static constexpr int NF = NKF + NVF;
  static constexpr int FB = kFragElems * (int)sizeof(T);
  static constexpr int STAGE = NF * FB;              // bytes per stage
  static constexpr int UPL = FB / 64 / 16;           // 16-byte units per lane per fragment
  static constexpr int LOADS = STAGE / 16 / (64 * NW);  // 1 KB copies per wave per stage
  static_assert(LOADS * 16 * 64 * NW == STAGE, "stage split");
  static_assert(2 * STAGE <= 131072, "LDS");
};

// Workgroup -> (row block, split, KV head), row block fastest, XCD-aware so that
// the row blocks and splits of one KV head share an L2.
template <typename T, int DH, int NW, int SUBS, int QT>
__global__ __launch_bounds__(64 * NW, 1) void k_attn(AttnArgs a) {
  using C = AttnCfg<T, DH, NW, SUBS>;
  constexpr int ROWS = 16 * QT;  // (head, query) rows per wave
  constexpr bool kSplitP = sizeof(T) == 2 && kAttnSplitP;
  constexpr int EPU = 16 / (int)sizeof(T);  // elements per 16-byte unit
  __shared__ uint4 lds0[C::STAGE / 16];
  __shared__ uint4 lds1[C::STAGE / 16];
  const int lane = lane_id(), w = wave_id();
  const int row16 = lane & 15, quad = lane >> 4;
  const int G = a.n_heads / a.n_kv_heads;
  const int qt32 = (a.q_rows + ROWS - 1) / ROWS;   // 32-query tiles per head
  const int n_wt = G * qt32;                                 // wave tasks per KV head
  const int nb = (n_wt + NW - 1) / NW;       // row blocks per KV head
  const int n_wg = nb * a.n_split * a.n_kv_heads;
  const int id = xcd_remap(blockIdx.x, n_wg);
  const int rb = id % nb;
  const int split = (id / nb) % a.n_split;
  const int g = id / (nb * a.n_split);

  const int wt = rb * NW + w;
  const bool active = wt < n_wt;
  const int j = active ? wt / qt32 : 0;           // head within the group
  const int q0 = active ? (wt % qt32) * ROWS : 0;
  const int h = g * G + j;

  // keys this workgroup may need: all of them, or (causal) up to its furthest query
  int64_t key_end = a.n_keys;
  if (a.causal) {
    int qmax = 0;
    for (int x = 0; x < NW; ++x) {
      const int wx = rb * NW + x;
      if (wx < n_wt) qmax = max(qmax, min((wx % qt32) * ROWS + ROWS - 1, a.q_rows - 1));
    }
    key_end = imin64(key_end, a.q_pos0 + qmax + 1);
  }
  const int64_t n_ch = (key_end + C::CHUNK - 1) / C::CHUNK;
  const int64_t per = (n_ch + a.n_split - 1) / a.n_split;
  const int64_t ch_begin = imin64(n_ch, (int64_t)split * per);
  const int64_t ch_end = imin64(n_ch, ch_begin + per);
  const int n_my = (int)(ch_end - ch_begin);

  const T* K = (const T*)a.kc + (int64_t)g * a.cap * DH;
  const T* Vt = (const T*)a.vc + (int64_t)g * DH * a.cap;

  // Stage layout: fragment f < NKF is K for (32-key step f / (2 KF), key tile (f / KF) % 2,
  // dh step f % KF); fragment NKF + f' is V^T for (32-key step f' / MTD, dh tile f' % MTD).
  // Unit u (16 bytes at byte 16u) is lane (u % (64 UPL)) / UPL, part u % UPL, of fragment
  // u / (64 UPL).  Wave w copies units (jj * 8 + w) * 64 + lane straight from global memory
  // into LDS (one contiguous 1 KB per instruction).  Addresses are clamped into the cache
  // row; keys at or past n_keys are masked out of the scores, and their values are zeroed in
  // LDS before use (memory there may hold anything).
  auto unit_src = [&](int64_t c0, int u) -> const T* {
    const int f = u / (64 * C::UPL), qq = u % (64 * C::UPL);
    const int l = qq / C::UPL, part = qq % C::UPL;
    if (f < C::NKF) {
      const int sub = f / (2 * C::KF), i = (f / C::KF) % 2, ks = f % C::KF;
      const int lr = l & 15;
      const int64_t key = imin64(c0 + 32 * sub + 8 * (lr >> 2) + (lr & 3) + 4 * i, a.cap - 1);
      return K + key * DH + 32 * ks + 8 * (l >> 4) + part * EPU;
    }
    const int ff = f - C::NKF;
    const int sub = ff / C::MTD, mt = ff % C::MTD;
    const int64_t key0 = imin64(c0 + 32 * sub + 8 * (l >> 4) + part * EPU, a.cap - EPU);
    return Vt + (int64_t)(16 * mt + (l & 15)) * a.cap + key0;
  };
  auto issue = [&](int64_t ch, uint4* buf) {
    const int64_t c0 = ch * C::CHUNK;
#pragma unroll
    for (int jj = 0; jj < C::LOADS; ++jj) {
      const int u0 = (jj * NW + w) * 64;
      __builtin_amdgcn_global_load_lds((const void*)unit_src(c0, u0 + lane), (lds_void*)(buf + u0), 16, 0, 0);
    }
  };
  // zero V^T entries of keys >= n_keys in a staged chunk (only the chunk holding the last key)
  auto fix_tail = [&](int64_t ch, uint4* buf) {
    const int64_t c0 = ch * C::CHUNK;
#pragma unroll
    for (int jj = 0; jj < C::LOADS; ++jj) {
      const int u = (jj * NW + w) * 64 + lane;
      const int f = u / (64 * C::UPL), qq = u % (64 * C::UPL);
      if (f < C::NKF) continue;
      const int l = qq / C::UPL, part = qq % C::UPL;
      const int sub = (f - C::NKF) / C::MTD;
      const int64_t key0 = c0 + 32 * sub + 8 * (l >> 4) + part * EPU;
      if (key0 + EPU > a.n_keys) {
        uint4 v = buf[u];
        T* e = reinterpret_cast<T*>(&v);
#pragma unroll
        for (int x = 0; x < EPU; ++x)
          if (key0 + x >= a.n_keys) e[x] = from_f32<T>(0.f);
        buf[u] = v;
      }
    }
  };

  Frag<T> qf[QT][C::KF];
  int64_t my_pos[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int mq = q0 + 16 * qt + row16;
    my_pos[qt] = a.q_pos0 + mq;
    const T* qrow = (const T*)a.q + ((int64_t)h * a.q_stride + a.row0 + min(mq, a.q_rows - 1)) * DH + quad * 8;
#pragma unroll
    for (int ks = 0; ks < C::KF; ++ks) qf[qt][ks].load(qrow + 32 * ks);
  }
  const float scale = 1.4426950408889634f / sqrtf((float)DH);
  const int64_t wave_last = a.q_pos0 + min(q0 + ROWS - 1, a.q_rows - 1);  // furthest key this wave sees

  float m_run[QT], l_run[QT];
  f32x4 o[QT][C::MTD];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = -INFINITY;
    l_run[qt] = 0.f;
#pragma unroll
    for (int mt = 0; mt < C::MTD; ++mt) o[qt][mt] = zero4();
  }

  // S^T tiles of both query tiles for 32-key step `sub` of a staged chunk
  auto scores = [&](const T* base, int sub, f32x4 (&sv)[QT][2]) {
    Frag<T> kf[2][C::KF];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int ks = 0; ks < C::KF; ++ks) kf[i][ks].load(base + ((sub * 2 + i) * C::KF + ks) * kFragElems);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        sv[qt][i] = zero4();
#pragma unroll
        for (int ks = 0; ks < C::KF; ++ks) mma(sv[qt][i], kf[i][ks], qf[qt][ks]);
      }
  };

  // One staged chunk, 32-key step by 32-key step (steps past the wave's last visible key are skipped).
  auto compute = [&](int64_t ch, const uint4* buf) {
    const int64_t c0 = ch * C::CHUNK;
    if (!active || c0 >= a.n_keys || (a.causal && c0 > wave_last)) return;  // wave-uniform
    const T* base = reinterpret_cast<const T*>(buf) + lane * 8;
#pragma unroll
    for (int sub = 0; sub < C::SUBS; ++sub) {
      const int64_t kbase = c0 + 32 * sub;
      if (kbase >= a.n_keys || (a.causal && kbase > wave_last)) continue;  // wave-uniform
      f32x4 svc[QT][2];
      scores(base, sub, svc);
      Frag<T> vf[C::MTD];
#pragma unroll
      for (int mt = 0; mt < C::MTD; ++mt) vf[mt].load(base + (C::NKF + sub * C::MTD + mt) * kFragElems);
      // keys [kbase, kbase + rel) exist; a step needs no mask when all 32 exist and (causal)
      // every query of the wave sees all of them
      const int rel = (int)imin64(a.n_keys - kbase, 32);
      const bool full = rel == 32 && (!a.causal || kbase + 31 <= a.q_pos0 + q0);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        // lane holds raw scores of keys kbase + 8*quad + x, x = 0..7, of its query
        float sr[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) sr[x] = svc[qt][x >> 2][x & 3];
        bool has_valid = true;
        if (!full) {
          const int lim = a.causal ? (int)imin64(rel, my_pos[qt] - kbase + 1) : rel;
#pragma unroll
          for (int x = 0; x < 8; ++x)
            if (quad * 8 + x >= lim) sr[x] = -INFINITY;
          has_valid = lim > quad * 8;
        }
        // Lazy softmax reference: probabilities are formed against the running reference
        // m_run, which moves only when some probability would exceed 2^8 (or on the row's
        // first keys).  Only then does the wave take the exact row max (two shuffles) and
        // rescale O; otherwise no max, shuffle or rescale is needed.  Same softmax.
        float pv[8];
        uint32_t pm = 0;
        {
          const float m_use = m_run[qt] == -INFINITY ? 0.f : m_run[qt];
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            pv[x] = __builtin_amdgcn_exp2f(__builtin_fmaf(sr[x], scale, -m_use));
            pm = max(pm, __float_as_uint(pv[x]));  // p >= 0 (or NaN): bit order is value order
          }
        }
        const bool need = m_run[qt] == -INFINITY ? has_valid : pm > kAttnLazyBits;
        if (__any(need)) {
          float mx = fmaxf(fmaxf(fmaxf(sr[0], sr[1]), fmaxf(sr[2], sr[3])), fmaxf(fmaxf(sr[4], sr[5]), fmaxf(sr[6], sr[7])));
          mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          const float m_new = fmaxf(m_run[qt], mx * scale);  // log2 units
          const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[qt] - m_new);
          l_run[qt] *= alpha;
          m_run[qt] = m_new;
#pragma unroll
          for (int mt = 0; mt < C::MTD; ++mt) o[qt][mt] *= alpha;
          const float m_use = m_new == -INFINITY ? 0.f : m_new;
#pragma unroll
          for (int x = 0; x < 8; ++x) pv[x] = __builtin_amdgcn_exp2f(__builtin_fmaf(sr[x], scale, -m_use));
        }
        Frag<T> pf, pl;
        float psum = 0.f;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const float p = pv[x];
          pf.set(x, p);
          if constexpr (kSplitP) {
            psum += p;
            pl.set(x, p - pf.get(x));
          } else {
            psum += pf.get(x);  // normalise with the same (rounded) weights that multiply V
          }
        }
        l_run[qt] += psum;
#pragma unroll
        for (int mt = 0; mt < C::MTD; ++mt) {
          mma(o[qt][mt], vf[mt], pf);
          if constexpr (kSplitP) mma(o[qt][mt], vf[mt], pl);
        }
      }
    }
  };

  // Double-buffered walk: the copy of chunk q+1 is in flight while chunk q is computed; the
  // barrier after each chunk both completes that copy and frees the buffer just read.
  if (n_my > 0) issue(ch_begin, lds0);
  __syncthreads();
  for (int q = 0; q < n_my; q += 2) {
    if (q + 1 < n_my) issue(ch_begin + q + 1, lds1);
    if ((ch_begin + q + 1) * C::CHUNK > a.n_keys) {
      fix_tail(ch_begin + q, lds0);
      __syncthreads();
    }
    compute(ch_begin + q, lds0);
    __syncthreads();
    if (q + 1 >= n_my) break;
    if (q + 2 < n_my) issue(ch_begin + q + 2, lds0);
    if ((ch_begin + q + 2) * C::CHUNK > a.n_keys) {
      fix_tail(ch_begin + q + 1, lds1);
      __syncthreads();
    }
    compute(ch_begin + q + 1, lds1);
    __syncthreads();
  }

  if (!active) return;
  // partials: O^T tile register x of tile mt on this lane = (query q0 + 16 qt + row16, dh 16 mt + 4 quad + x)
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float l_tot = l_run[qt];
    l_tot += __shfl_xor(l_tot, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const int mq = q0 + 16 * qt + row16;
    if (mq < a.q_rows) {
      const int64_t row = ((int64_t)split * a.n_heads + h) * a.q_rows + mq;
      float* op = a.o_part + row * DH + quad * 4;
#pragma unroll
      for (int mt = 0; mt < C::MTD; ++mt) *reinterpret_cast<f32x4*>(op + 16 * mt) = o[qt][mt];
      if (quad == 0) {
        a.ml_part[row * 2] = m_run[qt];
        a.ml_part[row * 2 + 1] = l_tot;
      }
    }
  }
}

// Merge split partials in split order and normalise: one thread per (row, head, 8 dh).  O is
// written fragment-tiled for the output projection's A operand.
// All of a thread's loads (every split's max, sum and partial) are issued before any is used
// (n_split <= kAttnMaxSplit).
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
  float ms[kAttnMaxSplit], ls[kAttnMaxSplit];
  f32x4 x0s[kAttnMaxSplit], x1s[kAttnMaxSplit];
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < kAttnMaxSplit; ++s) {  // every load of the thread is in flight at once
    ms[s] = -INFINITY;
    ls[s] = 0.f;
    x0s[s] = x1s[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (s < a.n_split) {
      const int64_t row = ((int64_t)s * a.n_heads + h) * a.q_rows + m;
      const float2 p = *reinterpret_cast<const float2*>(a.ml_part + row * 2);
      const float* op = a.o_part + row * DH + c;
      x0s[s] = *reinterpret_cast<const f32x4*>(op);
      x1s[s] = *reinterpret_cast<const f32x4*>(op + 4);
      ms[s] = p.x;
      ls[s] = p.y;
      mx = fmaxf(mx, p.x);
    }
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
#pragma unroll
  for (int s = 0; s < kAttnMaxSplit; ++s) {
    if (s < a.n_split && ms[s] != -INFINITY) {
      const float f = exp2f(ms[s] - mx);
      L += ls[s] * f;
      const f32x4 x0 = x0s[s];
      const f32x4 x1 = x1s[s];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc[t] += x0[t] * f;
        acc[t + 4] += x1[t] * f;
      }
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] *= inv;
  Vec8<T>::store((T*)a.o + tiled_offset(a.row0 + m, h * DH + c, a.n_heads * DH), acc);
}

// Key splits: enough workgroups to cover the chip (~256), at least two key chunks per split, and then
// as few splits as give the same chunks per split (the longest split sets the time; fewer splits mean
// fewer partials for the merge to read).
int attention_splits(int64_t n_keys, int q_rows, int n_heads, int n_kv_heads, int causal, int max_split) {
  (void)causal;
  const int64_t n_ch = (n_keys + kAttnChunk - 1) / kAttnChunk;
  const int n_wt = (n_heads / n_kv_heads) * ((q_rows + kAttnRows - 1) / kAttnRows);
  const int base = n_kv_heads * ((n_wt + kAttnWaves - 1) / kAttnWaves);
  int s = (256 + base - 1) / base;
  if (s > max_split) s = max_split;
  if (s > kAttnMaxSplit) s = kAttnMaxSplit;
  const int64_t by_chunks = n_ch / 2;
  if (s > by_chunks) s = (int)by_chunks;
  if (s < 1) s = 1;
  const int64_t per = (n_ch + s - 1) / s;
  return (int)((n_ch + per - 1) / per);
}

template <typename T, int DH>
static void launch_attn_t(const AttnArgs& a, hipStream_t s) {
  const int n_wt = (a.n_heads / a.n_kv_heads) * ((a.q_rows + kAttnRows - 1) / kAttnRows);
  const int nb = (n_wt + kAttnWaves - 1) / kAttnWaves;
  hipLaunchKernelGGL((k_attn<T, DH, kAttnWaves, kAttnChunk / 32, kAttnQT>), dim3(nb * a.n_split * a.n_kv_heads),
                     dim3(64 * kAttnWaves), 0, s, a);
}

template <typename T>
hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.head_dim == 128)
    launch_attn_t<T, 128>(a, s);
  else
    launch_attn_t<T, 64>(a, s);
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
