// k_head.hip — tied vocab projection fused with per-slot softmax statistics.
//
// For each canvas slot the pass needs the argmax token, the confidence (largest
// softmax probability) and the entropy over the whole vocabulary ([P5] "When to
// use a diffusion LLM", "How block diffusion works": keep the most confident
// slots, stop when the mean entropy is small; [P2] "DiffusionGemma 26B: How
// Google's Text Diffusion Model Generates Tokens in Parallel", "Architecture
// Details": 262K vocabulary).  None of it needs the logits themselves, so they
// stay in registers: per slot the kernel keeps a running
//     m  = max logit, a = its (lowest) token id,
//     Z  = sum exp(l - m),  S1 = sum exp(l - m) (l - m)
// and two such states merge as
//     m = max(ma, mb); Z = Za e^(ma-m) + Zb e^(mb-m);
//     S1 = e^(ma-m) (S1a + (ma-m) Za) + e^(mb-m) (S1b + (mb-m) Zb).
// Finally conf = 1/Z and entropy = ln Z - S1/Z.
//
// logits^T = E_tile X^T on the matrix core.  fp32 kernel (k_vocab_head), LDS-tiled; the bf16 kernel
// (k_vocab_head_bf16, below) reads E straight into registers.  A workgroup (8 waves)
// owns 256 slots and walks 256-token vocabulary tiles blockIdx.x, +gridDim.x, ...
// For each pair of 32-wide K steps it stages the tiles' fragments of E (16 row
// fragments, read once from HBM) and of X (16 slot fragments, from L2) in LDS,
// double-buffered so that the next stage's global loads are in flight while
// the matrix core works on this one.  Wave w computes 64 tokens (w % 4) x 128
// slots (w / 4): each lane holds one slot per 16-slot fragment and 16 of its
// logits per tile, folds them into a running per-slot state, and at the end the
// four quads of a wave and the four token waves of a slot are merged in fixed
// order into one partial per (workgroup, slot).  A merge kernel combines the
// workgroups in fixed order (deterministic).
//
// Sampling variant (gumbel): the recommended sampler draws each slot's token from
// the softmax at the pass's temperature ([P2] "Architecture Details").  By the
// Gumbel-max identity the token argmax_v (beta l_v + G_v), with independent
// standard Gumbel G_v, is such a draw, so the fold also keeps the best perturbed
// score, its token and its scaled logit; conf becomes the probability of the drawn
// token, e^(beta l_a - m) / Z.  G_v = -ln(-ln u), u = (2 floor(w / 2^9) + 1) / 2^24
// (exact in fp32, never 0 or 1), w = word v mod 4 of Philox4x32-10 at counter
// (v / 4, row + 2^16 step, block, 1): one generator call serves four tokens.
#include <type_traits>
#include <utility>

#include "dg_device.h"
#include "dg_kernels.h"
#include "dg_wave_gemm.h"

namespace dg {

struct Stat {
  float m, z, s1;
  int a;
};

__device__ __forceinline__ void stat_merge(Stat& x, const Stat& y) {
  // y may come from lower token ids only through the explicit id comparison below
  const bool take = y.m > x.m || (y.m == x.m && y.a < x.a);
  const float m = fmaxf(x.m, y.m);
  if (m == -INFINITY) {
    if (take) x = y;
    return;
  }
  const float ex = exp2f((x.m - m) * 1.4426950408889634f);
  const float ey = exp2f((y.m - m) * 1.4426950408889634f);
  const float dx = x.m == -INFINITY ? 0.f : x.m - m;
  const float dy = y.m == -INFINITY ? 0.f : y.m - m;
  const float z = x.z * ex + y.z * ey;
  const float s1 = ex * (x.s1 + dx * x.z) + ey * (y.s1 + dy * y.z);
  x.a = take ? y.a : x.a;
  x.m = m;
  x.z = z;
  x.s1 = s1;
}

// the draw of the sampling variant: best perturbed score g, its scaled logit l, its token a
struct Draw {
  float g, l;
  int a;
};
__device__ __forceinline__ void draw_merge(Draw& x, const Draw& y) {
  if (y.g > x.g || (y.g == x.g && y.a < x.a)) x = y;
}
__device__ __forceinline__ Draw draw_shfl(const Draw& x, int o) {
  return Draw{__shfl_xor(x.g, o, 64), __shfl_xor(x.l, o, 64), __shfl_xor(x.a, o, 64)};
}
constexpr Draw kNoDraw{-INFINITY, 0.f, 0x7fffffff};

// Gumbel noise of tokens 4q .. 4q+3 of row `row`.  -ln u is taken from the Mercator series of
// -ln(1 - e), e = 1 - u (exact), when u > 15/16, where a log of u itself would lose the small
// result to cancellation; eight terms leave a relative error below 1e-10 there.  The logs are the
// hardware log2 (normal inputs only: u >= 2^-24, -ln u >= 2^-24).
__device__ __forceinline__ float gumbel_of(uint32_t w) {
  constexpr float kLn2 = 0.6931471805599453f;
  const uint32_t k = w >> 9;                                     // u = (2k + 1) / 2^24
  const float u = (float)(2u * k + 1u) * 0x1p-24f;
  const float e = (float)((1u << 24) - 2u * k - 1u) * 0x1p-24f;  // 1 - u
  float sr = 1.f / 8.f;
#pragma unroll
  for (int n = 7; n >= 1; --n) sr = fmaf(e, sr, 1.f / (float)n);
  const float far = -kLn2 * __builtin_amdgcn_logf(u);
  const float inner = e < 0.0625f ? e * sr : far;
  return -kLn2 * __builtin_amdgcn_logf(inner);
}
__device__ __forceinline__ void gumbel4(const HeadArgs& a, uint32_t q, uint32_t row, float (&g)[4]) {
  const uint4 w = philox4x32_10(q, row + (a.step << 16), a.block, 1u, a.k0, a.k1);
  g[0] = gumbel_of(w.x);
  g[1] = gumbel_of(w.y);
  g[2] = gumbel_of(w.z);
  g[3] = gumbel_of(w.w);
}

// calls f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>) in order: a loop that is always
// fully unrolled (register arrays indexed by the counter stay in registers at any body size)
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <typename T>
struct HeadCfg {
  static constexpr int KC = sizeof(T) == 2 ? 2 : 1;   // K steps per stage
  static constexpr int FB = kFragElems * (int)sizeof(T);  // bytes per fragment
  static constexpr int STAGE = KC * 32 * FB;           // 16 E + 16 X fragments per K step: 64 KB
  static constexpr int UPL = FB / 64 / 16;             // 16-byte units per lane per fragment
  static constexpr int LOADS = STAGE / 16 / 512;       // 16-byte loads per thread per stage
};

constexpr int kHeadSlots = 256;    // slots per workgroup
constexpr int kHeadTokens = 256;   // vocabulary rows per tile
constexpr int kHeadMaxGroups = 256;

// grid = (n_groups, ceil(n / 256)); block = 512
template <typename T, bool DRAW>
__global__ __launch_bounds__(512, 1) void k_vocab_head(HeadArgs a) {
  using C = HeadCfg<T>;
  static_assert(C::LOADS == 8, "stage layout");
  __shared__ uint4 lds[2 * C::STAGE / 16];
  const int t = threadIdx.x, lane = lane_id(), w = wave_id();
  const int wv = w & 3, wsl = w >> 2;  // token quarter, slot half
  const int quad = lane >> 4, row16 = lane & 15;
  const int slot_base = blockIdx.y * kHeadSlots;
  const int ks = a.d / 32;
  const int nch = (ks + C::KC - 1) / C::KC;
  const int n_tiles = (a.V + kHeadTokens - 1) / kHeadTokens;
  const int G = gridDim.x;
  const int my_tiles = (n_tiles - (int)blockIdx.x + G - 1) / G;
  const int total = my_tiles * nch;
  const int last_rt = (a.V + 15) / 16 - 1;
  const T* E = (const T*)a.E;
  const T* X = (const T*)a.x;
  const float beta = a.beta_log2e * 0.6931471805599453f;  // inverse temperature

  // Stage q = (tile blockIdx.x + (q / nch) * G, chunk q % nch).  Thread t moves the
  // 16-byte units j*512 + t of the stage: unit u is byte 16u of the stage, i.e.
  // fragment u / (64*UPL) (K step, then 16 E fragments, then 16 X fragments),
  // lane (u % (64*UPL)) / UPL of it, part u % UPL of that lane's 8 elements.
  auto issue = [&](int q, uint4 (&r)[C::LOADS]) {
    const int tile = (int)blockIdx.x + (q / nch) * G, c = q % nch;
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) {
      const int u = j * 512 + t;
      const int g = u / (64 * C::UPL), qq = u % (64 * C::UPL);
      const int fl = qq / C::UPL, part = qq % C::UPL;
      const int kk = g >> 5, which = (g >> 4) & 1, idx = g & 15;
      const int s = c * C::KC + kk;
      const T* src;
      if (which == 0) {
        const int rt = min(tile * (kHeadTokens / 16) + idx, last_rt);
        src = E + ((int64_t)rt * ks + min(s, ks - 1)) * kFragElems + fl * 8;
      } else {
        const int row = min(slot_base + 16 * idx + (fl & 15), a.n - 1);
        src = X + (int64_t)row * a.d + 32 * min(s, ks - 1) + 8 * (fl >> 4);
      }
      src += part * (16 / (int)sizeof(T));
      r[j] = s < ks ? *reinterpret_cast<const uint4*>(src) : uint4{0u, 0u, 0u, 0u};
    }
  };
  auto commit = [&](int buf, const uint4 (&r)[C::LOADS]) {
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) lds[buf * (C::STAGE / 16) + j * 512 + t] = r[j];
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = zero4();
  Stat st[8];
  Draw dr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    st[j] = Stat{-INFINITY, 0.f, 0.f, 0x7fffffff};
    dr[j] = kNoDraw;
  }

  uint4 r[C::LOADS];
  if (total > 0) {
    issue(0, r);
    commit(0, r);
  }
  __syncthreads();
  for (int q = 0; q < total; ++q) {
    if (q + 1 < total) issue(q + 1, r);
    const T* base = reinterpret_cast<const T*>(lds) + (q & 1) * (C::STAGE / (int)sizeof(T));
#pragma unroll
    for (int kk = 0; kk < C::KC; ++kk) {
      const T* kb = base + kk * 32 * kFragElems + lane * 8;
      Frag<T> fa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i].load(kb + (4 * wv + i) * kFragElems);
      if constexpr (sizeof(T) == 2) {
        Frag<T> fb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) fb[j].load(kb + (16 + 8 * wsl + j) * kFragElems);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) mma(acc[i][j], fa[i], fb[j]);
      } else {  // fp32 fragments are twice the size: one slot fragment at a time
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          Frag<T> fb;
          fb.load(kb + (16 + 8 * wsl + j) * kFragElems);
#pragma unroll
          for (int i = 0; i < 4; ++i) mma(acc[i][j], fa[i], fb);
        }
      }
    }
    if (q % nch == nch - 1) {
      // tile finished: lane holds, for slot slot_base + 128*wsl + 16*j + row16,
      // tokens v0 + 16*i + 4*quad + rr
      const int v0 = ((int)blockIdx.x + (q / nch) * G) * kHeadTokens + 64 * wv;
      static_for<8>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        Stat loc{-INFINITY, 0.f, 0.f, 0x7fffffff};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int v = v0 + 16 * i + 4 * quad + rr;
            const float l = acc[i][j][rr] * beta;
            if (v < a.V && l > loc.m) { loc.m = l; loc.a = v; }
          }
        if (loc.m != -INFINITY) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int v = v0 + 16 * i + 4 * quad + rr;
              if (v < a.V) {
                const float dl = acc[i][j][rr] * beta - loc.m;
                const float e = exp2f(dl * 1.4426950408889634f);
                loc.z += e;
                loc.s1 += e * dl;
              }
            }
        }
        stat_merge(st[j], loc);
        if constexpr (DRAW) {
          const uint32_t row = (uint32_t)(slot_base + 128 * wsl + 16 * j + row16);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float gn[4];
            gumbel4(a, (uint32_t)(v0 + 16 * i + 4 * quad) >> 2, row, gn);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int v = v0 + 16 * i + 4 * quad + rr;
              const float l = acc[i][j][rr] * beta;
              if (v < a.V && l + gn[rr] > dr[j].g) dr[j] = Draw{l + gn[rr], l, v};
            }
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = zero4();
      });
    }
    if (q + 1 < total) commit((q + 1) & 1, r);
    __syncthreads();
  }
  // merge the four quads (lanes 16 apart hold the same slot), then the four token waves
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      Stat y;
      y.m = __shfl_xor(st[j].m, o, 64);
      y.z = __shfl_xor(st[j].z, o, 64);
      y.s1 = __shfl_xor(st[j].s1, o, 64);
      y.a = __shfl_xor(st[j].a, o, 64);
      stat_merge(st[j], y);
      if constexpr (DRAW) draw_merge(dr[j], draw_shfl(dr[j], o));
    }
  }
  float4* red = reinterpret_cast<float4*>(lds);  // [4 token waves][256 slots]; stages are no longer read
  float4* redd = red + 4 * kHeadSlots;          // the draws, same layout
  if (quad == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int o = wv * kHeadSlots + 128 * wsl + 16 * j + row16;
      red[o] = make_float4(st[j].m, __int_as_float(st[j].a), st[j].z, st[j].s1);
      if constexpr (DRAW) redd[o] = make_float4(dr[j].g, dr[j].l, __int_as_float(dr[j].a), 0.f);
    }
  }
  __syncthreads();
  if (t < kHeadSlots && slot_base + t < a.n) {
    float4 p = red[t];
    Stat x{p.x, p.z, p.w, __float_as_int(p.y)};
#pragma unroll
    for (int k = 1; k < 4; ++k) {
      p = red[k * kHeadSlots + t];
      stat_merge(x, Stat{p.x, p.z, p.w, __float_as_int(p.y)});
    }
    const int64_t o = (int64_t)blockIdx.x * a.n + slot_base + t;
    if constexpr (DRAW) {
      Draw y = kNoDraw;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 q = redd[k * kHeadSlots + t];
        draw_merge(y, Draw{q.x, q.y, __float_as_int(q.z)});
      }
      x.a = y.a;
      a.part2[o] = make_float2(y.g, y.l);
    }
    a.part[o] = make_float4(x.m, __int_as_float(x.a), x.z, x.s1);
  }
}

// bf16: wave w owns 32 tokens (two E fragments, tokens 32w .. 32w+31 of the tile) x all 256 slots, so
// every E fragment is loaded by exactly one wave, straight into a four-deep register ring, with
// non-temporal loads (the vocabulary is read once per pass; streaming it past the caches measured 15%
// faster).  The slot
// operand X (16 fragments per K step) is staged in LDS, two K steps per stage, double-buffered, and
// read by all eight waves; its global loads (L2 hits) are issued two stages ahead of use, since one
// stage of matrix work is shorter than their round trip while the vocabulary stream loads the memory
// system.  The running per-slot states live in LDS and the eight token waves of a slot merge in wave
// order.
constexpr int kHeadKC = 2;  // K steps per X stage; the E ring holds the K steps of two stages (a loop turn):
                            // the ring slot of a K step is KC * (stage parity) + its index in the stage

// FP8 vocabulary (F8): E holds E4M3 codes in the FP8 pair-tiled layout; the register ring holds each K step's
// 8 code bytes per lane and fragment (half the bytes and registers of the bf16 ring), decoded to bf16 fragments
// when used; the fold multiplies each token's fp32 dot product by its row scale (read once per tile, at the
// tile's first stage).
template <bool DRAW, bool F8>
__global__ __launch_bounds__(512, 1) void k_vocab_head_bf16(HeadArgs a) {
  using T = bf16;
  // the draw's generator needs registers: it runs with one K step per stage (a two-step E ring)
  constexpr int KC = DRAW ? 1 : kHeadKC;
  constexpr int EDEPTH = 2 * KC;
  constexpr int STAGE = KC * 16 * kFragElems * 2;  // X fragments of KC steps: 32 KB at KC = 2
  constexpr int LOADS = STAGE / 16 / 512;                // 16-byte units per thread per stage
  static_assert(LOADS * 16 * 512 == STAGE, "stage layout");
  __shared__ uint4 lds[2 * STAGE / 16];
  __shared__ float4 run[8][kHeadSlots];  // running (max, argmax bits, Z, S1) per token wave and slot
  __shared__ float4 rund[DRAW ? 8 : 1][kHeadSlots];  // gumbel: running draw (g, l, token bits, -)
  const int t = threadIdx.x, lane = lane_id(), w = wave_id();
  const int quad = lane >> 4;
  const int row16 = lane & 15;
  const int slot_base = blockIdx.y * kHeadSlots;
  const int ks = a.d / 32;
  const int nch = (ks + KC - 1) / KC;
  const int n_tiles = (a.V + kHeadTokens - 1) / kHeadTokens;
  const int G = gridDim.x;
  const int my_tiles = (n_tiles - (int)blockIdx.x + G - 1) / G;
  const int total = my_tiles * nch;
  const int last_rt = (a.V + 15) / 16 - 1;
  const T* E = (const T*)a.E;
  const T* X = (const T*)a.x;
  const float beta = a.beta_log2e * 0.6931471805599453f;  // inverse temperature

  // X stage q = (tile q / nch, chunk q % nch): unit u = j*512 + t is lane u % 64 of X fragment u / 64
  // (K step (u / 64) / 16 of the chunk, slot fragment (u / 64) % 16)
  auto issue = [&](int q, uint4 (&r)[LOADS]) __attribute__((always_inline)) {
    const int c = q % nch;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int u = j * 512 + t;
      const int g = u >> 6, fl = u & 63;
      const int s = c * KC + (g >> 4);
      const int row = min(slot_base + 16 * (g & 15) + (fl & 15), a.n - 1);
      const T* src = X + (int64_t)row * a.d + 32 * min(s, ks - 1) + 8 * (fl >> 4);
      r[j] = s < ks ? *reinterpret_cast<const uint4*>(src) : uint4{0u, 0u, 0u, 0u};
    }
  };
  auto commit = [&](int buf, const uint4 (&r)[LOADS]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) lds[buf * (STAGE / 16) + j * 512 + t] = r[j];
  };

  // FP8: the row scales (times beta) of this lane's 8 tokens of the current tile
  float sc[2][4];
  auto scale_load = [&](int q) __attribute__((always_inline)) {
    const int v0 = ((int)blockIdx.x + (q / nch) * G) * kHeadTokens + 32 * w + 4 * quad;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sc[i][rr] = a.e_scale[min(v0 + 16 * i + rr, a.V - 1)] * beta;
  };
  // E fragments of flat K step f (over this workgroup's tiles); steps past the end reload the last one
  const int nsteps = total * KC;
  // FP8: this lane's 8 code bytes of the two fragments of flat K step f: half (step & 1) of the lane's 16 bytes
  // in the step's 64-column block
  const uint8_t* E8 = (const uint8_t*)a.E;
  auto e8_load = [&](int f, u32x2 (&e)[2]) __attribute__((always_inline)) {
    f = min(f, nsteps - 1);
    const int tl = f / (nch * KC), st = f % (nch * KC);
    const int tile = (int)blockIdx.x + tl * G;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rt = min(tile * (kHeadTokens / 16) + 2 * w + i, last_rt);
      const uint8_t* p = E8 + ((int64_t)rt * (ks / 2) + st / 2) * 1024 + lane * 16 + (st & 1) * 8;
      e[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));  // read once per pass: streamed
    }
  };
  auto e_load = [&](int f, Frag<T> (&e)[2]) __attribute__((always_inline)) {
    f = min(f, nsteps - 1);
    const int tl = f / (nch * KC), s = f % (nch * KC);
    const int tile = (int)blockIdx.x + tl * G;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rt = min(tile * (kHeadTokens / 16) + 2 * w + i, last_rt);
      e[i].load_nt(tiled_frag(E, rt, ks, min(s, ks - 1)));  // read once per pass: streamed
    }
  };

  f32x4 acc[2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] = zero4();
  for (int i = lane; i < kHeadSlots; i += 64) {
    run[w][i] = make_float4(-INFINITY, __int_as_float(0x7fffffff), 0.f, 0.f);
    if constexpr (DRAW) rund[w][i] = make_float4(-INFINITY, 0.f, __int_as_float(0x7fffffff), 0.f);
  }

  // tile finished: lane holds, for slot slot_base + 16*j + row16, tokens v0 + 16*i + 4*quad + rr
  auto fold_tile = [&](int q) __attribute__((always_inline)) {
    const int v0 = ((int)blockIdx.x + (q / nch) * G) * kHeadTokens + 32 * w;
    static_for<16>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      Stat loc{-INFINITY, 0.f, 0.f, 0x7fffffff};
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int v = v0 + 16 * i + 4 * quad + rr;
          const float l = acc[i][j][rr] * (F8 ? sc[i][rr] : beta);
          if (v < a.V && l > loc.m) { loc.m = l; loc.a = v; }
        }
      if (loc.m != -INFINITY) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int v = v0 + 16 * i + 4 * quad + rr;
            if (v < a.V) {
              const float dl = acc[i][j][rr] * (F8 ? sc[i][rr] : beta) - loc.m;
              const float e = exp2f(dl * 1.4426950408889634f);
              loc.z += e;
              loc.s1 += e * dl;
            }
          }
      }
      // the four quads hold the same slot: merge them, then fold into the running state
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        Stat y;
        y.m = __shfl_xor(loc.m, o, 64);
        y.z = __shfl_xor(loc.z, o, 64);
        y.s1 = __shfl_xor(loc.s1, o, 64);
        y.a = __shfl_xor(loc.a, o, 64);
        stat_merge(loc, y);
      }
      Draw dl = kNoDraw;
      if constexpr (DRAW) {
        const uint32_t row = (uint32_t)(slot_base + 16 * j + row16);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          float gn[4];
          gumbel4(a, (uint32_t)(v0 + 16 * i + 4 * quad) >> 2, row, gn);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int v = v0 + 16 * i + 4 * quad + rr;
            const float l = acc[i][j][rr] * (F8 ? sc[i][rr] : beta);
            if (v < a.V && l + gn[rr] > dl.g) dl = Draw{l + gn[rr], l, v};
          }
        }
#pragma unroll
        for (int o = 16; o <= 32; o <<= 1) draw_merge(dl, draw_shfl(dl, o));
      }
      if (quad == 0) {
        const float4 p = run[w][16 * j + row16];
        Stat x{p.x, p.z, p.w, __float_as_int(p.y)};
        stat_merge(x, loc);
        run[w][16 * j + row16] = make_float4(x.m, __int_as_float(x.a), x.z, x.s1);
        if constexpr (DRAW) {
          const float4 q = rund[w][16 * j + row16];
          Draw y{q.x, q.y, __float_as_int(q.z)};
          draw_merge(y, dl);
          rund[w][16 * j + row16] = make_float4(y.g, y.l, __int_as_float(y.a), 0.f);
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[i][j] = zero4();
    });
  };

  Frag<T> ering[F8 ? 1 : EDEPTH][2];
  u32x2 ering8[F8 ? EDEPTH : 1][2];
#pragma unroll
  for (int dd = 0; dd < EDEPTH; ++dd) {
    if constexpr (F8) e8_load(dd, ering8[dd]);
    else e_load(dd, ering[dd]);
  }
  // X loads run two stages ahead of their LDS stage: stage q's data is requested at the start of stage
  // q - 2 into register set q & 1 and written to LDS buffer q & 1 at the end of stage q - 1
  uint4 r[2][LOADS];
  if (total > 0) {
    issue(0, r[0]);
    commit(0, r[0]);
  }
  if (total > 1) issue(1, r[1]);
  __syncthreads();
  // stage q (X buffer and register set q & 1 = B): K steps 2q, 2q+1 use ring slots 2B, 2B+1
  auto stage = [&](int q, auto bparity) __attribute__((always_inline)) {
    constexpr int B = decltype(bparity)::value;
    if (q + 2 < total) issue(q + 2, r[B]);
    if constexpr (F8)
      if (q % nch == 0) scale_load(q);
    const T* base = reinterpret_cast<const T*>(lds) + B * (STAGE / 2) + lane * 8;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      Frag<T> ea[2];
      if constexpr (F8) {
        ea[0] = fp8x8_to_bf16(ering8[KC * B + kk][0]);
        ea[1] = fp8x8_to_bf16(ering8[KC * B + kk][1]);
      } else {
        ea[0] = ering[KC * B + kk][0];
        ea[1] = ering[KC * B + kk][1];
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        Frag<T> fb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) fb[j].load(base + (kk * 16 + 8 * half + j) * kFragElems);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) mma(acc[i][8 * half + j], ea[i], fb[j]);
      }
      if constexpr (F8) e8_load(q * KC + kk + EDEPTH, ering8[KC * B + kk]);
      else e_load(q * KC + kk + EDEPTH, ering[KC * B + kk]);
    }
    if (q % nch == nch - 1) fold_tile(q);
    if (q + 1 < total) commit(1 - B, r[1 - B]);
    __syncthreads();
  };
  for (int q = 0; q < total; q += 2) {
    stage(q, std::integral_constant<int, 0>{});
    if (q + 1 < total) stage(q + 1, std::integral_constant<int, 1>{});
  }
  if (t < kHeadSlots && slot_base + t < a.n) {
    float4 p = run[0][t];
    Stat x{p.x, p.z, p.w, __float_as_int(p.y)};
#pragma unroll
    for (int k2 = 1; k2 < 8; ++k2) {
      p = run[k2][t];
      stat_merge(x, Stat{p.x, p.z, p.w, __float_as_int(p.y)});
    }
    const int64_t o = (int64_t)blockIdx.x * a.n + slot_base + t;
    if constexpr (DRAW) {
      Draw y = kNoDraw;
#pragma unroll
      for (int k2 = 0; k2 < 8; ++k2) {
        const float4 q = rund[k2][t];
        draw_merge(y, Draw{q.x, q.y, __float_as_int(q.z)});
      }
      x.a = y.a;
      a.part2[o] = make_float2(y.g, y.l);
    }
    a.part[o] = make_float4(x.m, __int_as_float(x.a), x.z, x.s1);
  }
}

// One wave per slot: lane i merges groups i, i+64, ... in order, then a fixed
// butterfly merges the lanes.
template <bool DRAW>
__global__ __launch_bounds__(256) void k_head_merge(HeadArgs a) {
  const int slot = blockIdx.x * 4 + wave_id();
  if (slot >= a.n) return;
  const int lane = lane_id();
  Stat st{-INFINITY, 0.f, 0.f, 0x7fffffff};
  Draw dr = kNoDraw;
  for (int gi = lane; gi < a.n_groups; gi += 64) {
    const int64_t o = (int64_t)gi * a.n + slot;
    float4 p = a.part[o];
    if constexpr (DRAW) {
      const float2 q = a.part2[o];
      draw_merge(dr, Draw{q.x, q.y, __float_as_int(p.y)});
      p.y = __int_as_float(0x7fffffff);  // the slot's argmax is not needed
    }
    Stat y{p.x, p.z, p.w, __float_as_int(p.y)};
    stat_merge(st, y);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    Stat y;
    y.m = __shfl_xor(st.m, o, 64);
    y.z = __shfl_xor(st.z, o, 64);
    y.s1 = __shfl_xor(st.s1, o, 64);
    y.a = __shfl_xor(st.a, o, 64);
    stat_merge(st, y);
    if constexpr (DRAW) draw_merge(dr, draw_shfl(dr, o));
  }
  if (lane == 0) {
    if constexpr (DRAW) {
      a.pred[slot] = dr.a;
      a.conf[slot] = exp2f((dr.l - st.m) * 1.4426950408889634f) / st.z;
    } else {
      a.pred[slot] = st.a;
      a.conf[slot] = 1.0f / st.z;
    }
    a.ent[slot] = logf(st.z) - st.s1 / st.z;
  }
}

int head_groups(int V) {
  const int n_tiles = (V + kHeadTokens - 1) / kHeadTokens;
  return n_tiles < kHeadMaxGroups ? n_tiles : kHeadMaxGroups;
}

template <typename T>
hipError_t launch_vocab_head(const HeadArgs& a, hipStream_t s) {
  dim3 grid(a.n_groups, (a.n + kHeadSlots - 1) / kHeadSlots);
  if constexpr (sizeof(T) == 2) {
    if (a.e_scale) {
      if (a.d % 64) return hipErrorInvalidValue;  // FP8 pair-tiled rows: whole 64-column blocks
      if (a.gumbel)
        hipLaunchKernelGGL((k_vocab_head_bf16<true, true>), grid, dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((k_vocab_head_bf16<false, true>), grid, dim3(512), 0, s, a);
    } else if (a.gumbel) {
      hipLaunchKernelGGL((k_vocab_head_bf16<true, false>), grid, dim3(512), 0, s, a);
    } else {
      hipLaunchKernelGGL((k_vocab_head_bf16<false, false>), grid, dim3(512), 0, s, a);
    }
  } else {
    if (a.gumbel)
      hipLaunchKernelGGL((k_vocab_head<T, true>), grid, dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((k_vocab_head<T, false>), grid, dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_head_merge(const HeadArgs& a, hipStream_t s) {
  if (a.gumbel)
    hipLaunchKernelGGL(k_head_merge<true>, dim3((a.n + 3) / 4), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_head_merge<false>, dim3((a.n + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_vocab_head<float>(const HeadArgs&, hipStream_t);
template hipError_t launch_vocab_head<bf16>(const HeadArgs&, hipStream_t);

}  // namespace dg
