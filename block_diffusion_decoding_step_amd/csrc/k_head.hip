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
// logits^T = E_tile X^T on the matrix core: a wave owns 64 vocabulary rows x 64
// slots, so each lane holds one slot (lane & 15 of each slot tile) and 16 of its
// logits per tile.  A workgroup (4 waves = 256 slots) walks vocabulary tiles
// group, group + n_groups, ...; each group writes one partial state per slot and
// a merge kernel combines the groups in fixed order (deterministic).
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

template <typename T>
struct HeadDepth;
template <>
struct HeadDepth<bf16> { static constexpr int v = 4; };
template <>
struct HeadDepth<float> { static constexpr int v = 1; };

// grid = (n_groups, ceil(n / 256)); block = 256 (4 waves x 64 slots)
template <typename T>
__global__ __launch_bounds__(256) void k_vocab_head(HeadArgs a) {
  const int lane = lane_id(), w = wave_id();
  const int row16 = lane & 15, quad = lane >> 4;
  const int slot0 = blockIdx.y * 256 + w * 64;
  if (slot0 >= a.n) return;
  const T* X = (const T*)a.x;
  const T* E = (const T*)a.E;
  const T* bp[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) bp[nt] = X + (int64_t)min(slot0 + 16 * nt + row16, a.n - 1) * a.d + quad * 8;
  Stat st[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) st[nt] = Stat{-INFINITY, 0.f, 0.f, 0x7fffffff};
  const float beta = a.beta_log2e * 0.6931471805599453f;  // inverse temperature
  const int n_vt = (a.V + 63) / 64;
  for (int vt = blockIdx.x; vt < n_vt; vt += a.n_groups) {
    const int v0 = vt * 64;
    const T* ap[4];  // E is fragment-tiled: one row tile per 16 tokens
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) ap[mt] = tiled_frag(E, min(v0 / 16 + mt, (a.V + 15) / 16 - 1), a.d / 32, 0);
    f32x4 acc[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = zero4();
    wave_gemm<T, 4, 4, HeadDepth<T>::v>(acc, ap, bp, a.d / 32, kFragElems, 32);
    // lane holds, for slot (slot0 + 16*nt + row16), tokens v0 + 16*mt + 4*quad + r
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      Stat loc{-INFINITY, 0.f, 0.f, 0x7fffffff};
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int v = v0 + 16 * mt + 4 * quad + r;
          const float l = acc[mt][nt][r] * beta;
          if (v < a.V && l > loc.m) { loc.m = l; loc.a = v; }
        }
      if (loc.m != -INFINITY) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int v = v0 + 16 * mt + 4 * quad + r;
            if (v < a.V) {
              const float dl = acc[mt][nt][r] * beta - loc.m;
              const float e = exp2f(dl * 1.4426950408889634f);
              loc.z += e;
              loc.s1 += e * dl;
            }
          }
      }
      stat_merge(st[nt], loc);
    }
  }
  // combine the four quads that share a slot, then write one partial per slot
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      Stat y;
      y.m = __shfl_xor(st[nt].m, o, 64);
      y.z = __shfl_xor(st[nt].z, o, 64);
      y.s1 = __shfl_xor(st[nt].s1, o, 64);
      y.a = __shfl_xor(st[nt].a, o, 64);
      stat_merge(st[nt], y);
    }
    const int slot = slot0 + 16 * nt + row16;
    if (quad == 0 && slot < a.n)
      a.part[(int64_t)blockIdx.x * a.n + slot] = make_float4(st[nt].m, __int_as_float(st[nt].a), st[nt].z, st[nt].s1);
  }
}

// One wave per slot: lane i merges groups i, i+64, ... in order, then a fixed
// butterfly merges the lanes.
__global__ __launch_bounds__(256) void k_head_merge(HeadArgs a) {
  const int slot = blockIdx.x * 4 + wave_id();
  if (slot >= a.n) return;
  const int lane = lane_id();
  Stat st{-INFINITY, 0.f, 0.f, 0x7fffffff};
  for (int gi = lane; gi < a.n_groups; gi += 64) {
    float4 p = a.part[(int64_t)gi * a.n + slot];
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
  }
  if (lane == 0) {
    a.pred[slot] = st.a;
    a.conf[slot] = 1.0f / st.z;
    a.ent[slot] = logf(st.z) - st.s1 / st.z;
  }
}

int head_groups(int V) {
  const int n_vt = (V + 63) / 64;
  return n_vt < 1024 ? n_vt : 1024;
}

template <typename T>
hipError_t launch_vocab_head(const HeadArgs& a, hipStream_t s) {
  dim3 grid(a.n_groups, (a.n + 255) / 256);
  hipLaunchKernelGGL(k_vocab_head<T>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_head_merge(const HeadArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_head_merge, dim3((a.n + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_vocab_head<float>(const HeadArgs&, hipStream_t);
template hipError_t launch_vocab_head<bf16>(const HeadArgs&, hipStream_t);

}  // namespace dg
