// dg_kernels.h — host-side launchers of the libdg kernels (internal to libdg).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dg.h"

namespace dg {

typedef __bf16 bf16;

// limits of the routing kernels: rows per launch (two per thread of the ordering workgroup) and
// the ordering workgroup's LDS masks, one per (expert, 64-token chunk)
constexpr int kRouteMaxRows = 2048;
constexpr int kRouteMasks = 4096;

// rows per routed-expert work tile, and the bound on the number of tiles.  A tile is the int4
// (expert, first pair, rows, packed) with packed = tiles of that expert | (index of this tile among
// them) << 8 | (rows of the expert's last tile) << 16; an expert holds at most 2048 pairs (64 tiles).
// Calls with many rows per expert (stacked canvases, prompt chunks) use tiles of kMoeWideRows.
constexpr int kMoeTileRows = 32;
constexpr int kMoeWideRows = 64;
inline int moe_tile_rows(int M, int E, int k) { return M * k >= 48 * E ? kMoeWideRows : kMoeTileRows; }
__host__ __device__ inline int moe_pack_tile_w(int tiles_of_expert, int index, int last_rows) {
  return tiles_of_expert | (index << 8) | (last_rows << 16);
}
inline int moe_max_tiles(int M, int E, int k) { return E + (M * k + kMoeTileRows - 1) / kMoeTileRows; }

inline int moe_max_rows(int E) {
  const int by_masks = 64 * (kRouteMasks / E);
  return by_masks < kRouteMaxRows ? by_masks : kRouteMaxRows;
}


struct StopParams {
  float threshold;
  float ln_vocab;
  int max_steps;
  int fixed_steps;
  int and_rule;  // early stop needs low entropy and two unchanged passes together
};

// keep the best `keep` slots (confidence, or lowest entropy with rank_entropy; locked slots first
// and always), kept slots take pred (locked ones keep their canvas token), the rest a Philox draw
struct CanvasArgs {
  const int32_t* pred;
  const float* conf;
  const float* ent;       // read with rank_entropy
  int rank_entropy;
  const uint8_t* lock;    // null, or the locked slots (may alias keep_mask)
  int S, keep;
  uint64_t seed;
  uint32_t block, step, V;
  int32_t* canvas;        // in/out (read at locked slots)
  uint8_t* keep_mask;     // optional output
};

// ---- k_misc.hip
template <typename T>
hipError_t launch_embed(const int32_t* tok, const T* E, T* X, int M, int d, int V, hipStream_t s);
// X[m] = bf16(code(E[tok[m]]) * scale[tok[m]]) for an E4M3 embedding in the FP8 pair-tiled layout
hipError_t launch_embed_f8(const int32_t* tok, const uint8_t* E, const float* scale, bf16* X, int M, int d, int V,
                           hipStream_t s);
template <typename T>
hipError_t launch_pack(const T* src, T* dst, int64_t batch, int64_t rows, int64_t cols, hipStream_t s);
// per-row E4M3 scales and codes of `batch` row-major [rows, cols] bf16 matrices (cols a multiple of 64), codes in
// the FP8 pair-tiled layout (rows padded to 16 with zeros)
hipError_t launch_quantize_e4m3(const bf16* src, uint8_t* dst, float* scale, int64_t batch, int64_t rows, int64_t cols,
                                hipStream_t s);
// Y (row-major) and / or Yt (fragment-tiled, rows padded to 16); either may be null
template <typename T>
hipError_t launch_rmsnorm(const T* X, const T* g, T* Y, T* Yt, int M, int d, float eps, hipStream_t s,
                          hipEvent_t done = nullptr);  // done (optional): completes with the kernel

// router logits + top-k, then softmax weights and the token->expert order (two launches;
// E <= 256, k <= 16, M <= moe_max_rows(E), d a multiple of 32)
struct RouteArgs {
  const void* Xt;     // FFN-normalised rows, fragment-tiled (rows padded to 16)
  const void* Wr;     // router weights [E, d], fragment-tiled
  float* logits;      // [M, E] fp32
  float* cand_v;      // [M][2][k] scratch: each expert slice's best logits, best first
  int32_t* cand_e;    // [M][2][k] scratch: their experts (-1: none)
  int32_t* idx;       // [M, k] chosen experts, best first
  float* w;           // [M, k] softmax over the chosen logits
  int32_t* counts;    // [E] pairs per expert
  int32_t* offsets;   // [E + 1] first pair of each expert
  int32_t* perm;      // [M * k] pair slot -> token
  int32_t* pos;       // [M * k] (token, choice) -> pair slot
  int4* tiles;        // work tiles (expert, first pair, rows, packed as moe_pack_tile_w)
  int32_t* n_tiles;
  int M, d, E, k;
  int tile_rows;      // kMoeTileRows or kMoeWideRows
};
constexpr int kRouteSlices = 2;  // expert slices of the router (candidate lists per row)
template <typename T>
hipError_t launch_route(const RouteArgs& a, hipStream_t s);
// X += Ys + sum_j w_j Yp[pos_j]; with g != null also Yn = RMSNorm(X) * g (tiled or row-major)
template <typename T>
hipError_t launch_moe_combine(T* X, const T* Ys, const T* Yp, const int32_t* pos, const float* w, int M, int d,
                              int k, const T* g, T* Yn, int yn_tiled, float eps, hipStream_t s);
// with lock (non-null) the locked slots' predictions are replaced by their canvas tokens first
hipError_t launch_stop_check(const float* ent, int32_t* pred, int32_t* prev, const int32_t* canvas,
                             const uint8_t* lock, int S, int step, StopParams sp, dg_block_status* out,
                             hipStream_t s);
hipError_t launch_canvas_update(const CanvasArgs& a, hipStream_t s);

// keys and values of one sequence's rows of a batched call: from the call's staging buffers (QKV epilogue
// with cap = M, pos0 = 0) to positions pos0.. of the sequence's cache
struct KvScatterArgs {
  const void* ks;  // [Hkv][M][Dh]
  const void* vs;  // [Hkv][Dh][M]
  int M, n_kv_heads, head_dim;
  void* kc;        // the layer's key cache   [Hkv][cap][Dh]
  void* vc;        // the layer's value cache [Hkv][Dh][cap]
  int64_t cap, pos0;
  int row0, rows;  // the sequence's rows of the call
};
template <typename T>
hipError_t launch_kv_scatter(const KvScatterArgs& a, hipStream_t s);

// ---- k_gemm.hip
enum class GemmEpi { Store, Resid, QKV, SwiGLU };

struct GemmArgs {
  const void* A;   // [M, K] rows, lda elements apart; or fragment-tiled (a_tiled, rows padded to 16)
  int a_tiled;
  const void* B;   // [N, K] rows (weights, [out, in])
  void* C;         // output (meaning depends on the epilogue)
  int M, N, K;
  int lda, ldb, ldc;
  // QKV epilogue
  void* q;         // [Hq][q_rows][Dh]
  void* kc;        // key cache of this layer   [Hkv][cap][Dh]
  void* vc;        // value cache of this layer [Hkv][Dh][cap]
  int n_heads, n_kv_heads, head_dim;
  int q_rows;
  int64_t cap, pos0;
  // SwiGLU epilogue: N = F (output width); B holds 2F rows: gate rows then up rows; the output
  // [M, F] is stored fragment-tiled (its only reader is the next GEMM's A operand)
};

template <typename T>
hipError_t launch_gemm(GemmEpi epi, const GemmArgs& a, hipStream_t s, hipEvent_t done = nullptr);

struct MoeArgs {
  const int4* tiles;      // (expert, first pair, rows, packed as moe_pack_tile_w)
  const int32_t* n_tiles;
  int max_tiles;
  const int32_t* perm;    // pair -> token (gate_up gathers rows through it)
  const void* X;          // gate_up: normalised hidden [M, d]; down: H [pairs, F]
  const void* W;          // gate_up: [E][2F][d]; down: [E][d][F]
  void* out;              // gate_up: H [pairs, F]; down: Yp [pairs, d]
  int d, F;
  int tile_rows;          // as the routing's
  const float* scale;     // FP8 weights: per-output-channel scales, gate_up [E][2F], down [E][d]
};
template <typename T>
hipError_t launch_moe_gate_up(const MoeArgs& a, hipStream_t s);
template <typename T>
hipError_t launch_moe_down(const MoeArgs& a, hipStream_t s);
// FP8 (E4M3) expert weights in the pair-tiled layout, bf16 activations
hipError_t launch_moe_gate_up_f8(const MoeArgs& a, hipStream_t s);
hipError_t launch_moe_down_f8(const MoeArgs& a, hipStream_t s);

// ---- k_attn.hip
struct AttnArgs {
  const void* q;      // [Hq][q_stride][Dh]; this launch's queries are rows [row0, row0 + q_rows) of each head
  const void* kc;     // [Hkv][cap][Dh]
  const void* vc;     // [Hkv][Dh][cap]
  float* o_part;      // [n_split][Hq][q_rows][Dh]
  float* ml_part;     // [n_split][Hq][q_rows][2]  (running max in log2 units, sum)
  void* o;            // [layer rows][Hq*Dh], fragment-tiled (rows padded to 16); this launch writes rows row0..
  int q_rows;         // query rows of this launch
  int q_stride;       // rows per head in q (the layer's rows)
  int row0;           // first row of this launch in q and in o
  int n_heads, n_kv_heads, head_dim;
  int64_t cap;
  int64_t n_keys;     // keys visible: [0, n_keys)
  int64_t q_pos0;     // absolute position of query row 0 (causal)
  int causal;
  int n_split;
};
template <typename T>
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
template <typename T>
hipError_t launch_attention_merge(const AttnArgs& a, hipStream_t s);
constexpr int kAttnMaxSplit = 16;  // key splits of one attention launch (partials per row)
int attention_splits(int64_t n_keys, int q_rows, int n_heads, int n_kv_heads, int causal, int max_split);

// ---- k_head.hip
struct HeadArgs {
  const void* x;      // normalised hidden [n, d]
  const void* E;      // [V, d]: fragment-tiled bf16, or (e_scale != null) E4M3 codes in the FP8 pair-tiled layout
  const float* e_scale;  // FP8 head: [V] row scales, applied to each row's fp32 dot product
  float4* part;       // [n_groups][n] partials (max, argmax or drawn token bits, Z, S1), natural units
  float2* part2;      // gumbel: [n_groups][n] (best perturbed score, scaled logit of the drawn token)
  int n, d, V;
  int n_groups;
  float beta_log2e;   // inv_temperature * log2(e)
  // gumbel: draw token v of row r with the Gumbel noise of Philox counter (v / 4, r + 65536 * step,
  // block, 1) under key (k0, k1) instead of taking the argmax; conf = probability of the draw
  int gumbel;
  uint32_t k0, k1, block, step;
  int32_t* pred;
  float* conf;
  float* ent;
};
template <typename T>
hipError_t launch_vocab_head(const HeadArgs& a, hipStream_t s);
hipError_t launch_head_merge(const HeadArgs& a, hipStream_t s);
int head_groups(int V);

}  // namespace dg
