// dg_api.cpp — host side of libdg: argument validation, workspace carving and the
// sequencing of one denoising pass, prefill/commit and the block loop.
//
// Page tags: [P2] "DiffusionGemma 26B: How Google's Text Diffusion Model Generates
// Tokens in Parallel"; [P3] "DiffusionGemma local text generation" (ctxwire);
// [P5] "When to use a diffusion LLM: I compared DiffusionGemma and Gemma 4".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/dg.h"
#include "dg_kernels.h"

using namespace dg;

namespace {

thread_local int g_hip_error = 0;

#define DG_TRY(expr)                          \
  do {                                        \
    hipError_t e_ = (expr);                   \
    if (e_ != hipSuccess) {                   \
      g_hip_error = (int)e_;                  \
      return DG_ERR_HIP;                      \
    }                                         \
  } while (0)

#define DG_CHECK(expr)               \
  do {                               \
    int r_ = (expr);                 \
    if (r_ != DG_OK) return r_;      \
  } while (0)

// ------------------------------------------------------------------ kernel timing (measurement support)
struct TimerRec {
  int id;
  hipEvent_t a, b;
};
struct Timer {
  uint64_t mask = 0;
  std::vector<TimerRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
thread_local Timer g_timer;

// Records an event pair around one launch when its kernel class is selected.
struct TimeScope {
  int id;
  hipStream_t s;
  hipEvent_t a = nullptr;
  TimeScope(int id_, hipStream_t s_) : id(id_), s(s_) {
    if ((g_timer.mask >> id) & 1ull) {
      a = g_timer.get();
      if (a) (void)hipEventRecord(a, s);
    }
  }
  ~TimeScope() {
    if (!a) return;
    hipEvent_t b = g_timer.get();
    if (!b) return;
    (void)hipEventRecord(b, s);
    g_timer.recs.push_back({id, a, b});
  }
};

// ------------------------------------------------------------------ side stream
// The shared expert depends only on the FFN-normalised rows.  With a caller-owned dg_side it runs on the
// side stream while the caller's stream does the routing and the routed experts, and the two join before
// the combine; without one it runs on the caller's stream.  The library creates and keeps nothing.
struct SideRef {
  hipStream_t s;
  hipEvent_t fork, join;
};
bool side_of(const dg_side* side, SideRef* out) {
  if (!side || !side->stream) return false;
  *out = SideRef{(hipStream_t)side->stream, (hipEvent_t)side->fork, (hipEvent_t)side->join};
  return true;
}
int check_side(const dg_side* side) {
  if (side && side->stream && (!side->fork || !side->join || side->fork == side->join)) return DG_ERR_INVALID;
  return DG_OK;
}

#define DG_LAUNCH(id, s, expr)    \
  do {                            \
    TimeScope ts_((int)(id), (s)); \
    DG_TRY(expr);                 \
  } while (0)

// ------------------------------------------------------------------ fixed scratch (dg_denoise_step_noalloc)
// The workspace of dg_denoise_step_noalloc: a file-scope device array, part of the loaded code object, so that
// the call allocates nothing.  Host code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol): its device address is looked up once per device with hipGetSymbolAddress, with that
// device current, and that address is what the kernels receive.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** out) {
  int dev = 0;
  DG_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return DG_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    DG_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p || ((uintptr_t)p & 255u)) return DG_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DG_OK;
}

constexpr int64_t kPartialRows = 4096;
constexpr int kMaxSeq = 8;  // sequences of one batched call  // attention split partials hold n_split * rows <= max(this, rows)

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline size_t esize(const dg_config* c) { return c->dtype == DG_BF16 ? 2 : 4; }
inline bool aligned16(const void* p) { return p && ((uintptr_t)p & 15u) == 0; }

// ------------------------------------------------------------------ workspace
struct Ws {
  void* X;   // residual stream [M, d]
  void* Xn;  // normalised rows [M, d] (routed-expert gathers, head)
  void* Xt;  // normalised rows, fragment-tiled (dense GEMM A operand)
  void* Q;
  void* O;   // attention output, fragment-tiled
  float* opart;
  float* mlpart;
  float* rlog;
  int32_t* ridx;
  float* rw;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* pos;
  int4* tiles;
  int32_t* n_tiles;
  float* cand_v;
  int32_t* cand_e;
  void* Hp;
  void* Yp;
  void* Hs;
  void* Ys;
  float4* hpart;
  float2* hpart2;
  void* kst;  // staging of a batched call's new keys   [Hkv][M][Dh]
  void* vst;  // staging of a batched call's new values [Hkv][Dh][M]
  dg_block_status* status;
  int32_t* prev_pred;
  int32_t* canvas;
  int32_t* pred;
  float* conf;
  float* ent;
  uint8_t* lock;
  size_t bytes;
  int64_t rows;
};

// Lays out every buffer for calls of up to M rows.  With base == nullptr only sizes.
Ws carve(const dg_config* c, int64_t M, char* base) {
  Ws w{};
  size_t off = 0;
  auto take = [&](size_t n) -> void* {
    void* p = base ? base + off : nullptr;
    off += align256(n);
    return p;
  };
  const size_t es = esize(c);
  const int64_t d = c->d_model, E = c->n_experts, k = c->top_k;
  const int64_t hd = (int64_t)c->n_heads * c->head_dim;
  const int64_t prow = std::max<int64_t>(kPartialRows, M);
  const int64_t pairs = M * k;
  w.rows = M;
  const int64_t Mp = (M + 15) / 16 * 16;  // rows of the fragment-tiled activations
  w.X = take(M * d * es);
  w.Xn = take(M * d * es);
  w.Xt = take(Mp * d * es);
  w.Q = take(M * hd * es);
  w.O = take(Mp * hd * es);
  w.opart = (float*)take(prow * hd * 4);
  w.mlpart = (float*)take(prow * c->n_heads * 2 * 4);
  w.rlog = (float*)take(M * E * 4);
  w.ridx = (int32_t*)take(pairs * 4);
  w.rw = (float*)take(pairs * 4);
  w.counts = (int32_t*)take(E * 4);
  w.offsets = (int32_t*)take((E + 1) * 4);
  w.perm = (int32_t*)take(pairs * 4);
  w.pos = (int32_t*)take(pairs * 4);
  w.tiles = (int4*)take((size_t)moe_max_tiles((int)M, (int)E, (int)k) * 16);
  w.n_tiles = (int32_t*)take(4);
  w.cand_v = (float*)take((size_t)pairs * kRouteSlices * 4);
  w.cand_e = (int32_t*)take((size_t)pairs * kRouteSlices * 4);
  w.Hp = take(pairs * c->ffn_expert * es);
  w.Yp = take(pairs * d * es);
  w.Hs = take(Mp * c->ffn_shared * es);
  w.Ys = take(M * d * es);
  w.hpart = (float4*)take((size_t)head_groups(c->vocab) * M * 16);
  w.hpart2 = (float2*)take((size_t)head_groups(c->vocab) * M * 8);
  w.kst = take((size_t)c->n_kv_heads * M * c->head_dim * es);
  w.vst = take((size_t)c->n_kv_heads * c->head_dim * M * es);
  // per-slot state of up to M / canvas canvases (at least one)
  const int64_t slots = std::max<int64_t>(M, c->canvas);
  w.status = (dg_block_status*)take(sizeof(dg_block_status) * kMaxSeq);
  w.prev_pred = (int32_t*)take(slots * 4);
  w.canvas = (int32_t*)take(slots * 4);
  w.pred = (int32_t*)take(slots * 4);
  w.conf = (float*)take(slots * 4);
  w.ent = (float*)take(slots * 4);
  w.lock = (uint8_t*)take(slots);
  w.bytes = off;
  return w;
}

// ------------------------------------------------------------------ validation
int check_cfg(const dg_config* c) {
  if (!c) return DG_ERR_INVALID;
  if (c->n_layers < 0 || c->d_model <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->n_experts <= 0 || c->top_k <= 0 || c->ffn_expert <= 0 || c->ffn_shared <= 0 || c->vocab <= 0 ||
      c->canvas <= 0)
    return DG_ERR_INVALID;
  if (c->dtype != DG_F32 && c->dtype != DG_BF16) return DG_ERR_INVALID;
  if (!(c->rms_eps >= 0.f)) return DG_ERR_INVALID;
  if (c->top_k > c->n_experts) return DG_ERR_INVALID;
  if (c->n_heads % c->n_kv_heads) return DG_ERR_INVALID;
  if (c->rope_theta != 0.f) return DG_ERR_UNSUPPORTED;
  if (c->d_model % 32 || c->ffn_expert % 32 || c->ffn_shared % 32) return DG_ERR_UNSUPPORTED;
  if (c->d_model > 8192) return DG_ERR_UNSUPPORTED;  // row kernels: one thread per 8 columns, <= 1024 threads
  if (c->head_dim != 64 && c->head_dim != 128) return DG_ERR_UNSUPPORTED;
  const int G = c->n_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4) return DG_ERR_UNSUPPORTED;
  if (c->n_experts > 256 || c->top_k > 16) return DG_ERR_UNSUPPORTED;
  if (c->canvas > 1024 || c->canvas > moe_max_rows(c->n_experts)) return DG_ERR_UNSUPPORTED;
  if (c->expert_dtype != 0 && c->expert_dtype != DG_E4M3 && c->expert_dtype != c->dtype) return DG_ERR_INVALID;
  if (c->expert_dtype == DG_E4M3 && (c->dtype != DG_BF16 || c->d_model % 64 || c->ffn_expert % 64))
    return DG_ERR_UNSUPPORTED;
  if (c->head_dtype != 0 && c->head_dtype != DG_E4M3 && c->head_dtype != c->dtype) return DG_ERR_INVALID;
  if (c->head_dtype == DG_E4M3 && (c->dtype != DG_BF16 || c->d_model % 64)) return DG_ERR_UNSUPPORTED;
  return DG_OK;
}

inline bool fp8_experts(const dg_config* c) { return c->expert_dtype == DG_E4M3; }
inline bool fp8_head(const dg_config* c) { return c->head_dtype == DG_E4M3; }

int check_layer_weights(const dg_config* c, const dg_layer_weights& l) {
  const void* p[] = {l.attn_norm, l.wqkv, l.wo, l.ffn_norm, l.w_router, l.w_gate_up, l.w_down, l.ws_gate_up,
                     l.ws_down};
  for (const void* q : p)
    if (!aligned16(q)) return DG_ERR_INVALID;
  if (fp8_experts(c) && (!aligned16(l.w_gate_up_scale) || !aligned16(l.w_down_scale))) return DG_ERR_INVALID;
  return DG_OK;
}

int check_weights(const dg_config* c, const dg_weights* w, bool need_layers, bool need_head) {
  if (!w) return DG_ERR_INVALID;
  if (!aligned16(w->embed)) return DG_ERR_INVALID;
  if (fp8_head(c) && !aligned16(w->embed_scale)) return DG_ERR_INVALID;
  if (need_head && !aligned16(w->final_norm)) return DG_ERR_INVALID;
  if (need_layers && c->n_layers > 0) {
    if (!w->h_layers) return DG_ERR_INVALID;
    for (int l = 0; l < c->n_layers; ++l) DG_CHECK(check_layer_weights(c, w->h_layers[l]));
  }
  return DG_OK;
}

int check_kv(const dg_kv* kv, int64_t rows) {
  if (!kv || !aligned16(kv->k) || !aligned16(kv->v)) return DG_ERR_INVALID;
  if (kv->capacity <= 0 || kv->capacity % 32 || kv->len < 0) return DG_ERR_INVALID;
  if (kv->len + rows > kv->capacity) return DG_ERR_KV_FULL;
  return DG_OK;
}

int check_ws(const dg_config* c, int64_t rows, void* ws, size_t ws_bytes) {
  if (!ws || ((uintptr_t)ws & 255u)) return DG_ERR_WORKSPACE;
  if (carve(c, rows, nullptr).bytes > ws_bytes) return DG_ERR_WORKSPACE;
  return DG_OK;
}

// Largest row count (<= limit) whose workspace fits in ws_bytes; 0 if none.
int64_t rows_supported(const dg_config* c, size_t ws_bytes, int64_t limit) {
  int64_t lo = 0, hi = limit;
  while (lo < hi) {
    int64_t mid = (lo + hi + 1) / 2;
    if (carve(c, mid, nullptr).bytes <= ws_bytes) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ------------------------------------------------------------------ one transformer block
// What the layer's final combine also produces: nothing, the next layer's attention-normalised rows
// (fragment-tiled, so that layer skips its own RMSNorm), or the final-normalised rows for the head.
enum class Next { None, NextLayer, Head };

// The rows of one layer call, by sequence: segment i holds rows [row0, row0 + rows) of the call, at
// positions pos0.. of its own cache; its first n_causal rows attend causally (a prompt chunk or a
// committed block), the rest to every key [0, pos0 + rows) (a canvas).
struct Seg {
  const dg_kv* kv;
  int64_t pos0, row0, rows, n_causal;
};
struct Segs {
  int n;
  Seg seg[kMaxSeq];
};
Segs one_seq(const dg_kv* kv, int64_t pos0, int64_t M, int64_t n_causal) {
  Segs g{};
  g.n = 1;
  g.seg[0] = Seg{kv, pos0, 0, M, n_causal};
  return g;
}

// One layer over M rows (the segments' rows).
template <typename T>
int layer_t(const dg_config* c, const dg_weights* w, int l, const Segs& sg, int64_t M, bool normed_in, Next next,
            const Ws& ws, const dg_side* side, hipStream_t s) {
  const dg_layer_weights& L = w->h_layers[l];
  const int d = c->d_model, hq = c->n_heads, hkv = c->n_kv_heads, dh = c->head_dim;
  const int E = c->n_experts, k = c->top_k;
  const int Mi = (int)M;
  const size_t es = sizeof(T);
  auto kbase = [&](const dg_kv* kv) { return (char*)kv->k + (size_t)l * hkv * kv->capacity * dh * es; };
  auto vbase = [&](const dg_kv* kv) { return (char*)kv->v + (size_t)l * hkv * dh * kv->capacity * es; };

  // attention half (normed_in: the previous layer's combine already wrote attn_norm(X) to ws.Xt)
  if (!normed_in)
    DG_LAUNCH(DG_K_RMSNORM, s, launch_rmsnorm<T>((const T*)ws.X, (const T*)L.attn_norm, nullptr, (T*)ws.Xt, Mi, d,
                                                  c->rms_eps, s));
  GemmArgs g{};
  g.A = ws.Xt; g.a_tiled = 1; g.B = L.wqkv; g.M = Mi; g.N = (hq + 2 * hkv) * dh; g.K = d; g.lda = d; g.ldb = d;
  g.q = ws.Q; g.n_heads = hq; g.n_kv_heads = hkv; g.head_dim = dh; g.q_rows = Mi;
  if (sg.n == 1) {  // keys and values go straight into the cache
    g.kc = kbase(sg.seg[0].kv); g.vc = vbase(sg.seg[0].kv); g.cap = sg.seg[0].kv->capacity; g.pos0 = sg.seg[0].pos0;
  } else {          // several caches: staged, then copied into each sequence's cache
    g.kc = ws.kst; g.vc = ws.vst; g.cap = M; g.pos0 = 0;
  }
  DG_LAUNCH(DG_K_GEMM_QKV, s, launch_gemm<T>(GemmEpi::QKV, g, s));
  if (sg.n > 1) {
    for (int i = 0; i < sg.n; ++i) {
      const Seg& q = sg.seg[i];
      KvScatterArgs ka{ws.kst, ws.vst, Mi, hkv, dh, kbase(q.kv), vbase(q.kv), q.kv->capacity, q.pos0, (int)q.row0,
                       (int)q.rows};
      DG_LAUNCH(DG_K_KV_SCATTER, s, launch_kv_scatter<T>(ka, s));
    }
  }

  // attention: one launch (and merge) per row range of one sequence and one mask
  auto attend = [&](const Seg& q, int64_t off, int64_t rows, bool causal) -> int {
    AttnArgs at{};
    at.q = ws.Q; at.kc = kbase(q.kv); at.vc = vbase(q.kv); at.o_part = ws.opart; at.ml_part = ws.mlpart;
    at.o = ws.O; at.q_rows = (int)rows; at.q_stride = Mi; at.row0 = (int)(q.row0 + off); at.n_heads = hq;
    at.n_kv_heads = hkv; at.head_dim = dh; at.cap = q.kv->capacity;
    at.n_keys = causal ? q.pos0 + off + rows : q.pos0 + q.rows;
    at.q_pos0 = q.pos0 + off; at.causal = causal ? 1 : 0;
    const int max_split =
        (int)std::min<int64_t>(kAttnMaxSplit, std::max<int64_t>(1, std::max(kPartialRows, M) / rows));
    at.n_split = attention_splits(at.n_keys, (int)rows, hq, hkv, at.causal, max_split);
    DG_LAUNCH(DG_K_ATTENTION, s, launch_attention<T>(at, s));
    DG_LAUNCH(DG_K_ATTN_MERGE, s, launch_attention_merge<T>(at, s));
    return DG_OK;
  };
  for (int i = 0; i < sg.n; ++i) {
    const Seg& q = sg.seg[i];
    if (q.n_causal > 0) DG_CHECK(attend(q, 0, q.n_causal, true));
    if (q.n_causal < q.rows) DG_CHECK(attend(q, q.n_causal, q.rows - q.n_causal, false));
  }

  g = GemmArgs{};
  g.A = ws.O; g.a_tiled = 1; g.B = L.wo; g.C = ws.X; g.M = Mi; g.N = d; g.K = hq * dh; g.lda = hq * dh; g.ldb = hq * dh; g.ldc = d;
  DG_LAUNCH(DG_K_GEMM_O, s, launch_gemm<T>(GemmEpi::Resid, g, s));

  // MoE half ([P2] "Architecture Details": 8 routed experts of 128, plus 1 shared)
  // shared expert: on the caller's side stream when there is one, concurrent with the routing and the routed
  // experts (the fork and join events complete with the norm and the shared down projection themselves);
  // otherwise on the caller's stream
  SideRef sd{};
  const bool fork = side_of(side, &sd);
  const hipStream_t ss = fork ? sd.s : s;
  DG_LAUNCH(DG_K_RMSNORM, s, launch_rmsnorm<T>((const T*)ws.X, (const T*)L.ffn_norm, (T*)ws.Xn, (T*)ws.Xt, Mi, d,
                                                c->rms_eps, s, fork ? sd.fork : nullptr));
  if (fork) DG_TRY(hipStreamWaitEvent(ss, sd.fork, 0));
  g = GemmArgs{};
  g.A = ws.Xt; g.a_tiled = 1; g.B = L.ws_gate_up; g.C = ws.Hs; g.M = Mi; g.N = c->ffn_shared; g.K = d; g.lda = d;
  g.ldb = d; g.ldc = c->ffn_shared;
  DG_LAUNCH(DG_K_SHARED_GATE_UP, ss, launch_gemm<T>(GemmEpi::SwiGLU, g, ss));
  g = GemmArgs{};
  g.A = ws.Hs; g.a_tiled = 1; g.B = L.ws_down; g.C = ws.Ys; g.M = Mi; g.N = d; g.K = c->ffn_shared;
  g.lda = c->ffn_shared; g.ldb = c->ffn_shared; g.ldc = d;
  DG_LAUNCH(DG_K_SHARED_DOWN, ss, launch_gemm<T>(GemmEpi::Store, g, ss, fork ? sd.join : nullptr));

  // router logits, top-k, softmax weights and the token->expert order
  RouteArgs ra{};
  ra.Xt = ws.Xt; ra.Wr = L.w_router; ra.logits = ws.rlog; ra.cand_v = ws.cand_v; ra.cand_e = ws.cand_e;
  ra.idx = ws.ridx; ra.w = ws.rw; ra.counts = ws.counts; ra.offsets = ws.offsets; ra.perm = ws.perm;
  ra.pos = ws.pos; ra.tiles = ws.tiles; ra.n_tiles = ws.n_tiles; ra.M = Mi; ra.d = d; ra.E = E; ra.k = k;
  ra.tile_rows = moe_tile_rows(Mi, E, k);
  DG_LAUNCH(DG_K_ROUTE, s, launch_route<T>(ra, s));

  MoeArgs ma{};
  ma.tiles = ws.tiles; ma.n_tiles = ws.n_tiles; ma.max_tiles = moe_max_tiles(Mi, E, k); ma.perm = ws.perm;
  ma.tile_rows = ra.tile_rows;
  ma.X = ws.Xn; ma.W = L.w_gate_up; ma.out = ws.Hp; ma.d = d; ma.F = c->ffn_expert; ma.scale = L.w_gate_up_scale;
  if (fp8_experts(c))
    DG_LAUNCH(DG_K_MOE_GATE_UP, s, launch_moe_gate_up_f8(ma, s));
  else
    DG_LAUNCH(DG_K_MOE_GATE_UP, s, launch_moe_gate_up<T>(ma, s));
  ma.X = ws.Hp; ma.W = L.w_down; ma.out = ws.Yp; ma.scale = L.w_down_scale;
  if (fp8_experts(c))
    DG_LAUNCH(DG_K_MOE_DOWN, s, launch_moe_down_f8(ma, s));
  else
    DG_LAUNCH(DG_K_MOE_DOWN, s, launch_moe_down<T>(ma, s));

  if (fork) DG_TRY(hipStreamWaitEvent(s, sd.join, 0));  // join: the combine reads the shared expert's output
  const T* g_next = next == Next::NextLayer ? (const T*)w->h_layers[l + 1].attn_norm
                    : next == Next::Head      ? (const T*)w->final_norm
                                              : nullptr;
  T* y_next = next == Next::NextLayer ? (T*)ws.Xt : (T*)ws.Xn;
  DG_LAUNCH(DG_K_MOE_COMBINE, s,
            launch_moe_combine<T>((T*)ws.X, (const T*)ws.Ys, (const T*)ws.Yp, ws.pos, ws.rw, Mi, d, k, g_next, y_next,
                                  next == Next::NextLayer ? 1 : 0, c->rms_eps, s));
  return DG_OK;
}

int layer(const dg_config* c, const dg_weights* w, int l, const Segs& sg, int64_t M, bool normed_in, Next next,
          const Ws& ws, const dg_side* side, hipStream_t s) {
  if (c->dtype == DG_BF16) return layer_t<bf16>(c, w, l, sg, M, normed_in, next, ws, side, s);
  return layer_t<float>(c, w, l, sg, M, normed_in, next, ws, side, s);
}
int layer(const dg_config* c, const dg_weights* w, int l, const dg_kv* kv, int64_t pos0, int64_t M, int64_t n_causal,
          bool normed_in, Next next, const Ws& ws, const dg_side* side, hipStream_t s) {
  return layer(c, w, l, one_seq(kv, pos0, M, n_causal), M, normed_in, next, ws, side, s);
}

// rows [row0, row0 + M) of ws.X = embeddings of tok[0, M)
int embed(const dg_config* c, const dg_weights* w, const int32_t* tok, int64_t M, const Ws& ws, hipStream_t s,
          int64_t row0 = 0) {
  const int64_t off = row0 * c->d_model;
  if (fp8_head(c))
    DG_LAUNCH(DG_K_EMBED, s, launch_embed_f8(tok, (const uint8_t*)w->embed, w->embed_scale, (bf16*)ws.X + off, (int)M,
                                              c->d_model, c->vocab, s));
  else if (c->dtype == DG_BF16)
    DG_LAUNCH(DG_K_EMBED, s, launch_embed<bf16>(tok, (const bf16*)w->embed, (bf16*)ws.X + off, (int)M, c->d_model,
                                                 c->vocab, s));
  else
    DG_LAUNCH(DG_K_EMBED, s, launch_embed<float>(tok, (const float*)w->embed, (float*)ws.X + off, (int)M, c->d_model,
                                                  c->vocab, s));
  return DG_OK;
}

// temperature and token choice of one pass: the argmax, or (gumbel) a draw from the tempered softmax
// keyed by (seed, block, step)
struct PassParams {
  float inv_temp;
  bool gumbel;
  uint64_t seed;
  uint32_t block, step;
};
PassParams argmax_pass(float inv_temp) { return PassParams{inv_temp, false, 0, 0, 0}; }

// 1 / T of pass `step`: the sampler's constant, or (anneal) T linear from temperature_first at pass 1 to
// temperature_last at the last pass of the budget
float pass_inv_temperature(const dg_sampler* sp, int step) {
  if (!(sp->flags & DG_SAMPLE_ANNEAL)) return sp->inv_temperature;
  const int n = sp->fixed_steps > 0 ? sp->fixed_steps : sp->max_steps;
  const double frac = n <= 1 ? 0.0 : std::min(1.0, (double)(step - 1) / (double)(n - 1));
  const double t = (double)sp->temperature_first + ((double)sp->temperature_last - sp->temperature_first) * frac;
  return (float)(1.0 / t);
}
PassParams sampler_pass(const dg_sampler* sp, uint32_t block, int step) {
  return PassParams{pass_inv_temperature(sp, step), (sp->flags & DG_SAMPLE_GUMBEL) != 0, sp->seed, block,
                    (uint32_t)step};
}

// final norm (unless normed: ws.Xn already holds it) + fused head over rows [row0, row0 + M) of ws.X
int head(const dg_config* c, const dg_weights* w, int64_t M, const PassParams& pp, int32_t* pred, float* conf,
         float* ent, bool normed, const Ws& ws, hipStream_t s, int64_t row0 = 0) {
  HeadArgs h{};
  h.x = (const char*)ws.Xn + row0 * c->d_model * esize(c); h.E = w->embed; h.part = ws.hpart; h.n = (int)M; h.d = c->d_model; h.V = c->vocab;
  h.n_groups = head_groups(c->vocab); h.beta_log2e = pp.inv_temp * 1.4426950408889634f;
  h.part2 = ws.hpart2; h.gumbel = pp.gumbel ? 1 : 0;
  h.k0 = (uint32_t)pp.seed; h.k1 = (uint32_t)(pp.seed >> 32); h.block = pp.block; h.step = pp.step;
  h.pred = pred; h.conf = conf; h.ent = ent;
  h.e_scale = fp8_head(c) ? w->embed_scale : nullptr;
  if (c->dtype == DG_BF16) {
    if (!normed)
      DG_LAUNCH(DG_K_RMSNORM, s, launch_rmsnorm<bf16>((const bf16*)ws.X + row0 * c->d_model, (const bf16*)w->final_norm,
                                                       (bf16*)ws.Xn + row0 * c->d_model, nullptr, (int)M, c->d_model,
                                                       c->rms_eps, s));
    DG_LAUNCH(DG_K_VOCAB_HEAD, s, launch_vocab_head<bf16>(h, s));
  } else {
    if (!normed)
      DG_LAUNCH(DG_K_RMSNORM, s, launch_rmsnorm<float>((const float*)ws.X + row0 * c->d_model,
                                                        (const float*)w->final_norm, (float*)ws.Xn + row0 * c->d_model,
                                                        nullptr, (int)M, c->d_model, c->rms_eps, s));
    DG_LAUNCH(DG_K_VOCAB_HEAD, s, launch_vocab_head<float>(h, s));
  }
  DG_LAUNCH(DG_K_HEAD_MERGE, s, launch_head_merge(h, s));
  return DG_OK;
}

// denoising pass with an already-validated configuration
int denoise(const dg_config* c, const dg_weights* w, const dg_kv* kv, const int32_t* canvas, const PassParams& pp,
            int32_t* pred, float* conf, float* ent, const dg_debug* dbg, const Ws& ws, const dg_side* side,
            hipStream_t s) {
  const int64_t S = c->canvas;
  DG_CHECK(embed(c, w, canvas, S, ws, s));
  const int L = c->n_layers;
  for (int l = 0; l < L; ++l) {
    DG_CHECK(layer(c, w, l, kv, kv->len, S, 0, l > 0, l + 1 < L ? Next::NextLayer : Next::Head, ws, side, s));
    if (dbg) {
      const size_t hb = (size_t)S * c->d_model * esize(c);
      if (dbg->hidden) DG_TRY(hipMemcpyAsync((char*)dbg->hidden + l * hb, ws.X, hb, hipMemcpyDeviceToDevice, s));
      const size_t rb = (size_t)S * c->top_k * 4;
      if (dbg->route_idx)
        DG_TRY(hipMemcpyAsync((char*)dbg->route_idx + l * rb, ws.ridx, rb, hipMemcpyDeviceToDevice, s));
      if (dbg->route_w) DG_TRY(hipMemcpyAsync((char*)dbg->route_w + l * rb, ws.rw, rb, hipMemcpyDeviceToDevice, s));
      const size_t lb = (size_t)S * c->n_experts * 4;
      if (dbg->router_logits)
        DG_TRY(hipMemcpyAsync((char*)dbg->router_logits + l * lb, ws.rlog, lb, hipMemcpyDeviceToDevice, s));
    }
  }
  return head(c, w, S, pp, pred, conf, ent, L > 0, ws, s);
}

// A pass that also commits the previous block: rows [0, S) are that block's tokens at cache rows
// len.. (causal: they become its committed keys and values), rows [S, 2S) are the canvas (scratch rows
// len + S..).  Every weight is streamed once for both; the head runs on the canvas rows only.  The
// caller advances kv->len by S afterwards.
int denoise_committing(const dg_config* c, const dg_weights* w, const dg_kv* kv, const int32_t* block_tokens,
                       const int32_t* canvas, const PassParams& pp, int32_t* pred, float* conf, float* ent, const Ws& ws,
                       const dg_side* side, hipStream_t s) {
  const int64_t S = c->canvas;
  DG_CHECK(embed(c, w, block_tokens, S, ws, s, 0));
  DG_CHECK(embed(c, w, canvas, S, ws, s, S));
  const int L = c->n_layers;
  for (int l = 0; l < L; ++l)
    DG_CHECK(layer(c, w, l, kv, kv->len, 2 * S, S, l > 0, l + 1 < L ? Next::NextLayer : Next::Head, ws, side, s));
  return head(c, w, S, pp, pred, conf, ent, L > 0, ws, s, S);
}

// causal forward of n tokens at kv->len.., chunked to the workspace; does not change kv->len
int prefill(const dg_config* c, const dg_weights* w, const dg_kv* kv, const int32_t* tokens, int64_t n, void* wsp,
            size_t ws_bytes, const dg_side* side, hipStream_t s) {
  const int64_t chunk = rows_supported(c, ws_bytes, moe_max_rows(c->n_experts));
  if (chunk < 1) return DG_ERR_WORKSPACE;
  for (int64_t r0 = 0; r0 < n; r0 += chunk) {
    const int64_t m = std::min(chunk, n - r0);
    Ws ws = carve(c, m, (char*)wsp);
    DG_CHECK(embed(c, w, tokens + r0, m, ws, s));
    const int L = c->n_layers;
    for (int l = 0; l < L; ++l)
      DG_CHECK(layer(c, w, l, kv, kv->len + r0, m, m, l > 0, l + 1 < L ? Next::NextLayer : Next::None, ws, side, s));
  }
  return DG_OK;
}

StopParams stop_params(const dg_config* c, const dg_sampler* sp) {
  StopParams p;
  p.threshold = sp->entropy_threshold;
  p.ln_vocab = logf((float)c->vocab);
  p.max_steps = sp->max_steps;
  p.fixed_steps = sp->fixed_steps;
  p.and_rule = (sp->flags & DG_STOP_AND) ? 1 : 0;
  return p;
}

int check_sampler(const dg_config* c, const dg_sampler* sp) {
  if (!sp) return DG_ERR_INVALID;
  if (sp->n_new < 0 || sp->max_steps < 1 || sp->fixed_steps < 0 || (sp->flags & ~DG_SAMPLER_FLAGS)) return DG_ERR_INVALID;
  if (std::isnan(sp->entropy_threshold)) return DG_ERR_INVALID;
  if (sp->flags & DG_SAMPLE_ANNEAL) {
    if (!(sp->temperature_first > 0.f) || !(sp->temperature_last > 0.f) || std::isinf(sp->temperature_first) ||
        std::isinf(sp->temperature_last))
      return DG_ERR_INVALID;
  } else if (!(sp->inv_temperature > 0.f)) {
    return DG_ERR_INVALID;
  }
  // the draw's Philox counter holds the slot and the pass in 16 bits each
  if ((sp->flags & DG_SAMPLE_GUMBEL) && (sp->max_steps > 65535 || sp->fixed_steps > 65535)) return DG_ERR_INVALID;
  (void)c;
  return DG_OK;
}

// One block's passes (initial canvas, passes t = 1.. with the stop check and, if not stopping, the canvas update)
// with an already-validated configuration; `pending` (nullable) is committed inside the first pass (kv->len grows
// by S).  The block's tokens (the last pass's predictions) are left in wsv.pred; *st receives the status (read from
// the device here, so it is valid when the stream reaches this point).
int block_loop(const dg_config* cfg, const dg_weights* w, dg_kv* kv, const dg_sampler* sp, uint32_t block,
               const int32_t* pending, const Ws& wsv, const dg_side* side, hipStream_t s, dg_block_status* st) {
  const int S = cfg->canvas;
  const StopParams stp = stop_params(cfg, sp);
  const bool fixed = sp->fixed_steps > 0;
  const int limit = fixed ? sp->fixed_steps : sp->max_steps;
  const bool lock = (sp->flags & DG_KEEP_LOCK) != 0;
  uint8_t* lock_mask = lock ? wsv.lock : nullptr;  // the locked slots; cleared by the initial draw
  CanvasArgs ca{nullptr, nullptr, nullptr, 0, nullptr, S, 0, sp->seed, block, 0, (uint32_t)cfg->vocab, wsv.canvas,
                lock_mask};
  DG_LAUNCH(DG_K_CANVAS_UPDATE, s, launch_canvas_update(ca, s));
  for (int t = 1;; ++t) {
    const PassParams pp = sampler_pass(sp, block, t);
    if (t == 1 && pending) {
      DG_CHECK(denoise_committing(cfg, w, kv, pending, wsv.canvas, pp, wsv.pred, wsv.conf, wsv.ent, wsv, side, s));
      kv->len += S;  // the pending block is committed (in stream order) before every later pass
    } else {
      DG_CHECK(denoise(cfg, w, kv, wsv.canvas, pp, wsv.pred, wsv.conf, wsv.ent, nullptr, wsv, side, s));
    }
    DG_LAUNCH(DG_K_STOP_CHECK, s,
              launch_stop_check(wsv.ent, wsv.pred, wsv.prev_pred, wsv.canvas, lock_mask, S, t, stp, wsv.status, s));
    bool stop;
    if (fixed) {
      stop = t >= limit;
    } else {
      DG_TRY(hipMemcpyAsync(st, wsv.status, sizeof(*st), hipMemcpyDeviceToHost, s));
      DG_TRY(hipStreamSynchronize(s));
      stop = st->reason != DG_STOP_NONE;
    }
    if (stop) break;
    ca = CanvasArgs{wsv.pred, wsv.conf, wsv.ent, (sp->flags & DG_KEEP_ENTROPY) ? 1 : 0, lock_mask, S,
                    (int)std::min<int64_t>(S, (int64_t)t * sp->n_new), sp->seed, block, (uint32_t)t,
                    (uint32_t)cfg->vocab, wsv.canvas, lock_mask};
    DG_LAUNCH(DG_K_CANVAS_UPDATE, s, launch_canvas_update(ca, s));
  }
  if (fixed) DG_TRY(hipMemcpyAsync(st, wsv.status, sizeof(*st), hipMemcpyDeviceToHost, s));
  return DG_OK;
}

// Greedy verify of a drafted block (validated configuration, workspace of S rows): the commit's causal forward
// over draft at kv->len.., the argmax of every row into ar_pred, then the accepted prefix (draft[0] as drafted,
// draft[i] while ar_pred[i - 1] == draft[i]); kv->len grows by it.  Synchronises the stream.
int verify_rows(const dg_config* cfg, const dg_weights* w, dg_kv* kv, const int32_t* draft, int32_t* ar_pred,
                const Ws& wsv, const dg_side* side, hipStream_t s, int32_t* accepted, int32_t* next_token) {
  const int S = cfg->canvas;
  DG_CHECK(embed(cfg, w, draft, S, wsv, s));
  const int L = cfg->n_layers;
  for (int l = 0; l < L; ++l)
    DG_CHECK(layer(cfg, w, l, kv, kv->len, S, S, l > 0, l + 1 < L ? Next::NextLayer : Next::Head, wsv, side, s));
  DG_CHECK(head(cfg, w, S, argmax_pass(1.0f), ar_pred, wsv.conf, wsv.ent, L > 0, wsv, s));
  std::vector<int32_t> hp(S), hd(S);
  DG_TRY(hipMemcpyAsync(hp.data(), ar_pred, (size_t)S * 4, hipMemcpyDeviceToHost, s));
  DG_TRY(hipMemcpyAsync(hd.data(), draft, (size_t)S * 4, hipMemcpyDeviceToHost, s));
  DG_TRY(hipStreamSynchronize(s));
  int n = 1;
  while (n < S && hp[n - 1] == hd[n]) ++n;
  *accepted = n;
  *next_token = hp[n - 1];
  kv->len += n;
  return DG_OK;
}

}  // namespace

// ====================================================================== C ABI
extern "C" {

int dg_workspace_size(const dg_config* cfg, int64_t max_tokens, size_t* h_bytes) {
  DG_CHECK(check_cfg(cfg));
  if (!h_bytes || max_tokens < 1 || max_tokens > moe_max_rows(cfg->n_experts)) return DG_ERR_INVALID;
  *h_bytes = carve(cfg, std::max<int64_t>(max_tokens, 1), nullptr).bytes;
  return DG_OK;
}

int dg_prefill_kv(const dg_config* cfg, const dg_weights* w, dg_kv* kv, const int32_t* tokens, int64_t n, void* ws,
                  size_t ws_bytes, const dg_side* side, void* stream) {
  DG_CHECK(check_cfg(cfg));
  DG_CHECK(check_side(side));
  DG_CHECK(check_weights(cfg, w, true, false));
  if (n < 0 || (n > 0 && !tokens)) return DG_ERR_INVALID;
  DG_CHECK(check_kv(kv, n));
  if (n == 0) return DG_OK;
  if (!ws || ((uintptr_t)ws & 255u) || rows_supported(cfg, ws_bytes, 1) < 1) return DG_ERR_WORKSPACE;
  DG_CHECK(prefill(cfg, w, kv, tokens, n, ws, ws_bytes, side, (hipStream_t)stream));
  kv->len += n;
  return DG_OK;
}

int dg_denoise_step(const dg_config* cfg, const dg_weights* w, const dg_kv* kv, const int32_t* canvas,
                    float inv_temperature, int32_t* pred, float* conf, float* entropy, const dg_debug* dbg, void* ws,
                    size_t ws_bytes, const dg_side* side, void* stream) {
  DG_CHECK(check_cfg(cfg));
  DG_CHECK(check_side(side));
  DG_CHECK(check_weights(cfg, w, true, true));
  if (!canvas || !pred || !conf || !entropy) return DG_ERR_INVALID;
  if (!(inv_temperature > 0.f)) return DG_ERR_INVALID;
  DG_CHECK(check_kv(kv, cfg->canvas));
  DG_CHECK(check_ws(cfg, cfg->canvas, ws, ws_bytes));
  Ws wsv = carve(cfg, cfg->canvas, (char*)ws);
  return denoise(cfg, w, kv, canvas, argmax_pass(inv_temperature), pred, conf, entropy, dbg, wsv, side,
                 (hipStream_t)stream);
}

int dg_denoise_step_noalloc(const dg_config* cfg, const dg_weights* w, const dg_kv* kv, const int32_t* canvas,
                            float inv_temperature, int32_t* pred, float* conf, float* entropy, const dg_side* side,
                            void* stream) {
  DG_CHECK(check_cfg(cfg));
  DG_CHECK(check_side(side));
  DG_CHECK(check_weights(cfg, w, true, true));
  if (!canvas || !pred || !conf || !entropy) return DG_ERR_INVALID;
  if (!(inv_temperature > 0.f)) return DG_ERR_INVALID;
  DG_CHECK(check_kv(kv, cfg->canvas));
  if (carve(cfg, cfg->canvas, nullptr).bytes > kScratchBytes) return DG_ERR_WORKSPACE;
  void* base = nullptr;
  DG_CHECK(scratch_of_current_device(&base));
  Ws wsv = carve(cfg, cfg->canvas, (char*)base);
  return denoise(cfg, w, kv, canvas, argmax_pass(inv_temperature), pred, conf, entropy, nullptr, wsv, side,
                 (hipStream_t)stream);
}

int dg_noalloc_scratch_bytes(size_t* h_bytes) {
  if (!h_bytes) return DG_ERR_INVALID;
  *h_bytes = kScratchBytes;
  return DG_OK;
}

int dg_denoise_step_sampler(const dg_config* cfg, const dg_weights* w, const dg_kv* kv, const dg_sampler* sampler,
                            uint32_t block, int32_t step, const int32_t* canvas, int32_t* pred, float* conf,
                            float* entropy, void* ws, size_t ws_bytes, const dg_side* side, void* stream) {
  DG_CHECK(check_cfg(cfg));
  DG_CHECK(check_side(side));
  DG_CHECK(check_weights(cfg, w, true, true));
  DG_CHECK(check_sampler(cfg, sampler));
  if (!canvas || !pred || !conf || !entropy || step < 1 || step > 65535) return DG_ERR_INVALID;
  DG_CHECK(check_kv(kv, cfg->canvas));
  DG_CHECK(check_ws(cfg, cfg->canvas, ws, ws_bytes));
  Ws wsv = carve(cfg, cfg->canvas, (char*)ws);
  return denoise(cfg, w, kv, canvas, sampler_pass(sampler, block, step), pred, conf, entropy, nullptr, wsv, side,
                 (hipStream_t)stream);
}

int dg_canvas_update(const dg_config* cfg, const int32_t* pred, const float* conf, int32_t keep_count, uint64_t seed,
                     uint32_t block, uint32_t step, int32_t* canvas_out, uint8_t* keep_mask, void* stream) {
  DG_CHECK(check_cfg(cfg));
  if (!canvas_out || keep_count < 0 || keep_count > cfg->canvas) return DG_ERR_INVALID;
  if (keep_count > 0 && (!pred || !conf)) return DG_ERR_INVALID;
  CanvasArgs ca{pred, conf, nullptr, 0, nullptr, cfg->canvas, keep_count, seed, block, step, (uint32_t)cfg->vocab,
                canvas_out, keep_mask};
  DG_LAUNCH(DG_K_CANVAS_UPDATE, (hipStream_t)stream, launch_canvas_update(ca, (hipStream_t)stream));
  return DG_OK;
}

int dg_canvas_update_sampler(const dg_config* cfg, const dg_sampler* sampler, uint32_t block, int32_t step,
                             const int32_t* pred, const float* conf, const float* entropy, int32_t* canvas,
                             uint8_t* lock_mask, void* stream) {
  DG_CHECK(check_cfg(cfg));
  DG_CHECK(check_sampler(cfg, sampler));
  if (step < 0 || !canvas) return DG_ERR_INVALID;
  const int keep = (int)std::min<int64_t>(cfg->canvas, (int64_t)step * sampler->n_new);
  const bool lock = (sampler->flags & DG_KEEP_LOCK) != 0, by_ent = (sampler->flags & DG_KEEP_ENTROPY) != 0;
  if (keep > 0 && (!pred || (by_ent ? !entropy : !conf))) return DG_ERR_INVALID;
  if (lock && !lock_mask) return DG_ERR_INVALID;
  CanvasArgs ca{pred, conf, entropy, by_ent ? 1 : 0, (lock && step > 0) ? lock_mask : nullptr, cfg->canvas, keep,
                sampler->seed, block, (uint32_t)step, (uint32_t)cfg->vocab, canvas, lock_mask};
  DG_LAUNCH(DG_K_CANVAS_UPDATE, (hipStream_t)stream, launch_canvas_update(ca, (hipStream_t)stream));
  return DG_OK;
}

int dg_commit_block(const dg_config* cfg, const dg_weights* w, dg_kv* kv, const int32_t* block_tokens, void* ws,
                    size_t ws_bytes, const dg_side* side, void* stream) {
  return dg_prefill_kv(cfg, w, kv, block_tokens, cfg ? cfg->canvas : 0, ws, ws_bytes, side, stream);
}

int dg_generate_block_overlapped(const dg_config* cfg, const dg_weights* w, dg_kv* kv, const dg_sampler* sp,
                                 uint32_t block, const int32_t* pending, int32_t defer_commit, int32_t* tokens_out,
                                 dg_block_status* h_status, void* ws, size_t ws_bytes, const dg_side* side, void* stream) {
  DG_CHECK(check_cfg(cfg));
  DG_CHECK(check_side(side));
  DG_CHECK(check_weights(cfg, w, true, true));
  DG_CHECK(check_sampler(cfg, sp));
  if (!tokens_out || !h_status || (defer_commit != 0 && defer_commit != 1)) return DG_ERR_INVALID;
  const int S = cfg->canvas;
  const int64_t rows = pending ? 2 * (int64_t)S : S;  // the first pass also commits `pending`
  if (rows > moe_max_rows(cfg->n_experts)) return DG_ERR_INVALID;  // rows one routing step orders
  DG_CHECK(check_kv(kv, rows));
  DG_CHECK(check_ws(cfg, rows, ws, ws_bytes));
  hipStream_t s = (hipStream_t)stream;
  Ws wsv = carve(cfg, rows, (char*)ws);
  dg_block_status st{};
  DG_CHECK(block_loop(cfg, w, kv, sp, block, pending, wsv, side, s, &st));
  DG_TRY(hipMemcpyAsync(tokens_out, wsv.pred, (size_t)S * 4, hipMemcpyDeviceToDevice, s));
  if (!defer_commit) {
    DG_CHECK(prefill(cfg, w, kv, tokens_out, S, ws, ws_bytes, side, s));
    kv->len += S;
  }
  DG_TRY(hipStreamSynchronize(s));
  *h_status = st;
  return DG_OK;
}

int dg_generate_block(const dg_config* cfg, const dg_weights* w, dg_kv* kv, const dg_sampler* sp, uint32_t block,
                      int32_t* tokens_out, dg_block_status* h_status, void* ws, size_t ws_bytes, const dg_side* side, void* stream) {
  return dg_generate_block_overlapped(cfg, w, kv, sp, block, nullptr, 0, tokens_out, h_status, ws, ws_bytes, side,
                                      stream);
}

int dg_generate_blocks_overlapped(const dg_config* cfg, const dg_weights* w, dg_kv* kvs, int32_t n_seq,
                                  const dg_sampler* sp, const uint32_t* h_blocks, const int32_t* pending,
                                  int32_t defer_commit, int32_t* tokens_out, dg_block_status* h_status, void* ws,
                                  size_t ws_bytes, const dg_side* side, void* stream) {
  DG_CHECK(check_cfg(cfg));
  DG_CHECK(check_side(side));
  DG_CHECK(check_weights(cfg, w, true, true));
  DG_CHECK(check_sampler(cfg, sp));
  if (!kvs || !h_blocks || !tokens_out || !h_status || n_seq < 1 || n_seq > kMaxSeq) return DG_ERR_INVALID;
  if (defer_commit != 0 && defer_commit != 1) return DG_ERR_INVALID;
  const int S = cfg->canvas;
  const int64_t M = (int64_t)n_seq * S;
  const int64_t rows = pending ? 2 * M : M;  // the first pass also commits the pending blocks
  if (rows > moe_max_rows(cfg->n_experts)) return DG_ERR_INVALID;
  for (int b = 0; b < n_seq; ++b) {
    DG_CHECK(check_kv(&kvs[b], pending ? 2 * S : S));
    for (int b2 = 0; b2 < b; ++b2)
      if (kvs[b2].k == kvs[b].k || kvs[b2].v == kvs[b].v) return DG_ERR_INVALID;  // each sequence its own cache
  }
  DG_CHECK(check_ws(cfg, rows, ws, ws_bytes));
  hipStream_t s = (hipStream_t)stream;
  Ws wsv = carve(cfg, rows, (char*)ws);
  const StopParams stp = stop_params(cfg, sp);
  const bool fixed = sp->fixed_steps > 0, lock = (sp->flags & DG_KEEP_LOCK) != 0;
  const bool by_ent = (sp->flags & DG_KEEP_ENTROPY) != 0, draw = (sp->flags & DG_SAMPLE_GUMBEL) != 0;
  const int L = cfg->n_layers;
  const uint32_t V = (uint32_t)cfg->vocab;
  Segs sg{};
  sg.n = n_seq;
  for (int b = 0; b < n_seq; ++b) sg.seg[b] = Seg{&kvs[b], kvs[b].len, (int64_t)b * S, S, 0};
  auto lock_of = [&](int b) { return lock ? wsv.lock + (size_t)b * S : nullptr; };

  for (int b = 0; b < n_seq; ++b) {
    CanvasArgs ca{nullptr, nullptr, nullptr, 0, nullptr, S, 0, sp->seed, h_blocks[b], 0, V, wsv.canvas + (size_t)b * S,
                  lock_of(b)};
    DG_LAUNCH(DG_K_CANVAS_UPDATE, s, launch_canvas_update(ca, s));
  }
  bool done[kMaxSeq] = {};
  int n_done = 0;
  dg_block_status st[kMaxSeq] = {};
  for (int t = 1; n_done < n_seq; ++t) {
    if (t == 1 && pending) {
      // sequence b's rows [2bS, 2bS + S) are its pending block (causal, committed at its cache's end), rows
      // [2bS + S, 2(b+1)S) its canvas, which sees the committed block
      Segs pg{};
      pg.n = n_seq;
      for (int b = 0; b < n_seq; ++b) {
        pg.seg[b] = Seg{&kvs[b], kvs[b].len, 2 * (int64_t)b * S, 2 * (int64_t)S, S};
        DG_CHECK(embed(cfg, w, pending + (size_t)b * S, S, wsv, s, 2 * (int64_t)b * S));
        DG_CHECK(embed(cfg, w, wsv.canvas + (size_t)b * S, S, wsv, s, (2 * (int64_t)b + 1) * S));
      }
      for (int l = 0; l < L; ++l)
        DG_CHECK(layer(cfg, w, l, pg, rows, l > 0, l + 1 < L ? Next::NextLayer : Next::Head, wsv, side, s));
      for (int b = 0; b < n_seq; ++b)
        DG_CHECK(head(cfg, w, S, sampler_pass(sp, h_blocks[b], t), wsv.pred + (size_t)b * S, wsv.conf + (size_t)b * S,
                      wsv.ent + (size_t)b * S, L > 0, wsv, s, (2 * (int64_t)b + 1) * S));
      for (int b = 0; b < n_seq; ++b) {  // committed (in stream order) before every later pass
        kvs[b].len += S;
        sg.seg[b].pos0 = kvs[b].len;
      }
    } else {
      // one pass over every canvas; a finished canvas still runs (its rows are ignored from then on)
      DG_CHECK(embed(cfg, w, wsv.canvas, M, wsv, s));
      for (int l = 0; l < L; ++l)
        DG_CHECK(layer(cfg, w, l, sg, M, l > 0, l + 1 < L ? Next::NextLayer : Next::Head, wsv, side, s));
      if (!draw) {
        DG_CHECK(head(cfg, w, M, sampler_pass(sp, 0, t), wsv.pred, wsv.conf, wsv.ent, L > 0, wsv, s));
      } else {  // each canvas draws with its own block's counters
        for (int b = 0; b < n_seq; ++b)
          if (!done[b])
            DG_CHECK(head(cfg, w, S, sampler_pass(sp, h_blocks[b], t), wsv.pred + (size_t)b * S,
                          wsv.conf + (size_t)b * S, wsv.ent + (size_t)b * S, L > 0, wsv, s, (int64_t)b * S));
      }
    }
    for (int b = 0; b < n_seq; ++b) {
      if (done[b]) continue;
      const size_t o = (size_t)b * S;
      DG_LAUNCH(DG_K_STOP_CHECK, s,
                launch_stop_check(wsv.ent + o, wsv.pred + o, wsv.prev_pred + o, wsv.canvas + o, lock_of(b), S, t,
                                  stp, wsv.status + b, s));
    }
    bool stop[kMaxSeq] = {};
    if (fixed) {
      for (int b = 0; b < n_seq; ++b) stop[b] = t >= sp->fixed_steps;
    } else {
      DG_TRY(hipMemcpyAsync(st, wsv.status, sizeof(dg_block_status) * n_seq, hipMemcpyDeviceToHost, s));
      DG_TRY(hipStreamSynchronize(s));
      for (int b = 0; b < n_seq; ++b) stop[b] = !done[b] && st[b].reason != DG_STOP_NONE;
    }
    for (int b = 0; b < n_seq; ++b) {
      if (done[b] || !stop[b]) continue;
      DG_TRY(hipMemcpyAsync(tokens_out + (size_t)b * S, wsv.pred + (size_t)b * S, (size_t)S * 4,
                            hipMemcpyDeviceToDevice, s));
      done[b] = true;
      ++n_done;
    }
    if (n_done == n_seq) break;
    const int keep = (int)std::min<int64_t>(S, (int64_t)t * sp->n_new);
    for (int b = 0; b < n_seq; ++b) {
      if (done[b]) continue;
      const size_t o = (size_t)b * S;
      CanvasArgs ca{wsv.pred + o, wsv.conf + o, wsv.ent + o, by_ent ? 1 : 0, lock_of(b), S, keep, sp->seed,
                    h_blocks[b], (uint32_t)t, V, wsv.canvas + o, lock_of(b)};
      DG_LAUNCH(DG_K_CANVAS_UPDATE, s, launch_canvas_update(ca, s));
    }
  }
  if (fixed) DG_TRY(hipMemcpyAsync(st, wsv.status, sizeof(dg_block_status) * n_seq, hipMemcpyDeviceToHost, s));
  if (!defer_commit) {
    // commit every block in one causal forward: each sequence's rows attend causally within its own cache
    DG_CHECK(embed(cfg, w, tokens_out, M, wsv, s));
    Segs cg = sg;
    for (int b = 0; b < n_seq; ++b) cg.seg[b].n_causal = S;
    for (int l = 0; l < L; ++l)
      DG_CHECK(layer(cfg, w, l, cg, M, l > 0, l + 1 < L ? Next::NextLayer : Next::None, wsv, side, s));
  }
  DG_TRY(hipStreamSynchronize(s));
  for (int b = 0; b < n_seq; ++b) {
    if (!defer_commit) kvs[b].len += S;
    h_status[b] = st[b];
  }
  return DG_OK;
}

int dg_generate_blocks(const dg_config* cfg, const dg_weights* w, dg_kv* kvs, int32_t n_seq, const dg_sampler* sp,
                       const uint32_t* h_blocks, int32_t* tokens_out, dg_block_status* h_status, void* ws,
                       size_t ws_bytes, const dg_side* side, void* stream) {
  return dg_generate_blocks_overlapped(cfg, w, kvs, n_seq, sp, h_blocks, nullptr, 0, tokens_out, h_status, ws,
                                       ws_bytes, side, stream);
}

int dg_verify_block(const dg_config* cfg, const dg_weights* w, dg_kv* kv, const int32_t* draft, int32_t* ar_pred,
                    int32_t* h_accepted, int32_t* h_next_token, void* ws, size_t ws_bytes, const dg_side* side,
                    void* stream) {
  DG_CHECK(check_cfg(cfg));
  DG_CHECK(check_side(side));
  DG_CHECK(check_weights(cfg, w, true, true));
  if (!draft || !ar_pred || !h_accepted || !h_next_token) return DG_ERR_INVALID;
  const int S = cfg->canvas;
  DG_CHECK(check_kv(kv, S));
  DG_CHECK(check_ws(cfg, S, ws, ws_bytes));
  Ws wsv = carve(cfg, S, (char*)ws);
  return verify_rows(cfg, w, kv, draft, ar_pred, wsv, side, (hipStream_t)stream, h_accepted, h_next_token);
}

int dg_generate_speculative(const dg_config* cfg, const dg_weights* w, dg_kv* kv, const dg_sampler* sp,
                            uint32_t block0, int32_t first_token, int32_t n_tokens, int32_t* tokens_out,
                            int32_t* h_accepted, dg_spec_status* h_status, void* ws, size_t ws_bytes,
                            const dg_side* side, void* stream) {
  DG_CHECK(check_cfg(cfg));
  DG_CHECK(check_side(side));
  DG_CHECK(check_weights(cfg, w, true, true));
  DG_CHECK(check_sampler(cfg, sp));
  if (!tokens_out || !h_status || n_tokens < 1 || first_token < 0 || first_token >= cfg->vocab)
    return DG_ERR_INVALID;
  const int S = cfg->canvas;
  // every round starts with kv->len below len0 + n_tokens and needs S rows after it
  DG_CHECK(check_kv(kv, (int64_t)n_tokens - 1 + S));
  DG_CHECK(check_ws(cfg, S, ws, ws_bytes));
  hipStream_t s = (hipStream_t)stream;
  Ws wsv = carve(cfg, S, (char*)ws);
  dg_spec_status out{};
  int32_t nxt = first_token;
  while (out.tokens < n_tokens) {
    dg_block_status st{};
    DG_CHECK(block_loop(cfg, w, kv, sp, block0 + (uint32_t)out.rounds, nullptr, wsv, side, s, &st));
    // the draft: the block's tokens with the known next token in slot 0 (wsv.canvas is free after the block)
    DG_TRY(hipMemcpyAsync(wsv.canvas, wsv.pred, (size_t)S * 4, hipMemcpyDeviceToDevice, s));
    DG_TRY(hipMemsetD32Async((hipDeviceptr_t)wsv.canvas, nxt, 1, s));
    int32_t acc = 0;
    DG_CHECK(verify_rows(cfg, w, kv, wsv.canvas, wsv.pred, wsv, side, s, &acc, &nxt));
    const int take = std::min(acc, n_tokens - out.tokens);
    DG_TRY(hipMemcpyAsync(tokens_out + out.tokens, wsv.canvas, (size_t)take * 4, hipMemcpyDeviceToDevice, s));
    if (h_accepted) h_accepted[out.rounds] = acc;
    out.tokens += take;
    out.accepted += acc;
    out.rounds += 1;
  }
  out.next_token = nxt;
  DG_TRY(hipStreamSynchronize(s));
  *h_status = out;
  return DG_OK;
}

int dg_layer_forward(const dg_config* cfg, const dg_weights* w, int32_t layer_i, const dg_kv* kv, const void* x_in,
                     void* x_out, int64_t n, int32_t causal, const dg_debug* dbg, void* ws, size_t ws_bytes,
                     const dg_side* side, void* stream) {
  DG_CHECK(check_cfg(cfg));
  DG_CHECK(check_side(side));
  if (!w || !w->h_layers || layer_i < 0 || layer_i >= cfg->n_layers) return DG_ERR_INVALID;
  DG_CHECK(check_layer_weights(cfg, w->h_layers[layer_i]));
  if (!aligned16(x_in) || !aligned16(x_out) || n < 1 || n > moe_max_rows(cfg->n_experts)) return DG_ERR_INVALID;
  if (causal != 0 && causal != 1) return DG_ERR_INVALID;
  DG_CHECK(check_kv(kv, n));
  DG_CHECK(check_ws(cfg, n, ws, ws_bytes));
  hipStream_t s = (hipStream_t)stream;
  Ws wsv = carve(cfg, n, (char*)ws);
  const size_t hb = (size_t)n * cfg->d_model * esize(cfg);
  DG_TRY(hipMemcpyAsync(wsv.X, x_in, hb, hipMemcpyDeviceToDevice, s));
  DG_CHECK(layer(cfg, w, layer_i, kv, kv->len, n, causal != 0 ? n : 0, false, Next::None, wsv, side, s));
  DG_TRY(hipMemcpyAsync(x_out, wsv.X, hb, hipMemcpyDeviceToDevice, s));
  if (dbg) {
    const size_t rb = (size_t)n * cfg->top_k * 4;
    if (dbg->route_idx) DG_TRY(hipMemcpyAsync(dbg->route_idx, wsv.ridx, rb, hipMemcpyDeviceToDevice, s));
    if (dbg->route_w) DG_TRY(hipMemcpyAsync(dbg->route_w, wsv.rw, rb, hipMemcpyDeviceToDevice, s));
    if (dbg->router_logits)
      DG_TRY(hipMemcpyAsync(dbg->router_logits, wsv.rlog, (size_t)n * cfg->n_experts * 4, hipMemcpyDeviceToDevice,
                            s));
  }
  return DG_OK;
}

int dg_vocab_head(const dg_config* cfg, const dg_weights* w, const void* x, int64_t n, float inv_temperature,
                  int32_t* pred, float* conf, float* entropy, void* ws, size_t ws_bytes, void* stream) {
  DG_CHECK(check_cfg(cfg));
  DG_CHECK(check_weights(cfg, w, false, true));
  if (!aligned16(x) || !pred || !conf || !entropy || n < 1 || n > moe_max_rows(cfg->n_experts))
    return DG_ERR_INVALID;
  if (!(inv_temperature > 0.f)) return DG_ERR_INVALID;
  DG_CHECK(check_ws(cfg, n, ws, ws_bytes));
  hipStream_t s = (hipStream_t)stream;
  Ws wsv = carve(cfg, n, (char*)ws);
  DG_TRY(hipMemcpyAsync(wsv.X, x, (size_t)n * cfg->d_model * esize(cfg), hipMemcpyDeviceToDevice, s));
  return head(cfg, w, n, argmax_pass(inv_temperature), pred, conf, entropy, false, wsv, s);
}

int dg_vocab_head_sampler(const dg_config* cfg, const dg_weights* w, const dg_sampler* sampler, uint32_t block,
                          int32_t step, const void* x, int64_t n, int32_t* pred, float* conf, float* entropy,
                          void* ws, size_t ws_bytes, void* stream) {
  DG_CHECK(check_cfg(cfg));
  DG_CHECK(check_weights(cfg, w, false, true));
  DG_CHECK(check_sampler(cfg, sampler));
  if (!aligned16(x) || !pred || !conf || !entropy || n < 1 || n > moe_max_rows(cfg->n_experts) || step < 1 ||
      step > 65535)
    return DG_ERR_INVALID;
  DG_CHECK(check_ws(cfg, n, ws, ws_bytes));
  hipStream_t s = (hipStream_t)stream;
  Ws wsv = carve(cfg, n, (char*)ws);
  DG_TRY(hipMemcpyAsync(wsv.X, x, (size_t)n * cfg->d_model * esize(cfg), hipMemcpyDeviceToDevice, s));
  return head(cfg, w, n, sampler_pass(sampler, block, step), pred, conf, entropy, false, wsv, s);
}

int dg_sampler_inv_temperature(const dg_sampler* sampler, int32_t step, float* h_inv_temperature) {
  if (!h_inv_temperature) return DG_ERR_INVALID;
  *h_inv_temperature = 0.f;
  DG_CHECK(check_sampler(nullptr, sampler));
  if (step < 1) return DG_ERR_INVALID;
  *h_inv_temperature = pass_inv_temperature(sampler, step);
  return DG_OK;
}

int dg_stop_check(const dg_config* cfg, const dg_sampler* sampler, int32_t step, const float* entropy, int32_t* pred,
                  int32_t* prev_pred, const int32_t* canvas, const uint8_t* lock_mask, dg_block_status* d_status,
                  void* stream) {
  DG_CHECK(check_cfg(cfg));
  DG_CHECK(check_sampler(cfg, sampler));
  if (step < 1 || !entropy || !pred || !prev_pred || !d_status) return DG_ERR_INVALID;
  const bool lock = (sampler->flags & DG_KEEP_LOCK) != 0;
  if (lock && (!canvas || !lock_mask)) return DG_ERR_INVALID;
  DG_LAUNCH(DG_K_STOP_CHECK, (hipStream_t)stream,
            launch_stop_check(entropy, pred, prev_pred, lock ? canvas : nullptr, lock ? lock_mask : nullptr,
                              cfg->canvas, step, stop_params(cfg, sampler), d_status, (hipStream_t)stream));
  return DG_OK;
}

int dg_side_create(dg_side* h_side) {
  if (!h_side) return DG_ERR_INVALID;
  *h_side = dg_side{nullptr, nullptr, nullptr};
  hipStream_t st = nullptr;
  hipEvent_t f = nullptr, j = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);  // default priority
  if (e == hipSuccess) e = hipEventCreateWithFlags(&f, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&j, hipEventDisableTiming);
  if (e != hipSuccess) {
    if (j) (void)hipEventDestroy(j);
    if (f) (void)hipEventDestroy(f);
    if (st) (void)hipStreamDestroy(st);
    g_hip_error = (int)e;
    return DG_ERR_HIP;
  }
  *h_side = dg_side{st, f, j};
  return DG_OK;
}

int dg_side_destroy(dg_side* h_side) {
  if (!h_side) return DG_ERR_INVALID;
  hipError_t e = hipSuccess, r;
  if (h_side->stream && (r = hipStreamSynchronize((hipStream_t)h_side->stream)) != hipSuccess) e = r;
  if (h_side->join && (r = hipEventDestroy((hipEvent_t)h_side->join)) != hipSuccess) e = r;
  if (h_side->fork && (r = hipEventDestroy((hipEvent_t)h_side->fork)) != hipSuccess) e = r;
  if (h_side->stream && (r = hipStreamDestroy((hipStream_t)h_side->stream)) != hipSuccess) e = r;
  *h_side = dg_side{nullptr, nullptr, nullptr};
  if (e != hipSuccess) {
    g_hip_error = (int)e;
    return DG_ERR_HIP;
  }
  return DG_OK;
}

int dg_packed_elems(int64_t rows, int64_t cols, int64_t* h_elems) {
  if (!h_elems) return DG_ERR_INVALID;
  *h_elems = 0;
  if (rows < 1 || cols < 32 || cols % 32) return DG_ERR_INVALID;
  *h_elems = (rows + 15) / 16 * 16 * cols;
  return DG_OK;
}

int dg_packed_bytes_e4m3(int64_t rows, int64_t cols, int64_t* h_bytes) {
  if (!h_bytes) return DG_ERR_INVALID;
  *h_bytes = 0;
  if (rows < 1 || cols < 64 || cols % 64) return DG_ERR_INVALID;
  *h_bytes = (rows + 15) / 16 * 16 * cols;
  return DG_OK;
}

int dg_quantize_e4m3(const void* src, void* dst, float* scale, int64_t batch, int64_t rows, int64_t cols,
                     void* stream) {
  int64_t per = 0;
  DG_CHECK(dg_packed_bytes_e4m3(rows, cols, &per));
  if (batch < 1 || !aligned16(src) || !aligned16(dst) || !scale || ((uintptr_t)scale & 3u)) return DG_ERR_INVALID;
  const uintptr_t s0 = (uintptr_t)src, s1 = s0 + (size_t)(batch * rows * cols) * 2;
  const uintptr_t d0 = (uintptr_t)dst, d1 = d0 + (size_t)(batch * per);
  const uintptr_t c0 = (uintptr_t)scale, c1 = c0 + (size_t)(batch * rows) * 4;
  if ((s0 < d1 && d0 < s1) || (s0 < c1 && c0 < s1) || (d0 < c1 && c0 < d1)) return DG_ERR_INVALID;
  DG_TRY(launch_quantize_e4m3((const bf16*)src, (uint8_t*)dst, scale, batch, rows, cols, (hipStream_t)stream));
  return DG_OK;
}

int dg_pack_matrix(const void* src, void* dst, int64_t batch, int64_t rows, int64_t cols, int32_t dtype,
                   void* stream) {
  int64_t per = 0;
  DG_CHECK(dg_packed_elems(rows, cols, &per));
  if (batch < 1 || !aligned16(src) || !aligned16(dst) || (dtype != DG_BF16 && dtype != DG_F32)) return DG_ERR_INVALID;
  const size_t es = dtype == DG_BF16 ? 2 : 4;
  const uintptr_t s0 = (uintptr_t)src, s1 = s0 + (size_t)(batch * rows * cols) * es;
  const uintptr_t d0 = (uintptr_t)dst, d1 = d0 + (size_t)(batch * per) * es;
  if (s0 < d1 && d0 < s1) return DG_ERR_INVALID;
  if (dtype == DG_BF16)
    DG_TRY(launch_pack<bf16>((const bf16*)src, (bf16*)dst, batch, rows, cols, (hipStream_t)stream));
  else
    DG_TRY(launch_pack<float>((const float*)src, (float*)dst, batch, rows, cols, (hipStream_t)stream));
  return DG_OK;
}

int dg_timing_start(uint64_t kernel_mask) {
  g_timer.mask = kernel_mask;
  return DG_OK;
}

int dg_timing_stop(double* h_ms, int64_t* h_launches) {
  g_timer.mask = 0;
  if (h_ms)
    for (int i = 0; i < DG_K_COUNT; ++i) h_ms[i] = 0.0;
  if (h_launches)
    for (int i = 0; i < DG_K_COUNT; ++i) h_launches[i] = 0;
  int rc = DG_OK;
  for (const TimerRec& r : g_timer.recs) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) {
      g_hip_error = (int)e;
      rc = DG_ERR_HIP;
    }
    if (h_ms) h_ms[r.id] += ms;
    if (h_launches) h_launches[r.id] += 1;
    g_timer.pool.push_back(r.a);
    g_timer.pool.push_back(r.b);
  }
  g_timer.recs.clear();
  return rc;
}

const char* dg_status_string(int status) {
  switch (status) {
    case DG_OK: return "ok";
    case DG_ERR_INVALID: return "invalid argument";
    case DG_ERR_UNSUPPORTED: return "unsupported configuration";
    case DG_ERR_KV_FULL: return "KV cache capacity exceeded";
    case DG_ERR_WORKSPACE: return "workspace missing or too small";
    case DG_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int dg_last_hip_error(void) { return g_hip_error; }

}  // extern "C"
