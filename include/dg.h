/* dg.h — C ABI of the MI355X block-diffusion denoising library (libdg.so).
 *
 * One denoising pass of a DiffusionGemma-style block-diffusion model at batch 1,
 * plus the canvas update, the stop rule, prompt prefill and block commit.
 * Page references:
 *   [P1] "DiffusionGemma: When Text Generation Stops Being Sequential" (blog)
 *   [P2] "DiffusionGemma 26B: How Google's Text Diffusion Model Generates Tokens
 *        in Parallel" (dev.to)
 *   [P3] "DiffusionGemma local text generation" (ctxwire)
 *   [P5] "When to use a diffusion LLM: I compared DiffusionGemma and Gemma 4"
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless the name starts with h_.
 *   - The caller owns all memory (weights, KV cache, inputs, outputs, workspace)
 *     and every stream and event; the library never allocates device memory and
 *     keeps no device state beyond its loaded code objects (which hold the fixed
 *     scratch of dg_denoise_step_noalloc).  Calls that run layers
 *     take an optional caller-owned dg_side (below) for the shared expert's
 *     concurrency.
 *     Calls on one caller stream must be issued from one host thread at a time.
 *   - Calls are stream-ordered and return after enqueueing on `stream` (a
 *     hipStream_t passed as void*; NULL = the default stream).  Exceptions:
 *     dg_generate_block in adaptive mode waits once per pass for a 16-byte status,
 *     and dg_workspace_size / dg_status_string are host-only.
 *   - Return value: DG_OK (0) or a negative dg_status.  Arguments are validated
 *     before any HIP call, so a validation error enqueues nothing and writes
 *     nothing.  DG_ERR_HIP keeps the HIP error code for dg_last_hip_error().
 *   - Calls on distinct workspaces and streams may run concurrently; two calls
 *     sharing one workspace must be ordered on one stream.
 *
 * Tensor layouts (dtype = cfg->dtype unless stated):
 *   hidden states      [n, d_model] row-major
 *   norm gains         [d_model]
 *   KV cache  k        [n_layers][n_kv_heads][capacity][head_dim] row-major
 *             v        [n_layers][n_kv_heads][head_dim][capacity] (positions contiguous)
 *   tokens / canvas    int32 [n]
 * Weight matrices, logically [out, in] (y = x W^T):
 *   embed (tied head)  [vocab, d_model]
 *   wqkv               [(n_heads + 2*n_kv_heads)*head_dim, d_model]
 *                      rows: query heads, then key heads, then value heads
 *   wo                 [d_model, n_heads*head_dim]
 *   w_router           [n_experts, d_model]
 *   w_gate_up          n_experts x [2*ffn_expert, d_model]  gate rows, then up rows
 *   w_down             n_experts x [d_model, ffn_expert]
 *   ws_gate_up         [2*ffn_shared, d_model]              gate rows, then up rows
 *   ws_down            [d_model, ffn_shared]
 * are stored in the FRAGMENT-TILED layout that dg_pack_matrix produces from a
 * row-major matrix: with R rows padded up to a multiple of 16 and C columns (a
 * multiple of 32), element (r, c) sits at
 *     ((r/16)*(C/32) + c/32)*512 + ((r%16) + 16*((c%32)/8))*8 + c%8,
 * i.e. each 16-row x 32-column block is one contiguous 512-element fragment in
 * the matrix cores' operand order (a 1 KB bf16 block that one 64-lane wave reads
 * with a single contiguous 16-byte-per-lane load).  Padded rows are zero.
 * Batched weights (w_gate_up, w_down) are n_experts such tiled matrices back to
 * back.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dg_status {
  DG_OK = 0,
  DG_ERR_INVALID = -1,     /* null pointer, bad dimension, out-of-range argument */
  DG_ERR_UNSUPPORTED = -2, /* valid but not built: e.g. head_dim not 64/128, rope_theta != 0 */
  DG_ERR_KV_FULL = -3,     /* kv->len + rows > kv->capacity */
  DG_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than dg_workspace_size() */
  DG_ERR_HIP = -5          /* a HIP runtime/launch call failed; see dg_last_hip_error() */
} dg_status;

/* DG_E4M3: OCP 8-bit float (4 exponent bits, bias 7, 3 mantissa bits, largest value 448), only for the
 * routed experts' weights (dg_config.expert_dtype), with one float scale per output channel. */
typedef enum dg_dtype { DG_F32 = 0, DG_BF16 = 1, DG_E4M3 = 2 } dg_dtype;

/* Why a block stopped ([P2] "How Diffusion Changes the Equation": entropy below a
 * threshold, or predictions unchanged over two consecutive passes, or 48 passes;
 * the three are OR-ed).  FIXED = a fixed pass count requested by the caller.
 * SETTLED = low entropy and two unchanged passes together (DG_STOP_AND). */
typedef enum dg_stop {
  DG_STOP_NONE = 0,
  DG_STOP_ENTROPY = 1,
  DG_STOP_STABLE = 2,
  DG_STOP_CAP = 3,
  DG_STOP_FIXED = 4,
  DG_STOP_SETTLED = 5
} dg_stop;

/* Model dimensions.  The pages give a 128-expert MoE with 8 routed + 1 shared
 * expert, a 262K vocabulary and a 256-slot canvas ([P2] "Architecture Details");
 * the per-layer widths are the caller's.  Constraints: d_model, ffn_expert and
 * ffn_shared multiples of 32; head_dim 64 or 128; n_heads a multiple of
 * n_kv_heads with n_heads/n_kv_heads in {1, 2, 4}; top_k <= n_experts <= 256,
 * top_k <= 16; canvas <= 1024; rope_theta must be 0 (no positional term). */
typedef struct dg_config {
  int32_t n_layers;
  int32_t d_model;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t n_experts;
  int32_t top_k;
  int32_t ffn_expert;
  int32_t ffn_shared;
  int32_t vocab;
  int32_t canvas;
  int32_t dtype;      /* dg_dtype: storage type of weights, activations and KV */
  float rms_eps;      /* RMSNorm epsilon */
  float rope_theta;   /* reserved; must be 0 */
  /* Storage of the routed experts' weights (w_gate_up, w_down): 0 = dtype; DG_E4M3 = FP8 codes in the
   * FP8 pair-tiled layout (dg_quantize_e4m3) with per-output-channel scales (dg_layer_weights
   * w_gate_up_scale, w_down_scale); needs dtype DG_BF16 and d_model, ffn_expert multiples of 64.
   * ([P2] "Benchmark Numbers": the headline figure runs FP8 weights; activations stay bf16 here.) */
  int32_t expert_dtype;
  /* Storage of the tied embedding / vocab head (dg_weights embed): 0 = dtype; DG_E4M3 = FP8 codes in the FP8
   * pair-tiled layout (dg_quantize_e4m3 of the [vocab, d_model] matrix) with one float scale per vocabulary row
   * (dg_weights embed_scale); the lookup yields code * scale rounded to bf16, the head scales each row's fp32 dot
   * product.  Needs dtype DG_BF16 and d_model a multiple of 64.  ([P2] "Benchmark Numbers": FP8 weights.) */
  int32_t head_dtype;
} dg_config;

typedef struct dg_layer_weights {
  const void* attn_norm;
  const void* wqkv;
  const void* wo;
  const void* ffn_norm;
  const void* w_router;
  const void* w_gate_up;
  const void* w_down;
  const void* ws_gate_up;
  const void* ws_down;
  const float* w_gate_up_scale;  /* expert_dtype DG_E4M3: [n_experts][2*ffn_expert] (else ignored, may be NULL) */
  const float* w_down_scale;     /* expert_dtype DG_E4M3: [n_experts][d_model] */
} dg_layer_weights;

typedef struct dg_weights {
  const void* embed;                 /* [vocab, d_model], also the output head (tied) */
  const void* final_norm;            /* [d_model] */
  const dg_layer_weights* h_layers;  /* HOST array of n_layers entries of device pointers */
  const float* embed_scale;          /* head_dtype DG_E4M3: [vocab] row scales (else ignored, may be NULL) */
} dg_weights;

/* KV cache.  len and capacity are host values; capacity must be a multiple of 32.
 * Rows [0, len) hold committed context (prompt and finished blocks). */
typedef struct dg_kv {
  void* k;
  void* v;
  int64_t len;
  int64_t capacity;
} dg_kv;

/* Caller-owned concurrency for the shared expert.  Each layer's shared expert reads only
 * the FFN-normalised rows ([P2] "Architecture Details": one shared expert beside the 8
 * routed ones), so it can run on a second stream while the caller's stream does the
 * routing and the routed experts; the two join before the combine.  stream: a hipStream_t
 * other than the caller's; fork, join: two distinct hipEvent_t (timing may be disabled).
 * Every call that runs layers takes a `const dg_side* side` before its stream: NULL (or a
 * NULL side->stream) runs the shared expert on the caller's stream, with the same results
 * bit for bit.  One dg_side serves one caller stream at a time.  The library keeps no
 * reference to it after a call returns; the caller destroys it once the work that used it
 * has completed.  DG_ERR_INVALID when side->stream is set and an event is NULL or the two
 * events are the same. */
typedef struct dg_side {
  void* stream;
  void* fork;
  void* join;
} dg_side;

/* Convenience for callers: create a non-blocking stream of default priority and two events
 * with timing disabled on the current device into *h_side (all NULL on failure,
 * DG_ERR_HIP).  The caller owns them. */
int dg_side_create(dg_side* h_side);

/* Wait for h_side->stream, destroy the stream and events and clear *h_side.  Also accepts
 * a side made by the caller's own HIP calls. */
int dg_side_destroy(dg_side* h_side);

/* Sampler variants (dg_sampler.flags), each off by default.  Together they give the
 * recommended sampler of [P2] "Architecture Details" (temperature falling linearly
 * from 0.8 to 0.4 over the passes, lowest-entropy tokens locked first, stop when
 * the mean entropy is below 0.005 and the top tokens are stable over two passes);
 * [P5] "Appendix: Methodology", "Decoding" runs it with a bound of 0.1.
 *   DG_SAMPLE_GUMBEL: each slot's token is drawn from the softmax at the pass's
 *     temperature (Gumbel-max: argmax_v of beta l_v + G_v, G_v = -ln(-ln u),
 *     u = (2 floor(w / 2^9) + 1) / 2^24, w = word v mod 4 of Philox4x32-10 with key
 *     (seed low, seed high) and counter (v / 4, slot + 65536 * pass, block, 1));
 *     conf is then the probability of the drawn token.  Passes and slots < 65536.
 *   DG_SAMPLE_ANNEAL: the temperature of pass t is temperature_first + (temperature_last
 *     - temperature_first) (t - 1) / (N - 1), N = fixed_steps if > 0 else max_steps
 *     (temperature_first when N = 1); inv_temperature is then ignored.
 *   DG_KEEP_ENTROPY: the keep rule ranks by entropy, lowest first (ties to the lower
 *     slot, NaN last), instead of by confidence.
 *   DG_KEEP_LOCK: a kept slot keeps its token for the rest of the block: its
 *     prediction is replaced by that token (so stability and the committed block see
 *     it), later updates keep it and add unlocked slots until k_t are locked.
 *   DG_STOP_AND: the early stop needs mean entropy < entropy_threshold and two
 *     unchanged passes together (reason SETTLED); fixed_steps and max_steps as before. */
#define DG_SAMPLE_GUMBEL 0x1u
#define DG_SAMPLE_ANNEAL 0x2u
#define DG_KEEP_ENTROPY 0x4u
#define DG_KEEP_LOCK 0x8u
#define DG_STOP_AND 0x10u
#define DG_SAMPLER_FLAGS 0x1Fu

/* Sampler of dg_generate_block.
 *   keep count after pass t: k_t = min(canvas, t * n_new) ([P5] "How block diffusion
 *   works": keep the most confident slots, re-randomise the rest);
 *   fixed_steps > 0: run exactly that many passes (timing mode, reason FIXED);
 *   otherwise stop on mean entropy < entropy_threshold, on two equal consecutive
 *   predictions, or at max_steps (<= 48 by default, any value >= 1 accepted).
 *   seed keys the Philox canvas draws; inv_temperature scales the logits.
 *   flags: DG_SAMPLE_* / DG_KEEP_* / DG_STOP_AND bits (above); other bits are invalid. */
typedef struct dg_sampler {
  int32_t n_new;
  int32_t max_steps;
  int32_t fixed_steps;
  float entropy_threshold;
  float inv_temperature;
  uint32_t flags;
  uint64_t seed;
  float temperature_first;  /* DG_SAMPLE_ANNEAL: temperature of pass 1 (> 0) */
  float temperature_last;   /* DG_SAMPLE_ANNEAL: temperature of the last pass of the budget (> 0) */
} dg_sampler;

/* Block status (host struct for dg_generate_block; device struct for dg_stop_check). */
typedef struct dg_block_status {
  int32_t steps;         /* passes run */
  int32_t reason;        /* dg_stop */
  float mean_entropy;    /* mean over all canvas slots of the last pass, nats */
  uint32_t flags;        /* DG_WARN_* bits */
} dg_block_status;

#define DG_WARN_NUMERIC 0x1u /* some slot entropy was NaN or outside [0, ln V] */

/* Optional per-layer dumps of dg_denoise_step (parity tests); any field may be NULL.
 *   hidden        [n_layers, canvas, d_model]    residual stream after each layer (dtype)
 *   route_idx     [n_layers, canvas, top_k]      int32 chosen experts, descending logit
 *   route_w       [n_layers, canvas, top_k]      float routing weights
 *   router_logits [n_layers, canvas, n_experts]  float router logits the choice was made on */
typedef struct dg_debug {
  void* hidden;
  int32_t* route_idx;
  float* route_w;
  float* router_logits;
} dg_debug;

/* Elements of the fragment-tiled form of a rows x cols matrix (rows rounded up to
 * 16; cols must be a positive multiple of 32, else 0 is written and DG_ERR_INVALID
 * returned).  Host-only. */
int dg_packed_elems(int64_t rows, int64_t cols, int64_t* h_elems);

/* Convert `batch` row-major [rows, cols] matrices at src (dtype DG_BF16 or DG_F32)
 * into the fragment-tiled layout at dst (batch * dg_packed_elems elements; padded
 * rows are written as zeros).  src and dst must not overlap; both 16-byte aligned.
 * This is how callers bring weights into the layout dg_weights expects. */
int dg_pack_matrix(const void* src, void* dst, int64_t batch, int64_t rows, int64_t cols, int32_t dtype,
                   void* stream);

/* Bytes of the FP8 pair-tiled form of a rows x cols matrix (rows rounded up to 16; cols a positive multiple of
 * 64, else 0 is written and DG_ERR_INVALID returned).  Host-only. */
int dg_packed_bytes_e4m3(int64_t rows, int64_t cols, int64_t* h_bytes);

/* Quantise `batch` row-major [rows, cols] bf16 matrices at src (cols a multiple of 64) to OCP E4M3 with one
 * scale per row (output channel): scale[b * rows + r] = amax / 448 of row r (1 for an all-zero row), code =
 * the E4M3 value nearest to w / scale (ties to the even mantissa, beyond 448 saturated; the division and the
 * decision in float32).  Codes go to dst in the FP8 pair-tiled layout (batch * dg_packed_bytes_e4m3 bytes):
 * with R rows padded to 16, element (r, c) is byte
 *     ((r/16)*(cols/64) + c/64)*1024 + ((r%16) + 16*((c%32)/8))*16 + ((c%64)/32)*8 + c%8,
 * so that one 16-byte load gives a 64-lane wave's lane its elements of two consecutive 32-wide K steps.
 * Padded rows are zero.  src, dst 16-byte aligned, scale 4-byte aligned; no overlap. */
int dg_quantize_e4m3(const void* src, void* dst, float* scale, int64_t batch, int64_t rows, int64_t cols,
                     void* stream);

/* Bytes of workspace needed by any call that processes up to max_tokens rows at
 * once (use cfg->canvas for denoising; a prefill chunk size for prefill/commit;
 * the larger of the two for both; 1 <= max_tokens <= min(2048, 64 * (4096 /
 * n_experts)), the rows one routing step orders).  Host-only.  Longer prefills
 * are split into chunks of the largest row count the given workspace supports. */
int dg_workspace_size(const dg_config* cfg, int64_t max_tokens, size_t* h_bytes);

/* Prompt prefill: a causal forward of n tokens placed at positions
 * kv->len .. kv->len+n-1; writes their keys/values for every layer and, on
 * success, sets kv->len += n.  The prompt is read into the KV cache once
 * ([P5] "How block diffusion works"; [P2] "Architecture Details": an
 * autoregressive pass caches the prompt context).  Query i sees cache rows
 * 0 .. kv->len + i.  Tokens outside [0, vocab) are clamped into range. */
int dg_prefill_kv(const dg_config* cfg, const dg_weights* w, dg_kv* kv, const int32_t* tokens, int64_t n,
                  void* ws, size_t ws_bytes, const dg_side* side, void* stream);

/* One denoising pass over the canvas ([P2] "How Diffusion Changes the Equation":
 * bidirectional attention over the whole block; [P5] "How block diffusion works"):
 * embed the canvas, run every layer with canvas queries attending to cache rows
 * [0, kv->len) and to all canvas slots (no mask), route each slot to top_k experts
 * plus the shared expert, then the final norm and the tied vocab head.  Per slot
 * it writes pred (argmax token, ties to the lowest id), conf (largest softmax
 * probability) and entropy (nats).  The canvas keys/values are written to cache
 * rows [kv->len, kv->len + canvas) as scratch; kv->len is unchanged, so this needs
 * kv->len + canvas <= capacity.  inv_temperature multiplies the logits. */
int dg_denoise_step(const dg_config* cfg, const dg_weights* w, const dg_kv* kv, const int32_t* canvas,
                    float inv_temperature, int32_t* pred, float* conf, float* entropy, const dg_debug* dbg,
                    void* ws, size_t ws_bytes, const dg_side* side, void* stream);

/* dg_denoise_step for callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): no workspace argument and no allocation
 * of any kind.  Its scratch is a fixed array of dg_noalloc_scratch_bytes() bytes (64 MiB)
 * inside the library's code object, one per GPU, held until the process ends; a
 * configuration whose dg_workspace_size(cfg, cfg->canvas) exceeds it is rejected with
 * DG_ERR_WORKSPACE before any device work (the full-width 256-slot pass needs 58 MiB).
 * Every call on one GPU shares that GPU's array and leaves its contents behind: calls that
 * overlap on one GPU (other streams, other threads) race and give wrong results.  Outputs
 * and other errors as dg_denoise_step (no debug dumps). */
int dg_denoise_step_noalloc(const dg_config* cfg, const dg_weights* w, const dg_kv* kv, const int32_t* canvas,
                            float inv_temperature, int32_t* pred, float* conf, float* entropy, const dg_side* side,
                            void* stream);

/* Bytes of the fixed scratch of dg_denoise_step_noalloc.  Host-only. */
int dg_noalloc_scratch_bytes(size_t* h_bytes);

/* Pass `step` (1-based, < 65536) of block `block` as dg_generate_block runs it under
 * `sampler` ([P2] "Architecture Details"): dg_denoise_step at that pass's temperature,
 * and with DG_SAMPLE_GUMBEL pred is the drawn token and conf its probability.  The
 * lock of DG_KEEP_LOCK is applied by dg_stop_check, not here.  Errors as
 * dg_denoise_step; DG_ERR_INVALID also for an invalid sampler or step. */
int dg_denoise_step_sampler(const dg_config* cfg, const dg_weights* w, const dg_kv* kv, const dg_sampler* sampler,
                            uint32_t block, int32_t step, const int32_t* canvas, int32_t* pred, float* conf,
                            float* entropy, void* ws, size_t ws_bytes, const dg_side* side, void* stream);

/* Canvas update ([P5] "How block diffusion works": keep the most confident slots,
 * re-randomise the others; any slot may change on a later pass).  The keep_count
 * slots of highest conf (ties to the lower slot, NaN last) take pred; every other
 * slot i takes U(seed, block, step, i) = floor(w0 * vocab / 2^32), w0 the first
 * output word of Philox4x32-10 (Salmon et al., SC'11) with key (seed low, seed high)
 * and counter (i, step, block, 0).  keep_count = 0 with step = 0 gives the initial
 * random canvas (pred and conf may then be NULL).  keep_mask (uint8, may be NULL)
 * receives 1 for kept slots.  0 <= keep_count <= canvas. */
int dg_canvas_update(const dg_config* cfg, const int32_t* pred, const float* conf, int32_t keep_count,
                     uint64_t seed, uint32_t block, uint32_t step, int32_t* canvas_out, uint8_t* keep_mask,
                     void* stream);

/* The canvas update after pass `step` as dg_generate_block runs it under `sampler`: keep
 * count k_step = min(canvas, step * n_new), ranked by conf or (DG_KEEP_ENTROPY) by
 * entropy; redraws as dg_canvas_update with the sampler's seed.  step = 0 gives the
 * initial canvas.  DG_KEEP_LOCK: lock_mask (device uint8 [canvas], required) holds the
 * locked slots on entry (ignored at step 0) and on return; locked slots keep their
 * token in `canvas` (in/out) and count toward k_step.  Without it lock_mask (may be
 * NULL) receives the keep mask.  pred and the ranking input may be NULL when nothing
 * is kept.  DG_ERR_INVALID for a NULL canvas, a missing input or step < 0. */
int dg_canvas_update_sampler(const dg_config* cfg, const dg_sampler* sampler, uint32_t block, int32_t step,
                             const int32_t* pred, const float* conf, const float* entropy, int32_t* canvas,
                             uint8_t* lock_mask, void* stream);

/* Commit a finished block ([P2] "How Diffusion Changes the Equation": each 256-token
 * block is committed to the KV cache before the next; [P3] "How diffusion text
 * generation differs").  Same as dg_prefill_kv of the canvas tokens: a causal
 * forward at positions kv->len .. kv->len+canvas-1; on success kv->len += canvas. */
int dg_commit_block(const dg_config* cfg, const dg_weights* w, dg_kv* kv, const int32_t* block_tokens,
                    void* ws, size_t ws_bytes, const dg_side* side, void* stream);

/* One whole block: initial random canvas, passes t = 1, 2, ... each followed by
 * the stop check and, if not stopping, the canvas update with k_t; then the last
 * pass's predictions are written to tokens_out [canvas] and committed (kv->len
 * grows by canvas).  h_status (host) receives steps, reason and mean entropy.
 * Adaptive mode synchronises `stream` once per pass to read a 16-byte status;
 * fixed mode (sampler->fixed_steps > 0) synchronises once at the end. */
int dg_generate_block(const dg_config* cfg, const dg_weights* w, dg_kv* kv, const dg_sampler* sampler,
                      uint32_t block, int32_t* tokens_out, dg_block_status* h_status, void* ws,
                      size_t ws_bytes, const dg_side* side, void* stream);

/* dg_generate_block with each commit overlapped on the next block's first pass.  The commit
 * and a pass are both a forward of 256 rows through every layer, and the expert and head
 * weights dominate their cost, so one forward of both row sets streams the weights once.
 * pending (nullable, device [canvas]): tokens of an earlier block generated with
 * defer_commit = 1 and not yet committed.  They are committed at kv->len inside this
 * block's first pass: rows 0 .. canvas-1 of that forward attend causally and their keys and
 * values become cache rows kv->len ..; then kv->len grows by canvas before the later passes.
 * defer_commit (0 or 1): with 1 this block's tokens (tokens_out) are not committed; pass them
 * as `pending` to the next call or commit them with dg_commit_block.  pending may alias
 * tokens_out (it is read in the first pass, before tokens_out is written).  With pending,
 * the workspace and the cache must hold 2 * canvas rows (dg_workspace_size(cfg, 2 * canvas,
 * ...); kv->len + 2 * canvas <= capacity), and 2 * canvas must not exceed the rows one
 * routing step orders, min(2048, 64 * (4096 / n_experts)) (else DG_ERR_INVALID).  The tokens and cache equal those of
 * dg_generate_block on the same blocks up to the summation order of the attention splits.
 * Errors as dg_generate_block; DG_ERR_INVALID also for defer_commit not 0 or 1. */
int dg_generate_block_overlapped(const dg_config* cfg, const dg_weights* w, dg_kv* kv,
                                 const dg_sampler* sampler, uint32_t block, const int32_t* pending,
                                 int32_t defer_commit, int32_t* tokens_out, dg_block_status* h_status,
                                 void* ws, size_t ws_bytes, const dg_side* side, void* stream);

/* Blocks of n_seq independent sequences at once (batch > 1 canvases; [P2] "Benchmark Numbers"
 * runs batch 4).  Sequence b has its own cache kvs[b] (host array of n_seq caches, no two sharing
 * memory), block id h_blocks[b] (host) for its Philox draws, and output tokens_out[b * canvas ..]
 * (device [n_seq][canvas]); h_status[b] (host) receives its status.  Each sequence's result equals
 * dg_generate_block on its own (up to the summation order of attention splits): the passes run
 * over all n_seq canvases together (every weight read serves all of them), each canvas attends to
 * its own cache, and its stop check and update are its own.  In adaptive mode a finished canvas is
 * carried along unchanged until every canvas has stopped.  The blocks are committed together at
 * the end (kvs[b].len += canvas).  1 <= n_seq <= 8, n_seq * canvas <= the routing row limit
 * (2048 for 128 experts); the workspace must hold n_seq * canvas rows and each cache canvas more
 * rows.  DG_ERR_INVALID for a bad count, aliasing caches or NULL arrays; others as
 * dg_generate_block. */
int dg_generate_blocks(const dg_config* cfg, const dg_weights* w, dg_kv* kvs, int32_t n_seq,
                       const dg_sampler* sampler, const uint32_t* h_blocks, int32_t* tokens_out,
                       dg_block_status* h_status, void* ws, size_t ws_bytes, const dg_side* side, void* stream);

/* dg_generate_blocks with each sequence's commit carried by the next call's first pass, as
 * dg_generate_block_overlapped does for one sequence.  pending (nullable, device [n_seq][canvas]):
 * blocks of an earlier call made with defer_commit = 1; sequence b's pending block is committed at
 * kvs[b].len inside this call's first pass (its rows attend causally, the canvas rows see them),
 * then kvs[b].len grows by canvas.  defer_commit (0 or 1): with 1 this call's blocks are not
 * committed.  pending may alias tokens_out.  With pending the pass holds 2 * n_seq * canvas rows
 * (<= the routing row limit: 4 canvases of 256 for 128 experts), the workspace must hold them and
 * each cache 2 * canvas more rows.  Errors as dg_generate_blocks; DG_ERR_INVALID also for
 * defer_commit not 0 or 1. */
int dg_generate_blocks_overlapped(const dg_config* cfg, const dg_weights* w, dg_kv* kvs, int32_t n_seq,
                                  const dg_sampler* sampler, const uint32_t* h_blocks, const int32_t* pending,
                                  int32_t defer_commit, int32_t* tokens_out, dg_block_status* h_status,
                                  void* ws, size_t ws_bytes, const dg_side* side, void* stream);

/* Self-speculative verify of a drafted block ([P1] "The result that complicates 'faster, not
 * smarter'": one set of weights drafts a block bidirectionally and verifies it causally over the
 * same KV cache).  The commit's causal forward over draft (device [canvas], e.g. dg_generate_block
 * output with the commit deferred) at positions kv->len.. writes their keys and values and the
 * greedy prediction of each row, the token the causal pass gives the position after it, to
 * ar_pred (device [canvas]).  draft[0] is taken as drafted; draft[i] (i >= 1) is accepted while
 * every earlier one was and ar_pred[i - 1] == draft[i].  h_accepted (host) receives the count
 * (1 .. canvas) and h_next_token (host) ar_pred[count - 1], the causal pass's token for the first
 * position not accepted.  kv->len grows by the count; the cache rows past it are scratch.  Needs
 * kv->len + canvas <= capacity and a workspace of canvas rows; synchronises `stream` once. */
int dg_verify_block(const dg_config* cfg, const dg_weights* w, dg_kv* kv, const int32_t* draft, int32_t* ar_pred,
                    int32_t* h_accepted, int32_t* h_next_token, void* ws, size_t ws_bytes, const dg_side* side, void* stream);

/* Status of dg_generate_speculative (host struct). */
typedef struct dg_spec_status {
  int32_t rounds;      /* drafts verified */
  int32_t tokens;      /* tokens written to tokens_out (n_tokens) */
  int32_t accepted;    /* draft tokens accepted over all rounds (>= tokens; the last round's surplus stays cached) */
  int32_t next_token;  /* the causal prediction for the position after the last accepted token */
} dg_spec_status;

/* Self-speculative decoding ([P1] "The result that complicates 'faster, not smarter'": the same weights draft a
 * block by diffusion and check it autoregressively over one shared KV cache).  first_token is the known token at
 * position kv->len (e.g. the causal prediction after the prompt).  Each round r drafts a block by diffusion at
 * the cache's end under `sampler` (block id block0 + r, the commit deferred), puts the known token in slot 0 of
 * the draft and verifies it as dg_verify_block does: the accepted prefix is committed and written to tokens_out,
 * and the causal prediction after it is the next round's known token.  Rounds run until n_tokens tokens are out
 * (device tokens_out [n_tokens]); the output equals greedy autoregressive decoding from first_token, and the
 * drafts decide how many tokens each causal pass confirms.  h_accepted (host, nullable, n_tokens entries)
 * receives each round's accepted count, h_status the totals.  kv->len grows by every accepted token.  Needs
 * kv->len + n_tokens - 1 + canvas <= capacity (DG_ERR_KV_FULL) and a workspace of canvas rows; synchronises the
 * stream once per round.  DG_ERR_INVALID for n_tokens < 1 or first_token outside [0, vocab). */
int dg_generate_speculative(const dg_config* cfg, const dg_weights* w, dg_kv* kv, const dg_sampler* sampler,
                            uint32_t block0, int32_t first_token, int32_t n_tokens, int32_t* tokens_out,
                            int32_t* h_accepted, dg_spec_status* h_status, void* ws, size_t ws_bytes,
                            const dg_side* side, void* stream);

/* --- finer-grained calls of the same path (each is one stage of dg_denoise_step) --- */

/* One transformer block `layer` over n hidden rows x_in -> x_out ([n, d_model];
 * x_out may equal x_in).  Rows sit at cache positions kv->len .. kv->len+n-1 and
 * their keys/values are written there for this layer; kv->len is unchanged.
 * causal = 0: every row sees all cache rows and all n rows (canvas pass);
 * causal = 1: row i sees cache rows 0 .. kv->len + i (prefill/commit).
 * dbg (may be NULL): route_idx / route_w / router_logits receive this layer's
 * [n, top_k] routing and [n, n_experts] logits; its hidden field is ignored
 * (x_out already holds the result). */
int dg_layer_forward(const dg_config* cfg, const dg_weights* w, int32_t layer, const dg_kv* kv,
                     const void* x_in, void* x_out, int64_t n, int32_t causal, const dg_debug* dbg, void* ws,
                     size_t ws_bytes, const dg_side* side, void* stream);

/* Final RMSNorm + tied vocab projection fused with the per-slot softmax
 * statistics: for each of n rows, pred/conf/entropy as in dg_denoise_step.  The
 * n x vocab logits are never written to memory. */
int dg_vocab_head(const dg_config* cfg, const dg_weights* w, const void* x, int64_t n, float inv_temperature,
                  int32_t* pred, float* conf, float* entropy, void* ws, size_t ws_bytes, void* stream);

/* dg_vocab_head at pass `step` (1..65535) of `block` under `sampler`: that pass's
 * temperature and, with DG_SAMPLE_GUMBEL, the draw of dg_denoise_step_sampler (row i
 * is slot i of the draw's counter). */
int dg_vocab_head_sampler(const dg_config* cfg, const dg_weights* w, const dg_sampler* sampler, uint32_t block,
                          int32_t step, const void* x, int64_t n, int32_t* pred, float* conf, float* entropy,
                          void* ws, size_t ws_bytes, void* stream);

/* Host only: 1 / temperature of pass `step` (>= 1) under `sampler` (inv_temperature, or the
 * DG_SAMPLE_ANNEAL schedule), as the passes above use it.  0 is written on error. */
int dg_sampler_inv_temperature(const dg_sampler* sampler, int32_t step, float* h_inv_temperature);

/* Stop check after pass `step` (1-based): writes a dg_block_status to d_status
 * (device) with reason ENTROPY if mean(entropy) < threshold, else STABLE if
 * step >= 2 and pred equals prev_pred on every slot, else CAP if step >= max_steps,
 * else NONE (fixed_steps > 0: FIXED when step >= fixed_steps, else NONE).  With
 * DG_STOP_AND the early stop needs both conditions (reason SETTLED).  Then copies pred
 * into prev_pred.  With DG_KEEP_LOCK, pred (in/out) first takes the canvas token
 * (`canvas`, the pass's input) at every slot set in lock_mask; canvas and lock_mask are
 * required then and ignored otherwise (may be NULL).  Uses cfg->canvas slots. */
int dg_stop_check(const dg_config* cfg, const dg_sampler* sampler, int32_t step, const float* entropy, int32_t* pred,
                  int32_t* prev_pred, const int32_t* canvas, const uint8_t* lock_mask, dg_block_status* d_status,
                  void* stream);

/* --- measurement support: HIP-event timing of kernel classes --------------------- */

/* Kernel classes of one pass, for dg_timing_*. */
typedef enum dg_kernel {
  DG_K_EMBED = 0,
  DG_K_RMSNORM,
  DG_K_GEMM_QKV,
  DG_K_ATTENTION,      /* split-KV attention partials */
  DG_K_ATTN_MERGE,
  DG_K_GEMM_O,         /* output projection + residual */
  DG_K_ROUTE,          /* router logits and top-k; softmax and token->expert order
                          (two launches, timed together) */
  DG_K_MOE_GATE_UP,    /* routed experts, gate/up projections + SwiGLU */
  DG_K_MOE_DOWN,       /* routed experts, down projection */
  DG_K_SHARED_GATE_UP,
  DG_K_SHARED_DOWN,
  DG_K_MOE_COMBINE,
  DG_K_VOCAB_HEAD,
  DG_K_HEAD_MERGE,
  DG_K_STOP_CHECK,
  DG_K_CANVAS_UPDATE,
  DG_K_KV_SCATTER,     /* batched calls: new keys/values into each sequence's cache */
  DG_K_COUNT
} dg_kernel;

/* Start recording a HIP event pair around every launch, on the caller's stream, of
 * the kernel classes whose bit (1 << dg_kernel) is set in kernel_mask, for calls
 * made by this thread.  Events come from a host-side pool (no device memory). */
int dg_timing_start(uint64_t kernel_mask);

/* Stop recording, wait for the recorded events and return per-class totals:
 * h_ms[DG_K_COUNT] milliseconds and h_launches[DG_K_COUNT] launch counts (either
 * pointer may be NULL). */
int dg_timing_stop(double* h_ms, int64_t* h_launches);

/* Static description of a dg_status value. */
const char* dg_status_string(int status);

/* HIP error code of the last DG_ERR_HIP returned on this thread (0 if none). */
int dg_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DG_H */
