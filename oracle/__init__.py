"""CPU oracle of the block-diffusion denoising step — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call this package.  The product path (the HIP
library and its Python binding) never does, and shares no code with it: the two
sides meet only in the seeded input generator ``dg_inputs``.

What it is: a plain, slow, obviously correct numpy implementation in float64 of
one denoising pass, the canvas update, the stop rule, prefill/commit and the
block loop, written from the pages' description:

  [P1] "DiffusionGemma: When Text Generation Stops Being Sequential"
       (laura-martel.com blog)
  [P2] "DiffusionGemma 26B: How Google's Text Diffusion Model Generates Tokens
       in Parallel" (dev.to)
  [P3] "DiffusionGemma local text generation" (ctxwire.com)
  [P5] "When to use a diffusion LLM: I compared DiffusionGemma and Gemma 4"
       (Medium repost)

Modules:
  numerics — bf16 round-to-nearest-even from float64, decision-precision helpers,
             OCP E4M3 decoding, rounding and per-channel quantisation
  philox   — Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) and the
             uniform token draw U(seed, block, step, slot)
  model    — RMSNorm, bidirectional/causal attention, router, MoE, vocab head
  sampler  — keep schedule, canvas update, stop rule, pass/prefill/commit/block

Pins (tests/test_oracle_*.py, all run without a GPU):
  * softmax/entropy/confidence: uniform logits give ln V exactly; two-level
    logits match the closed form; sum of probabilities is 1; entropy in [0, ln V]
  * head: equals an independent pure-Python loop softmax on tiny sizes;
    argmax ties resolve to the lowest token id
  * attention: a single key returns its value; identical keys return the mean
    of the values; permutation equivariance over canvas slots (no positional
    term); pure-Python loop brute force on tiny sizes; causal first row = V[0]
  * RMSNorm: constant input closed form
  * router: weights sum to 1; equal logits pick experts 0..k-1; brute force
  * MoE: identical experts reduce to the dense SwiGLU FFN whatever the routing
  * keep/update: |kept| = k_t, kept slots equal pred, unkept slots equal the
    Philox draw, canvas always S in-range tokens
  * Philox: published known-answer vectors of Philox4x32-10
  * stop rule: engineered cases E1 (uniform logits -> stable at step 2),
    E2 (self-retrieval -> entropy stop at step 1), fixed-T stop, 48-step cap
  * bf16 rounding: exhaustive agreement with the fp32 route on all bf16
    neighbours and ties
  * layer wiring (tests/test_oracle_wiring.py): closed forms for weights that
    make the block solvable by hand (W_o = 0 with routed experts equal to the
    shared one; W_q = 0 with zero down projections; both), computed with plain
    loops and distinct attention / FFN norm gains
  * canvas token mapping: the all-zero Philox counter's published word 0
    mapped by the multiply-shift (104607 of 262144, 1634 of 4096)
  * SiLU: silu(1), silu(-1), silu(0) and the large-|z| limits
  * FP8 (OCP E4M3) weights (tests/test_oracle_fp8.py): every code decoded and
    every tie rounded as torch's float8_e4m3fn conversion does, the format's
    fixed points (448, 2^-6, 2^-9, NaN codes), saturation, per-channel
    quantisation closed forms and error bound, scaled experts equal to the
    dequantised FFN, the FP8 tied embedding dequantised per vocabulary row
    (exact for representable rows, the E4M3 bound per row, lookup rounded)
Parity unpinned: none of the functions above is left without a pin; the
whole-model forward has no golden values on the pages and is pinned only
through its parts.
"""
from . import numerics, philox, model, sampler  # noqa: F401
