"""Canvas update, stop rule and the block loop, in float64 (test infrastructure only).

Page tags as in oracle.model.  The loop follows the pages' account:
  * prompt read into the KV cache once, then a 256-slot canvas of random
    vocabulary tokens ([P5] "How block diffusion works");
  * each pass predicts every slot, keeps the most confident ones and
    re-randomises the others ([P5] "How block diffusion works"; [P3] "How
    diffusion text generation differs");
  * stop when the mean canvas entropy is below a threshold, or when the
    predictions are unchanged over two consecutive passes, or after 48 passes
    ([P2] "How Diffusion Changes the Equation"; the three triggers are OR-ed);
  * the finished block joins the context (KV cache) and a fresh canvas starts
    ([P2] "How Diffusion Changes the Equation"; [P3] "How diffusion text
    generation differs").
Readings: keep count k_t = min(S, t * n_new) with no freezing (every pass
re-ranks all slots, since the pages say any slot can be revised later); ranking
by fp32 confidence, descending, ties to the lower slot, NaN last; stability
compares predictions (not the canvas) and can first fire at t = 2; the
committed block is the last pass's predictions, written to the cache by a
causal forward over the block.

Variants of the recommended sampler ([P2] "Architecture Details"; [P5] "Appendix:
Methodology", "Decoding"), each off by default:
  * gumbel: each slot's token is drawn from the softmax at the pass's temperature
    (Gumbel-max, oracle.philox.gumbel_noise) instead of taken as the argmax;
    confidence is then the probability of the token drawn;
  * anneal (T_first, T_last): the temperature falls linearly from T_first at pass 1
    to T_last at the last pass of the budget (fixed_steps when set, else max_steps);
  * rank_entropy: the keep rule takes the lowest-entropy slots first (fp32 entropy,
    ascending, ties to the lower slot, NaN last) instead of the most confident;
  * lock: a kept slot keeps its token for the rest of the block: its prediction is
    its token, later passes only add slots until k_t are locked;
  * stop_and: the early stop needs low mean entropy AND two unchanged passes
    together (the cap still applies); reason STOP_SETTLED.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

from .model import KVCache, Model
from .numerics import f32
from .philox import uniform_tokens

STOP_NONE, STOP_ENTROPY, STOP_STABLE, STOP_CAP, STOP_FIXED, STOP_SETTLED = 0, 1, 2, 3, 4, 5


@dataclass
class Sampler:
    n_new: int
    max_steps: int = 48
    entropy_threshold: float = 0.05
    fixed_steps: int = 0          # >0: run exactly this many passes (timing mode), no early stop
    seed: int = 1
    inv_temperature: float = 1.0
    gumbel: bool = False
    anneal: Optional[Tuple[float, float]] = None
    rank_entropy: bool = False
    lock: bool = False
    stop_and: bool = False


def pass_inv_temperature(s: Sampler, step: int) -> float:
    """1 / T of pass ``step`` (1-based): constant, or linear in T over the pass budget."""
    if s.anneal is None:
        return float(s.inv_temperature)
    t_first, t_last = s.anneal
    n = s.fixed_steps if s.fixed_steps > 0 else s.max_steps
    frac = 0.0 if n <= 1 else min(1.0, (step - 1) / (n - 1))
    return 1.0 / (t_first + (t_last - t_first) * frac)


def keep_count(step: int, n_new: int, slots: int) -> int:
    """k_t = min(S, t * n_new) slots kept after pass t."""
    return min(slots, step * n_new)


def keep_mask(conf, k: int) -> np.ndarray:
    """The k slots of highest fp32 confidence; ties to the lower slot; NaN ranks last."""
    c = f32(conf)
    key = np.where(np.isnan(c), -np.inf, c)
    order = np.argsort(-key, kind="stable")
    mask = np.zeros(c.shape[0], dtype=bool)
    mask[order[:k]] = True
    return mask


def rank_key(conf, ent, rank_entropy: bool) -> np.ndarray:
    """Larger ranks first: fp32 confidence, or minus the fp32 entropy."""
    return -f32(ent) if rank_entropy else f32(conf)


def select_keep(key, k: int, locked=None) -> np.ndarray:
    """Locked slots, then the best unlocked slots by ``key`` (descending, ties to the lower
    slot, NaN last) until k slots are selected (more if more are locked)."""
    c = np.asarray(key)
    key = np.where(np.isnan(c), -np.inf, c)
    if locked is not None:
        key = np.where(locked, np.inf, key)
    order = np.argsort(-key, kind="stable")
    mask = np.zeros(c.shape[0], dtype=bool)
    mask[order[:k]] = True
    if locked is not None:
        mask |= locked
    return mask


def initial_canvas(seed: int, block: int, slots: int, vocab: int) -> np.ndarray:
    return uniform_tokens(seed, block, 0, np.arange(slots), vocab)


def canvas_update(pred, conf, k: int, seed: int, block: int, step: int, vocab: int, ent=None,
                  rank_entropy: bool = False, locked=None, canvas=None):
    """Kept slots take the prediction; every other slot takes a fresh uniform draw.

    With ``locked`` (the lock variant) the locked slots stay kept and keep their token
    ``canvas``; newly kept slots take the prediction."""
    if rank_entropy or locked is not None:
        mask = select_keep(rank_key(conf, ent, rank_entropy), k, locked)
    else:
        mask = keep_mask(conf, k)
    fresh = uniform_tokens(seed, block, step, np.arange(len(mask)), vocab)
    take = np.asarray(pred, dtype=np.int64)
    if locked is not None:
        take = np.where(locked, np.asarray(canvas, dtype=np.int64), take)
    return np.where(mask, take, fresh), mask


def stop_reason(step: int, mean_entropy: float, pred, prev_pred, s: Sampler) -> int:
    if s.fixed_steps > 0:
        return STOP_FIXED if step >= s.fixed_steps else STOP_NONE
    low = mean_entropy < s.entropy_threshold
    stable = prev_pred is not None and step >= 2 and np.array_equal(pred, prev_pred)
    if s.stop_and:
        if low and stable:
            return STOP_SETTLED
    elif low:
        return STOP_ENTROPY
    elif stable:
        return STOP_STABLE
    if step >= s.max_steps:
        return STOP_CAP
    return STOP_NONE


@dataclass
class PassRecord:
    canvas: np.ndarray
    pred: np.ndarray
    conf: np.ndarray
    ent: np.ndarray
    margin: np.ndarray
    keep: Optional[np.ndarray] = None
    traces: list = field(default_factory=list)


@dataclass
class BlockResult:
    tokens: np.ndarray
    steps: int
    reason: int
    mean_entropy: float
    passes: List[PassRecord]


def denoise_pass(model: Model, kv: KVCache, canvas, inv_temperature: float = 1.0, keep_traces: bool = False,
                 gumbel=None):
    """One pass: embed the canvas, run every block bidirectionally over cache + canvas, then the head
    (gumbel = (seed, block, step) draws the tokens instead of taking the argmax)."""
    x = model.embed(canvas)
    x, traces = model.body(x, kv, causal=False, append=False)
    pred, conf, ent, margin = model.head(x, inv_temperature, gumbel)
    rec = PassRecord(canvas=np.asarray(canvas), pred=pred, conf=conf, ent=ent, margin=margin)
    if keep_traces:
        rec.traces = traces
    return rec, x


def prefill(model: Model, kv: KVCache, tokens) -> None:
    """Causal forward of ``tokens`` appended after the cached rows; writes their keys/values."""
    x = model.embed(tokens)
    model.body(x, kv, causal=True, append=True)


def commit(model: Model, kv: KVCache, block_tokens) -> None:
    prefill(model, kv, block_tokens)


def generate_block(model: Model, kv: KVCache, s: Sampler, block: int, keep_traces: bool = False,
                   do_commit: bool = True) -> BlockResult:
    d = model.d
    canvas = initial_canvas(s.seed, block, d.canvas, d.vocab)
    prev = None
    locked = np.zeros(d.canvas, dtype=bool) if s.lock else None
    passes: List[PassRecord] = []
    step = 0
    reason = STOP_NONE
    mean_ent = float("nan")
    while True:
        step += 1
        rec, _ = denoise_pass(model, kv, canvas, pass_inv_temperature(s, step), keep_traces,
                              (s.seed, block, step) if s.gumbel else None)
        if locked is not None:  # a locked slot's prediction is its token
            rec.pred = np.where(locked, canvas, rec.pred)
        passes.append(rec)
        mean_ent = float(np.mean(rec.ent))
        reason = stop_reason(step, mean_ent, rec.pred, prev, s)
        if reason != STOP_NONE:
            break
        k = keep_count(step, s.n_new, d.canvas)
        canvas, rec.keep = canvas_update(rec.pred, rec.conf, k, s.seed, block, step, d.vocab, rec.ent,
                                         s.rank_entropy, locked, canvas)
        if locked is not None:
            locked = rec.keep.copy()
        prev = rec.pred
    tokens = passes[-1].pred.copy()
    if do_commit:
        commit(model, kv, tokens)
    return BlockResult(tokens=tokens, steps=step, reason=reason, mean_entropy=mean_ent, passes=passes)


@dataclass
class VerifyResult:
    accepted: int          # draft tokens accepted (>= 1)
    ar_pred: np.ndarray    # greedy prediction of the causal pass at each draft row (for the position after it)
    next_token: int        # ar_pred[accepted - 1]: the causal pass's token for the first position not accepted
    margin: np.ndarray     # fp32 top-2 logit margin of each row's prediction


def verify_block(model: Model, kv: KVCache, draft) -> VerifyResult:
    """Self-speculative verify ([P1] "The result that complicates 'faster, not smarter'": one set of weights
    drafts a block bidirectionally and verifies it causally over the same KV cache).

    Reading: a causal forward of the draft after the committed cache (the commit's forward) gives, at each row i,
    the greedy next-token prediction a_i.  Token d_0 is taken as drafted (its causal prediction would need the
    previous row's hidden state, which the cache does not keep); token d_i (i >= 1) is accepted while every
    earlier one was and a_(i-1) == d_i.  The accepted rows stay in the cache; a_(accepted - 1) is the causal
    pass's token for the next position, for the caller to use."""
    draft = np.asarray(draft, dtype=np.int64)
    base = kv.length
    x = model.embed(draft)
    x, _ = model.body(x, kv, causal=True, append=True)
    pred, _, _, margin = model.head(x)
    n = 1
    while n < len(draft) and pred[n - 1] == draft[n]:
        n += 1
    kv.truncate(base + n)
    return VerifyResult(accepted=n, ar_pred=pred, next_token=int(pred[n - 1]), margin=margin)


@dataclass
class SpeculativeResult:
    tokens: np.ndarray          # the n_tokens output tokens (positions len0 .. len0 + n_tokens - 1)
    accepted: List[int]         # tokens accepted by each verify
    drafts: List[np.ndarray]    # each verify's draft (slot 0 replaced by the token carried in)


def generate_speculative(model: Model, kv: KVCache, s: Sampler, block0: int, first_token: int,
                         n_tokens: int) -> SpeculativeResult:
    """Self-speculative decoding ([P1] "The result that complicates 'faster, not smarter'": the same weights draft a
    block by diffusion and check it autoregressively over one shared KV cache).

    Reading: the token at the cache's next position is known (``first_token``, e.g. the causal prediction after
    the prompt).  Each round drafts a block by diffusion at the cache's end (generate_block with the commit
    deferred, block id block0 + round), puts the known token in slot 0 of the draft, and verifies the draft
    (verify_block): the accepted prefix is committed and output, and the causal pass's prediction for the first
    position not accepted becomes the next round's known token.  The rounds stop once n_tokens are out (the
    last round's surplus is dropped; its rows stay in the cache).  Every output token after the first is the
    causal model's greedy prediction after the ones before it, so the output equals greedy autoregressive
    decoding from ``first_token``; the drafts decide only how many tokens each causal pass confirms."""
    out: List[int] = []
    accepted: List[int] = []
    drafts: List[np.ndarray] = []
    nxt = int(first_token)
    r = 0
    while len(out) < n_tokens:
        res = generate_block(model, kv, s, block=block0 + r, do_commit=False)
        draft = res.tokens.copy()
        draft[0] = nxt
        v = verify_block(model, kv, draft)
        out.extend(int(t) for t in draft[:v.accepted])
        accepted.append(v.accepted)
        drafts.append(draft)
        nxt = v.next_token
        r += 1
    return SpeculativeResult(tokens=np.asarray(out[:n_tokens], dtype=np.int64), accepted=accepted, drafts=drafts)


def greedy_autoregressive(model: Model, kv: KVCache, first_token: int, n_tokens: int) -> np.ndarray:
    """Plain greedy decoding, one causal step per token: the first output is ``first_token`` at the cache's next
    position; each later one is the argmax of the head after the previous token's causal step."""
    out = [int(first_token)]
    while len(out) < n_tokens:
        x = model.embed([out[-1]])
        x, _ = model.body(x, kv, causal=True, append=True)
        out.append(int(model.head(x)[0][0]))
    return np.asarray(out, dtype=np.int64)
