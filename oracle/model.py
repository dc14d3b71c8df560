"""The MoE transformer of one denoising pass, in float64 (test infrastructure only).

Page tags: [P1] "DiffusionGemma: When Text Generation Stops Being Sequential";
[P2] "DiffusionGemma 26B: How Google's Text Diffusion Model Generates Tokens in
Parallel"; [P3] "DiffusionGemma local text generation" (ctxwire);
[P5] "When to use a diffusion LLM: I compared DiffusionGemma and Gemma 4".

Readings taken where the pages are silent (each is listed with its reason in
the design notes): RMSNorm with eps 1e-6 and unit gains; no positional term;
attention scale 1/sqrt(head_dim); query head h reads KV head h*Hkv//Hq; router
logits in fp32, top-k with ties to the lower expert id, softmax over the k
chosen logits; shared expert added with weight 1; head tied to the embedding,
no embedding scaling and no logit soft-cap.

Weights arrive as float64 arrays holding exact storage values:
  embed [V, d], final_norm [d], and per layer
  attn_norm [d], wqkv [(Hq+2Hkv)*Dh, d] (query heads, then key heads, then
  value heads), wo [d, Hq*Dh], ffn_norm [d], w_router [E, d],
  w_gate_up [E, 2*fe, d] (gate rows then up rows), w_down [E, d, fe],
  ws_gate_up [2*fs, d], ws_down [d, fs].
Every matrix is [out, in]: y = x @ W.T.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from .numerics import f32, from_storage, rounder
from .numerics import round_e4m3_rows as e4m3_rows
from .philox import gumbel_noise


# ----------------------------------------------------------------------------- building blocks

def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal_offset: Optional[int] = None,
              q_pos: Optional[np.ndarray] = None) -> np.ndarray:
    """softmax(Q K^T / sqrt(Dh)) V per query head, GQA head grouping, fp64.

    q: [Hq, n, Dh]; k, v: [Hkv, m, Dh].  With ``causal_offset = P`` query i sits at
    absolute position P + i (or ``q_pos[i]`` when given) and sees keys up to its own
    position; with None every query sees every key — the bidirectional canvas
    attention of [P2] "How Diffusion Changes the Equation" and [P5] "How block
    diffusion works" (no mask inside the canvas).
    Returns [n, Hq*Dh] (token-major, heads concatenated).
    """
    hq, n, dh = q.shape
    hkv, m, _ = k.shape
    out = np.empty((n, hq, dh))
    if causal_offset is not None and q_pos is None:
        q_pos = causal_offset + np.arange(n)
    for h in range(hq):
        g = h * hkv // hq
        s = q[h] @ k[g].T / np.sqrt(dh)
        if causal_offset is not None:
            allowed = np.arange(m)[None, :] <= np.asarray(q_pos)[:, None]
            s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[g]
    return out.reshape(n, hq * dh)


def route(xn: np.ndarray, w_router: np.ndarray, top_k: int):
    """Top-k of 128-expert routing ([P2] "Architecture Details": 8 of 128 experts active plus one shared).

    Logits are formed in fp64 and rounded to fp32, the precision in which the
    kernel ranks them.  Ties go to the lower expert id (stable sort).  The weights
    are the softmax over the k chosen logits.  Returns (idx [n,k], w [n,k],
    logits32 [n,E], gap [n] = k-th minus (k+1)-th largest logit; inf if k == E).
    """
    r = f32(xn @ w_router.T)
    order = np.argsort(-r, axis=1, kind="stable")
    idx = order[:, :top_k]
    sel = np.take_along_axis(r, idx, axis=1)
    e = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = e / e.sum(axis=1, keepdims=True)
    if top_k < r.shape[1]:
        nxt = np.take_along_axis(r, order[:, top_k:top_k + 1], axis=1)[:, 0]
        gap = sel[:, -1] - nxt
    else:
        gap = np.full(r.shape[0], np.inf)
    return idx, w, r, gap


def swiglu_ffn(x: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray, rnd, s_gate_up=None,
               s_down=None) -> np.ndarray:
    """(silu(x Wg^T) * (x Wu^T)) Wd^T with the hidden product stored (rounded) before the down projection.

    With per-output-channel scales (FP8 weights: the matrices hold the E4M3 code values and row r of a matrix
    stands for s[r] times that row) each projection is multiplied by its channel's scale after the dot
    products: gate/up = (x Q^T) * s_gate_up, down = (h Q_d^T) * s_down."""
    f = w_gate_up.shape[0] // 2
    gu = x @ w_gate_up.T
    if s_gate_up is not None:
        gu = gu * s_gate_up
    h = rnd(silu(gu[:, :f]) * gu[:, f:])
    y = h @ w_down.T
    if s_down is not None:
        y = y * s_down
    return rnd(y)


def moe_routed(xn: np.ndarray, idx: np.ndarray, w: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray,
               rnd, s_gate_up=None, s_down=None) -> np.ndarray:
    """Sum over each token's k chosen experts of weight * expert output (expert output stored, then weighted).
    s_gate_up [E, 2F] / s_down [E, d]: per-output-channel scales of FP8 expert weights (None: plain weights)."""
    n, k = idx.shape
    out = np.zeros((n, w_down.shape[1]))
    for e in np.unique(idx):
        tok, slot = np.nonzero(idx == e)
        y = swiglu_ffn(xn[tok], w_gate_up[e], w_down[e], rnd, None if s_gate_up is None else s_gate_up[e],
                       None if s_down is None else s_down[e])
        np.add.at(out, tok, w[tok, slot][:, None] * y)
    return out


# ----------------------------------------------------------------------------- model

@dataclass
class Dims:
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    ffn_expert: int
    ffn_shared: int
    vocab: int
    canvas: int
    dtype: str
    rms_eps: float = 1e-6


@dataclass
class LayerTrace:
    """Per-layer diagnostics of one forward: routing and the residual stream after the layer."""
    idx: np.ndarray
    w: np.ndarray
    router_logits: np.ndarray
    gap: np.ndarray
    hidden: np.ndarray


class KVCache:
    """Per-layer key/value rows, float64 storage values: k[l], v[l] are [Hkv, len, Dh]."""

    def __init__(self, n_layers: int, n_kv_heads: int, head_dim: int):
        self.k = [np.zeros((n_kv_heads, 0, head_dim)) for _ in range(n_layers)]
        self.v = [np.zeros((n_kv_heads, 0, head_dim)) for _ in range(n_layers)]

    @property
    def length(self) -> int:
        return self.k[0].shape[1] if self.k else 0

    def append(self, layer: int, k_new: np.ndarray, v_new: np.ndarray) -> None:
        self.k[layer] = np.concatenate([self.k[layer], k_new], axis=1)
        self.v[layer] = np.concatenate([self.v[layer], v_new], axis=1)

    def truncate(self, length: int) -> None:
        """Keep rows [0, length) of every layer."""
        self.k = [k[:, :length] for k in self.k]
        self.v = [v[:, :length] for v in self.v]


def weights_to_f64(storage: dict, dtype: str) -> dict:
    """Convert a storage-form weight dict (as produced by the input generator) to float64 values."""
    out = {}
    for key, val in storage.items():
        if key == "layers":
            out[key] = [{n: from_storage(a, dtype) for n, a in layer.items()} for layer in val]
        else:
            out[key] = from_storage(val, dtype)
    return out


EXPERT_MATRICES = ("w_gate_up", "w_down")


def fp8_expert_layer(layer: dict) -> dict:
    """A float64 layer dict with its routed experts' matrices quantised to E4M3 with per-output-channel scales:
    w_gate_up / w_down become the E4M3 values and w_gate_up_scale [E, 2F] / w_down_scale [E, d] their scales
    (numerics.round_e4m3_rows; the other tensors are unchanged)."""
    out = dict(layer)
    for n in EXPERT_MATRICES:
        values, scales = e4m3_rows(layer[n])
        out[n] = values
        out[n + "_scale"] = scales.astype(np.float64)
    return out


def fp8_embed(weights: dict) -> dict:
    """A float64 weight dict whose tied embedding is quantised to E4M3 with one scale per vocabulary row
    (numerics.round_e4m3_rows): "embed" becomes the dequantised matrix value * scale, which both the lookup
    (rounded to the storage type there) and the head read; the other tensors are unchanged."""
    out = dict(weights)
    values, scales = e4m3_rows(weights["embed"])
    out["embed"] = values * scales.astype(np.float64)[:, None]
    return out


class Model:
    """The denoiser: embedding, n_layers MoE blocks, final norm, tied vocab head."""

    def __init__(self, dims: Dims, weights: dict):
        self.d = dims
        self.w = weights
        self.rnd = rounder(dims.dtype)

    # one transformer block -------------------------------------------------
    def layer(self, l: int, x: np.ndarray, kv: KVCache, causal: bool, append: bool):
        """One block over n rows at cache positions kv.length .. kv.length+n-1.

        The new rows' keys/values join the cached ones for this layer's attention; with
        ``append`` they are also written to the cache (prefill/commit), otherwise they
        are scratch for this pass only (denoising pass).
        """
        d, w, rnd = self.d, self.w["layers"][l], self.rnd
        hq, hkv, dh = d.n_heads, d.n_kv_heads, d.head_dim
        n = x.shape[0]
        p0 = kv.k[l].shape[1]
        xn = rnd(rmsnorm(x, w["attn_norm"], d.rms_eps))
        qkv = xn @ w["wqkv"].T
        q = rnd(qkv[:, :hq * dh]).reshape(n, hq, dh).transpose(1, 0, 2)
        k = rnd(qkv[:, hq * dh:(hq + hkv) * dh]).reshape(n, hkv, dh).transpose(1, 0, 2)
        v = rnd(qkv[:, (hq + hkv) * dh:]).reshape(n, hkv, dh).transpose(1, 0, 2)
        k_all = np.concatenate([kv.k[l], k], axis=1)
        v_all = np.concatenate([kv.v[l], v], axis=1)
        o = rnd(attention(q, k_all, v_all, causal_offset=p0 if causal else None))
        x = rnd(x + o @ w["wo"].T)
        xn2 = rnd(rmsnorm(x, w["ffn_norm"], d.rms_eps))
        idx, rw, rlog, gap = route(xn2, w["w_router"], d.top_k)
        y = moe_routed(xn2, idx, rw, w["w_gate_up"], w["w_down"], rnd, w.get("w_gate_up_scale"),
                       w.get("w_down_scale"))
        ys = swiglu_ffn(xn2, w["ws_gate_up"], w["ws_down"], rnd)
        x = rnd(x + ys + y)
        if append:
            kv.append(l, k, v)
        return x, LayerTrace(idx=idx, w=rw, router_logits=rlog, gap=gap, hidden=x)

    def layer_rows(self, l: int, x: np.ndarray, kv: KVCache, causal: bool, rows: np.ndarray, return_kv=False):
        """``layer(l, x, kv, causal, append=False)`` evaluated for the rows ``rows`` only.

        Every row's keys and values are still formed (all of them take part in the
        attention of the rows asked for); everything after the attention is per row.
        Returns (x_out[rows], LayerTrace of those rows), and with ``return_kv`` also the
        keys and values of all the new rows ([Hkv, n, Dh] each, as the layer stores them)."""
        d, w, rnd = self.d, self.w["layers"][l], self.rnd
        hq, hkv, dh = d.n_heads, d.n_kv_heads, d.head_dim
        rows = np.asarray(rows, dtype=np.int64)
        n = x.shape[0]
        p0 = kv.k[l].shape[1]
        xn = rnd(rmsnorm(x, w["attn_norm"], d.rms_eps))
        kvp = xn @ w["wqkv"][hq * dh:].T
        k = rnd(kvp[:, :hkv * dh]).reshape(n, hkv, dh).transpose(1, 0, 2)
        v = rnd(kvp[:, hkv * dh:]).reshape(n, hkv, dh).transpose(1, 0, 2)
        q = rnd(xn[rows] @ w["wqkv"][:hq * dh].T).reshape(len(rows), hq, dh).transpose(1, 0, 2)
        k_all = np.concatenate([kv.k[l], k], axis=1)
        v_all = np.concatenate([kv.v[l], v], axis=1)
        o = rnd(attention(q, k_all, v_all, causal_offset=p0 if causal else None,
                          q_pos=(p0 + rows) if causal else None))
        xr = rnd(x[rows] + o @ w["wo"].T)
        xn2 = rnd(rmsnorm(xr, w["ffn_norm"], d.rms_eps))
        idx, rw, rlog, gap = route(xn2, w["w_router"], d.top_k)
        y = moe_routed(xn2, idx, rw, w["w_gate_up"], w["w_down"], rnd, w.get("w_gate_up_scale"),
                       w.get("w_down_scale"))
        ys = swiglu_ffn(xn2, w["ws_gate_up"], w["ws_down"], rnd)
        xr = rnd(xr + ys + y)
        tr = LayerTrace(idx=idx, w=rw, router_logits=rlog, gap=gap, hidden=xr)
        if return_kv:
            return xr, tr, k, v
        return xr, tr

    def embed(self, tokens) -> np.ndarray:
        """Rows of the tied embedding, in the storage type (exact for stored rows; a dequantised FP8 row
        code * scale is rounded there)."""
        return self.rnd(self.w["embed"][np.asarray(tokens, dtype=np.int64)])

    def body(self, x: np.ndarray, kv: KVCache, causal: bool, append: bool):
        traces: List[LayerTrace] = []
        for l in range(self.d.n_layers):
            x, tr = self.layer(l, x, kv, causal, append)
            traces.append(tr)
        return x, traces

    def head(self, x: np.ndarray, inv_temperature: float = 1.0, gumbel=None):
        return head_stats(x, self.w["final_norm"], self.w["embed"], inv_temperature, self.d.rms_eps, self.rnd,
                          gumbel=gumbel)


def head_stats(x: np.ndarray, g_final: np.ndarray, embed: np.ndarray, inv_temperature: float, eps: float, rnd,
               chunk: int = 64, gumbel=None, slots=None):
    """Final norm, tied vocab projection and per-slot softmax statistics.

    logits = beta * (rms(x) * g) E^T; pred = argmax (fp32 logits, ties to the lowest
    id); p = softmax(logits) (max subtracted, then exp and normalise);
    conf = max_v p (the confidence the keep rule ranks by, [P5] "How block diffusion
    works"); ent = -sum_v p ln p in nats, 0 ln 0 = 0 (the entropy the stop rule averages,
    [P2] "How Diffusion Changes the Equation").  Also returns the fp32 top-2 logit
    margin of each slot.

    gumbel = (seed, block, step) samples instead of taking the argmax (the recommended
    sampler's temperature, [P2] "Architecture Details"): pred = argmax of the fp32
    perturbed score logits + G, G from oracle.philox.gumbel_noise with row i as slot i
    (or as slot slots[i]; ties to the lowest id); conf = p[pred], the probability of the token drawn; the
    margin is then the top-2 gap of the perturbed scores.  The entropy is unchanged.
    """
    xf = rnd(rmsnorm(x, g_final, eps))
    n = xf.shape[0]
    pred = np.empty(n, dtype=np.int64)
    conf = np.empty(n)
    ent = np.empty(n)
    margin = np.empty(n)
    for s0 in range(0, n, chunk):
        lg = inv_temperature * (xf[s0:s0 + chunk] @ embed.T)
        score = lg
        if gumbel is not None:
            seed, block, step = gumbel
            rows = np.arange(s0, s0 + lg.shape[0]) if slots is None else np.asarray(slots)[s0:s0 + lg.shape[0]]
            score = lg + gumbel_noise(seed, block, step, rows, lg.shape[1])
        l32 = f32(score)
        choice = np.argmax(l32, axis=1)
        pred[s0:s0 + chunk] = choice
        top2 = -np.partition(-l32, 1, axis=1)[:, :2]
        margin[s0:s0 + chunk] = top2[:, 0] - top2[:, 1]
        m = lg.max(axis=1, keepdims=True)
        e = np.exp(lg - m)
        p = e / e.sum(axis=1, keepdims=True)
        conf[s0:s0 + chunk] = p.max(axis=1) if gumbel is None else p[np.arange(p.shape[0]), choice]
        with np.errstate(divide="ignore", invalid="ignore"):
            plogp = np.where(p > 0, p * np.log(p), 0.0)
        ent[s0:s0 + chunk] = -plogp.sum(axis=1)
    return pred, conf, ent, margin
