"""GPU-side test helpers: device weights, KV caches and workspaces for the libdg calls."""
from __future__ import annotations

import numpy as np
import torch

import block_diffusion_decoding_step_amd as dg
from dg_inputs import device as gdev
from dg_inputs import recipe


class Session:
    """Device model + KV cache + workspace for one set of dimensions."""

    def __init__(self, d: recipe.Dims, capacity: int, max_tokens: int = None, weights: dict = None,
                 kv_capacity_round: int = 32, packed: bool = False):
        """weights: natural (row-major) device weights, converted here unless packed=True; None builds the
        seeded model directly in the library's layout."""
        self.d = d
        self.cfg = dg.make_config(d)
        if weights is None:
            weights = gdev.packed_model_weights_device(d)
        elif not packed:
            weights = dg.pack_weights(weights)
        self.w = weights
        self.weights = dg.Weights(weights["embed"], weights["final_norm"], weights["layers"])
        cap = ((capacity + kv_capacity_round - 1) // kv_capacity_round) * kv_capacity_round
        self.k, self.v = gdev.kv_tensors(d, cap)
        self.kv = dg.KV(self.k, self.v, cap, 0)
        mt = max_tokens or d.canvas
        self.ws_bytes = dg.dg_workspace_size(self.cfg, mt)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.S = d.canvas

    def i32(self, n):
        return torch.empty(n, dtype=torch.int32, device="cuda")

    def f32(self, n):
        return torch.empty(n, dtype=torch.float32, device="cuda")

    def prefill(self, tokens: np.ndarray):
        t = torch.from_numpy(np.asarray(tokens, dtype=np.int32)).cuda()
        dg.dg_prefill_kv(self.cfg, self.weights, self.kv, t, len(tokens), self.ws, self.ws_bytes)

    def denoise(self, canvas, dbg=None, inv_temperature=1.0):
        c = canvas if torch.is_tensor(canvas) else torch.from_numpy(np.asarray(canvas, dtype=np.int32)).cuda()
        pred, conf, ent = self.i32(self.S), self.f32(self.S), self.f32(self.S)
        dg.dg_denoise_step(self.cfg, self.weights, self.kv, c, inv_temperature, pred, conf, ent, dbg, self.ws,
                           self.ws_bytes)
        return pred, conf, ent

    def kv_numpy(self, layer: int, length: int):
        """(K [Hkv, len, Dh], V [Hkv, len, Dh]) of one layer as float64."""
        k = self.k[layer, :, :length, :].float().cpu().numpy().astype(np.float64)
        v = self.v[layer, :, :, :length].float().cpu().numpy().astype(np.float64).transpose(0, 2, 1)
        return k, v


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def allclose_report(got: np.ndarray, ref: np.ndarray, atol: float, rtol: float):
    """(ok, worst excess, index) for |got - ref| <= atol + rtol |ref|."""
    err = np.abs(got - ref) - (atol + rtol * np.abs(ref))
    i = int(np.argmax(err))
    return bool(err.max() <= 0), float(err.flat[i]), np.unravel_index(i, got.shape)


def compare_routing(g_idx: np.ndarray, g_w: np.ndarray, g_logits: np.ndarray, o_logits: np.ndarray,
                    o_idx: np.ndarray, logit_tol, rows=None) -> np.ndarray:
    """Routing parity in three parts.

    1. The GPU's decision is exact on its own logits: its expert list is the top-k of its fp32 logits in
       (logit descending, expert ascending) order, bit for bit, and its weights are the softmax of those k.
    2. Its logits match the oracle's within ``logit_tol`` = (atol, rtol).
    3. The chosen SET matches the oracle's wherever the oracle's k-th/(k+1)-th gap exceeds twice the
       token's largest logit difference (otherwise the two sides legitimately sit on either side of a tie).
    ``rows`` (optional mask): parts 2 and 3 only on these rows (rows whose inputs already diverged at an
    earlier near-tie are not comparable).  Returns the mask of compared tokens whose sets match.
    """
    n, k = g_idx.shape
    E = g_logits.shape[1]
    order = np.lexsort((np.broadcast_to(np.arange(E), g_logits.shape), -g_logits.astype(np.float64)), axis=1)
    assert np.array_equal(order[:, :k], g_idx), "GPU top-k is not the top-k of its own logits"
    sel = np.take_along_axis(g_logits.astype(np.float64), g_idx, axis=1)
    ex = np.exp(sel - sel[:, :1])
    np.testing.assert_allclose(g_w, ex / ex.sum(axis=1, keepdims=True), rtol=1e-5, atol=1e-6)
    atol, rtol = logit_tol
    if rows is not None:
        g_idx, g_logits, o_logits, o_idx = g_idx[rows], g_logits[rows], o_logits[rows], o_idx[rows]
        n = int(np.sum(rows))
    diff = np.abs(g_logits.astype(np.float64) - o_logits)
    assert np.all(diff <= atol + rtol * np.abs(o_logits)), f"router logits differ by up to {diff.max():.3e}"
    srt = -np.sort(-o_logits, axis=1)
    gap = srt[:, k - 1] - srt[:, k] if k < E else np.full(n, np.inf)
    same = np.all(np.sort(g_idx, axis=1) == np.sort(o_idx, axis=1), axis=1)
    bad = ~same & (gap > 2 * diff.max(axis=1))
    assert not bad.any(), f"expert sets differ away from a tie: tokens {np.nonzero(bad)[0][:10]}"
    if rows is not None:
        full = np.zeros(rows.shape[0], dtype=bool)
        full[np.nonzero(rows)[0]] = same
        return full
    return same
