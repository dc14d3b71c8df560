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
                 kv_capacity_round: int = 32):
        self.d = d
        self.cfg = dg.make_config(d)
        if weights is None:
            weights = gdev.model_weights_device(d)
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


def compare_routing(g_idx: np.ndarray, g_w: np.ndarray, o_idx: np.ndarray, o_w: np.ndarray, gap: np.ndarray,
                    gap_tol: float, w_tol: float = 1e-4) -> np.ndarray:
    """Routing parity.  The decision is the SET of chosen experts (order inside the top-k only fixes the
    summation order): sets must match exactly wherever the oracle's k-th/(k+1)-th logit gap is at least
    ``gap_tol``; where they match, each expert's weight must match.  Returns the mask of matching tokens."""
    gs = np.sort(g_idx, axis=1)
    os_ = np.sort(o_idx, axis=1)
    same = np.all(gs == os_, axis=1)
    bad = ~same & (gap >= gap_tol)
    assert not bad.any(), f"expert sets differ away from a near-tie: tokens {np.nonzero(bad)[0][:10]}, gaps {gap[bad][:10]}"
    for t in np.nonzero(same)[0]:
        go = np.argsort(g_idx[t])
        oo = np.argsort(o_idx[t])
        np.testing.assert_allclose(g_w[t][go], o_w[t][oo], atol=w_tol, rtol=w_tol)
    return same
