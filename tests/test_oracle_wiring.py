"""Pins of the oracle's layer wiring, its canvas-token mapping and its SiLU.

The layer is a composition of parts that are each pinned elsewhere (attention,
routing, MoE, RMSNorm).  What those pins cannot see is how the parts are wired
together: which residual each norm reads, which rows feed the shared expert, and
whether the FFN input carries the attention output.  The tests below choose
weights for which the layer has a closed form, computed here with plain Python
loops that share nothing with the oracle's vectorised code, and use different
attention and FFN norm gains so that a swap shows.

Each test names the mistakes it catches.  Architecture: 8 routed experts of 128
plus one shared expert per layer ([P2] "DiffusionGemma 26B: How Google's Text
Diffusion Model Generates Tokens in Parallel", "Architecture Details"); pre-norm
blocks with residual adds (the plainest reading where the pages are silent).
"""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import model as om
from oracle import numerics, philox

# ----------------------------------------------------------------------------- plain-loop building blocks


def _rms_row(x, g, eps):
    ms = sum(v * v for v in x) / len(x)
    s = 1.0 / math.sqrt(ms + eps)
    return [v * s * gi for v, gi in zip(x, g)]


def _matvec(W, x):
    """W [out][in] times x [in] with Python floats."""
    return [sum(wij * xj for wij, xj in zip(row, x)) for row in W]


def _logistic(z):
    return 1.0 / (1.0 + math.exp(-z))


def _ffn_row(x, w_gate_up, w_down, rnd):
    """SwiGLU of one row: (z_g * logistic(z_g) * z_u) projected down; the hidden product is stored (rnd)."""
    f = len(w_gate_up) // 2
    z = _matvec(w_gate_up, x)
    h = [rnd(z[i] * _logistic(z[i]) * z[f + i]) for i in range(f)]
    return [rnd(v) for v in _matvec(w_down, h)]


def _scalar_rnd(dtype):
    if dtype == "bf16":
        return lambda v: float(numerics.bf16_round(np.array([v]))[0])
    return lambda v: float(v)


DIMS = dict(n_layers=1, d_model=16, n_heads=4, n_kv_heads=2, head_dim=8, n_experts=4, top_k=2, ffn_expert=6,
            ffn_shared=6, vocab=32, canvas=5)


def _weights(dtype, seed):
    """Random small weights (storage values of the dtype), distinct attention and FFN norm gains."""
    rng = np.random.default_rng(seed)
    rnd = numerics.rounder(dtype)
    d, hq, hkv, dh = DIMS["d_model"], DIMS["n_heads"], DIMS["n_kv_heads"], DIMS["head_dim"]
    E, fe, fs = DIMS["n_experts"], DIMS["ffn_expert"], DIMS["ffn_shared"]
    lw = {
        "attn_norm": rnd(rng.uniform(0.5, 1.5, size=d)),
        "wqkv": rnd(rng.normal(size=((hq + 2 * hkv) * dh, d)) * 0.3),
        "wo": rnd(rng.normal(size=(d, hq * dh)) * 0.3),
        "ffn_norm": rnd(rng.uniform(1.6, 2.6, size=d)),
        "w_router": rnd(rng.normal(size=(E, d))),
        "w_gate_up": rnd(rng.normal(size=(E, 2 * fe, d)) * 0.3),
        "w_down": rnd(rng.normal(size=(E, d, fe)) * 0.3),
        "ws_gate_up": rnd(rng.normal(size=(2 * fs, d)) * 0.3),
        "ws_down": rnd(rng.normal(size=(d, fs)) * 0.3),
    }
    assert np.all(np.abs(lw["attn_norm"] - lw["ffn_norm"]) > 0.05)
    return lw


def _model(dtype, lw):
    dims = om.Dims(dtype=dtype, **DIMS)
    return om.Model(dims, {"embed": None, "final_norm": None, "layers": [lw]})


def _cache(dtype, seed, length):
    rng = np.random.default_rng(seed)
    rnd = numerics.rounder(dtype)
    kv = om.KVCache(1, DIMS["n_kv_heads"], DIMS["head_dim"])
    kv.k[0] = rnd(rng.normal(size=(DIMS["n_kv_heads"], length, DIMS["head_dim"])))
    kv.v[0] = rnd(rng.normal(size=(DIMS["n_kv_heads"], length, DIMS["head_dim"])))
    return kv


def _mean_value_attention(x_rows, lw, kv, rnd, eps):
    """Attention output of every row when W_q = 0: all scores are equal, so each query head returns the mean of
    its KV head's values over the visible keys (cache rows, then the new rows' own values, no mask)."""
    hq, hkv, dh = DIMS["n_heads"], DIMS["n_kv_heads"], DIMS["head_dim"]
    wv = lw["wqkv"][(hq + hkv) * dh:]
    vals = [[[float(v) for v in kv.v[0][g, j]] for j in range(kv.v[0].shape[1])] for g in range(hkv)]
    for x in x_rows:
        xn = [rnd(v) for v in _rms_row(x, lw["attn_norm"], eps)]
        vrow = [rnd(v) for v in _matvec(wv, xn)]
        for g in range(hkv):
            vals[g].append(vrow[g * dh:(g + 1) * dh])
    o = []
    for h in range(hq):
        g = h * hkv // hq
        n = len(vals[g])
        o += [rnd(sum(vals[g][j][c] for j in range(n)) / n) for c in range(dh)]
    return o  # identical for every row


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_identical_experts_without_attention(dtype):
    """W_o = 0 and every routed expert equal to the shared expert: the layer is
    x + 2 FFN(rms(x) g_ffn), each FFN output stored at the storage precision.

    Catches: the shared expert fed x or the attention-normed rows, the FFN norm
    using the attention gain (norms swapped), a shared-expert weight other than 1,
    the routed weights not summing to one, a missing residual."""
    lw = _weights(dtype, 11)
    lw["wo"] = np.zeros_like(lw["wo"])
    lw["w_gate_up"] = np.broadcast_to(lw["ws_gate_up"], lw["w_gate_up"].shape).copy()
    lw["w_down"] = np.broadcast_to(lw["ws_down"], lw["w_down"].shape).copy()
    m = _model(dtype, lw)
    rnd = _scalar_rnd(dtype)
    rng = np.random.default_rng(12)
    x = numerics.rounder(dtype)(rng.normal(size=(DIMS["canvas"], DIMS["d_model"])) * 2.0)
    kv = _cache(dtype, 13, 3)
    got, _ = m.layer(0, x, kv, causal=False, append=False)
    eps = 1e-6
    for i in range(x.shape[0]):
        xr = [float(v) for v in x[i]]
        xn = [rnd(v) for v in _rms_row(xr, lw["ffn_norm"], eps)]
        y = _ffn_row(xn, lw["ws_gate_up"].tolist(), lw["ws_down"].tolist(), rnd)
        want = [rnd(a + 2.0 * b) for a, b in zip(xr, y)]
        # bf16: the routed sum is y * (w_1 + w_2), one fp64 rounding away from y
        np.testing.assert_allclose(got[i], want, rtol=1e-12 if dtype == "f32" else 2 ** -8, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_mean_value_attention_without_ffn(dtype):
    """W_q = 0 (uniform attention) and every FFN down projection zero: the layer is x + mean(V) W_o^T, where V
    holds the cache values and the canvas rows' own values rms(x) g_attn W_v^T (no mask in a canvas pass).

    Catches: attention on un-normed rows, the attention norm using the FFN gain, the canvas rows' keys/values
    left out of the attention, a transposed W_o, a missing residual."""
    lw = _weights(dtype, 21)
    hq, dh = DIMS["n_heads"], DIMS["head_dim"]
    lw["wqkv"][:hq * dh] = 0.0
    lw["w_down"] = np.zeros_like(lw["w_down"])
    lw["ws_down"] = np.zeros_like(lw["ws_down"])
    m = _model(dtype, lw)
    rnd = _scalar_rnd(dtype)
    rng = np.random.default_rng(22)
    x = numerics.rounder(dtype)(rng.normal(size=(DIMS["canvas"], DIMS["d_model"])) * 2.0)
    kv = _cache(dtype, 23, 4)
    got, _ = m.layer(0, x, kv, causal=False, append=False)
    o = _mean_value_attention([[float(v) for v in r] for r in x], lw, kv, rnd, 1e-6)
    ao = _matvec(lw["wo"].tolist(), o)
    for i in range(x.shape[0]):
        want = [rnd(rnd(float(a) + b)) for a, b in zip(x[i], ao)]
        np.testing.assert_allclose(got[i], want, rtol=1e-12, atol=1e-12)


def test_layer_ffn_reads_attention_residual():
    """W_q = 0 (uniform attention) and every routed expert equal to the shared expert: the layer is
    h + 2 FFN(rms(h) g_ffn) with h = x + mean(V) W_o^T (fp32 workload, no rounding).

    Catches: the FFN (routed or shared) reading the block input x instead of the residual after attention, and
    every wiring mistake of the two tests above at once."""
    dtype = "f32"
    lw = _weights(dtype, 31)
    hq, dh = DIMS["n_heads"], DIMS["head_dim"]
    lw["wqkv"][:hq * dh] = 0.0
    lw["w_gate_up"] = np.broadcast_to(lw["ws_gate_up"], lw["w_gate_up"].shape).copy()
    lw["w_down"] = np.broadcast_to(lw["ws_down"], lw["w_down"].shape).copy()
    m = _model(dtype, lw)
    rnd = _scalar_rnd(dtype)
    rng = np.random.default_rng(32)
    x = rng.normal(size=(DIMS["canvas"], DIMS["d_model"]))
    kv = _cache(dtype, 33, 2)
    got, _ = m.layer(0, x, kv, causal=False, append=False)
    o = _mean_value_attention([[float(v) for v in r] for r in x], lw, kv, rnd, 1e-6)
    ao = _matvec(lw["wo"].tolist(), o)
    for i in range(x.shape[0]):
        h = [float(a) + b for a, b in zip(x[i], ao)]
        hn = _rms_row(h, lw["ffn_norm"], 1e-6)
        y = _ffn_row(hn, lw["ws_gate_up"].tolist(), lw["ws_down"].tolist(), rnd)
        want = [a + 2.0 * b for a, b in zip(h, y)]
        np.testing.assert_allclose(got[i], want, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- canvas token mapping

def test_uniform_token_of_the_all_zero_counter():
    """U(seed 0, block 0, step 0, slot 0) is word 0 of Philox4x32-10 at the all-zero counter and key, whose
    published value is 0x6627e8d5 (Random123 known-answer vector), mapped to [0, V) by the multiply-shift
    floor(w V / 2^32): 104607 for V = 262144 and 1634 for V = 4096.

    Catches: the remainder w mod V instead of the multiply-shift (256213 and 3285 here), another output word,
    the counter's slot and step words swapped into a non-zero position."""
    w0 = 0x6627E8D5
    assert (w0 * 262144) >> 32 == 104607 and (w0 * 4096) >> 32 == 1634
    assert int(philox.uniform_tokens(0, 0, 0, [0], 262144)[0]) == 104607
    assert int(philox.uniform_tokens(0, 0, 0, [0], 4096)[0]) == 1634
    assert w0 % 262144 != 104607 and w0 % 4096 != 1634


# ----------------------------------------------------------------------------- SiLU

def test_silu_values():
    """silu(z) = z / (1 + e^-z): silu(1) = 1/(1 + 1/e) = 0.7310585786..., silu(-1) = -1/(1 + e) =
    -0.2689414213..., silu(0) = 0, and silu(z) -> z for large z, -> 0 for very negative z.

    Catches: z tanh(z), the logistic alone, a sign error in the exponent."""
    got = om.silu(np.array([1.0, -1.0, 0.0, 40.0, -40.0]))
    np.testing.assert_allclose(got[:2], [0.7310585786300049, -0.2689414213699951], rtol=1e-15)
    assert got[2] == 0.0
    np.testing.assert_allclose(got[3], 40.0, rtol=1e-15)
    assert abs(got[4]) < 1e-15
