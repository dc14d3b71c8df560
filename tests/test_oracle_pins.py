"""Pins of the CPU oracle against closed forms, invariants, published vectors and brute force.

None of these tests imports the HIP path.  Each test names the plausible oracle
mistake it would catch.
"""
from __future__ import annotations

import itertools
from dataclasses import replace
import json
import math
import os

import numpy as np
import pytest

import dg_inputs
from dg_inputs import recipe
from oracle import model as om
from oracle import numerics, philox
from oracle import sampler as osm
from tests._helpers import oracle_dims, oracle_model, small_dims

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- bf16 rounding

def test_bf16_round_exhaustive_ties_and_neighbours():
    """Every finite positive bf16 value v and its successor v': the midpoint rounds to the even one,
    a hair either side rounds to the nearer one (catches truncation or round-half-up)."""
    bits = np.arange(0x0080, 0x7F7F, dtype=np.uint32)  # positive normal bf16, excluding the largest
    v = numerics.from_bf16_bits(bits)
    vn = numerics.from_bf16_bits(bits + 1)
    mid = (v + vn) / 2
    even = np.where(bits % 2 == 0, v, vn)
    assert np.array_equal(numerics.bf16_round(mid), even)
    eps = (vn - v) * 1e-6
    assert np.array_equal(numerics.bf16_round(mid - eps), v)
    assert np.array_equal(numerics.bf16_round(mid + eps), vn)
    assert np.array_equal(numerics.bf16_round(-mid), -even)
    assert np.array_equal(numerics.bf16_round(v), v)


def test_bf16_round_matches_generator_rounding():
    """The input generator's fp32->bf16 rounding and the oracle's fp64->bf16 rounding agree on fp32 values."""
    x = dg_inputs.normal((20000,), 7, 3, 1.0, "f32").astype(np.float64)
    bits = dg_inputs.const(x.shape, 0.0, "bf16")  # placeholder for shape
    u = x.astype(np.float32).view(np.uint32)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(numerics.from_bf16_bits(bits), numerics.bf16_round(x))


# ----------------------------------------------------------------------------- Philox

def _kat_rows():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            w = [int(t, 16) for t in line.split()]
            rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


@pytest.mark.parametrize("ctr,key,expect", _kat_rows())
def test_philox_known_answers(ctr, key, expect):
    """Published Philox4x32-10 known-answer vectors (catches a wrong constant, round count or word order)."""
    out = philox.philox4x32_10([np.array([c], dtype=np.uint64) for c in ctr], key)
    assert [int(o[0]) for o in out] == expect


def test_uniform_tokens_range_and_uniformity():
    """Draws lie in [0, V) and are uniform (chi-square), and distinct counters give distinct draws."""
    V = 4096
    n = 200_000
    t = philox.uniform_tokens(1, 0, 0, np.arange(n), V)
    assert t.min() >= 0 and t.max() < V
    counts = np.bincount(t, minlength=V)
    chi2 = ((counts - n / V) ** 2 / (n / V)).sum()
    # chi-square with V-1 dof: mean 4095, sd ~ 90.5; 6 sd band
    assert abs(chi2 - (V - 1)) < 6 * math.sqrt(2 * (V - 1))
    a = philox.uniform_tokens(1, 0, 1, np.arange(64), 1 << 30)
    b = philox.uniform_tokens(1, 0, 2, np.arange(64), 1 << 30)
    c = philox.uniform_tokens(1, 1, 1, np.arange(64), 1 << 30)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


# ----------------------------------------------------------------------------- head statistics

def _head_direct(logits):
    """Textbook per-row softmax statistics with Python floats (independent of numpy vectorisation)."""
    out = []
    for row in logits:
        m = max(row)
        e = [math.exp(v - m) for v in row]
        z = sum(e)
        p = [x / z for x in e]
        ent = -sum(q * math.log(q) for q in p if q > 0)
        best = max(range(len(row)), key=lambda i: (row[i], -i))
        out.append((best, max(p), ent))
    return out


def test_head_uniform_logits():
    """E = 0: every logit is 0 -> entropy exactly ln V, confidence 1/V, prediction token 0."""
    V, d = 4096, 16
    x = np.random.default_rng(0).normal(size=(5, d))
    pred, conf, ent, _ = om.head_stats(x, np.ones(d), np.zeros((V, d)), 1.0, 1e-6, lambda a: a)
    assert np.all(pred == 0)
    np.testing.assert_allclose(ent, math.log(V), rtol=0, atol=1e-12)
    np.testing.assert_allclose(conf, 1.0 / V, rtol=1e-12)


def test_head_two_level_closed_form():
    """One logit a, the rest 0: Z = e^a + V - 1, conf = e^a/Z, ent = ln Z - a e^a / Z."""
    V, d = 1000, 2
    for a, vstar in [(3.0, 17), (-2.0, 999), (12.0, 0)]:
        E = np.zeros((V, d))
        E[vstar] = [a / 2, a / 2]
        x = np.array([[1.0, 1.0]])
        pred, conf, ent, _ = om.head_stats(x, np.ones(d), E, 1.0, 0.0, lambda t: t)
        Z = math.exp(a) + V - 1
        assert abs(conf[0] - max(math.exp(a), 1.0) / Z) < 1e-12
        assert abs(ent[0] - (math.log(Z) - a * math.exp(a) / Z)) < 1e-12
        assert pred[0] == (vstar if a > 0 else (0 if vstar != 0 else 1))


def test_head_matches_textbook_loop_and_bounds():
    rng = np.random.default_rng(3)
    V, d = 300, 8
    E = rng.normal(size=(V, d))
    x = rng.normal(size=(6, d))
    beta = 0.7
    pred, conf, ent, margin = om.head_stats(x, np.ones(d), E, beta, 1e-6, lambda t: t)
    xf = om.rmsnorm(x, np.ones(d), 1e-6)
    logits = beta * (xf @ E.T)
    for i, (b, c, h) in enumerate(_head_direct(logits.tolist())):
        assert pred[i] == b
        assert abs(conf[i] - c) < 1e-12 and abs(ent[i] - h) < 1e-12
    assert np.all(ent >= 0) and np.all(ent <= math.log(V) + 1e-12)
    assert np.all(margin >= 0)


def test_head_argmax_ties_lowest_id():
    V, d = 50, 2
    E = np.zeros((V, d))
    E[7] = [1.0, 1.0]
    E[31] = [1.0, 1.0]
    pred, _, _, margin = om.head_stats(np.array([[1.0, 1.0]]), np.ones(d), E, 1.0, 0.0, lambda t: t)
    assert pred[0] == 7 and margin[0] == 0.0


# ----------------------------------------------------------------------------- attention

def _attn_loops(q, k, v, causal_offset=None):
    hq, n, dh = q.shape
    hkv, m, _ = k.shape
    out = np.zeros((n, hq * dh))
    grp = hq // hkv
    for h in range(hq):
        g = h // grp
        for i in range(n):
            keys = [j for j in range(m) if causal_offset is None or j <= causal_offset + i]
            s = [sum(q[h, i, t] * k[g, j, t] for t in range(dh)) / math.sqrt(dh) for j in keys]
            mx = max(s)
            e = [math.exp(z - mx) for z in s]
            z = sum(e)
            for t in range(dh):
                out[i, h * dh + t] = sum(e[a] * v[g, keys[a], t] for a in range(len(keys))) / z
    return out


@pytest.mark.parametrize("causal", [None, 3])
def test_attention_brute_force(causal):
    rng = np.random.default_rng(1)
    q = rng.normal(size=(4, 5, 3))
    k = rng.normal(size=(2, 9, 3))
    v = rng.normal(size=(2, 9, 3))
    got = om.attention(q, k, v, causal)
    np.testing.assert_allclose(got, _attn_loops(q, k, v, causal), rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(2)
    q = rng.normal(size=(4, 6, 8))
    v = rng.normal(size=(2, 1, 8))
    k = rng.normal(size=(2, 1, 8))
    out = om.attention(q, k, v).reshape(6, 4, 8)
    for h in range(4):
        np.testing.assert_allclose(out[:, h], np.broadcast_to(v[h // 2, 0], (6, 8)), atol=1e-14)
    # identical keys -> plain mean of the values
    k = np.broadcast_to(rng.normal(size=(2, 1, 8)), (2, 11, 8)).copy()
    v = rng.normal(size=(2, 11, 8))
    out = om.attention(q, k, v).reshape(6, 4, 8)
    for h in range(4):
        np.testing.assert_allclose(out[:, h], np.broadcast_to(v[h // 2].mean(axis=0), (6, 8)), atol=1e-12)
    # causal, first query at offset 0 sees only key 0
    out = om.attention(q, rng.normal(size=(2, 6, 8)), v[:, :6], causal_offset=0).reshape(6, 4, 8)
    for h in range(4):
        np.testing.assert_allclose(out[0, h], v[h // 2, 0], atol=1e-14)


def test_attention_explicit_query_positions():
    """Queries given by explicit positions equal the same rows of the consecutive-position call (catches a
    mask built from row numbers instead of positions)."""
    rng = np.random.default_rng(5)
    q = rng.normal(size=(4, 7, 3))
    k = rng.normal(size=(2, 12, 3))
    v = rng.normal(size=(2, 12, 3))
    full = om.attention(q, k, v, causal_offset=5)
    rows = np.array([6, 0, 3])
    sub = om.attention(q[:, rows], k, v, causal_offset=5, q_pos=5 + rows)
    np.testing.assert_allclose(sub, full[rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sub, _attn_loops(q, k, v, 5)[rows], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_layer_rows_equals_full_layer(causal):
    """The row-subset layer used for long-context sampling equals the full layer on those rows."""
    dd = small_dims(dtype="bf16")
    d = oracle_dims(dd)
    m = oracle_model(dd)
    kv = om.KVCache(1, d.n_kv_heads, d.head_dim)
    rng = np.random.default_rng(6)
    kv.k[0] = numerics.bf16_round(rng.normal(size=(d.n_kv_heads, 9, d.head_dim)))
    kv.v[0] = numerics.bf16_round(rng.normal(size=(d.n_kv_heads, 9, d.head_dim)))
    x = numerics.bf16_round(rng.normal(size=(10, d.d_model)))
    full, trf = m.layer(0, x, kv, causal, append=False)
    rows = np.array([9, 2, 5])
    sub, trs = m.layer_rows(0, x, kv, causal, rows)
    np.testing.assert_allclose(sub, full[rows], rtol=1e-12, atol=1e-12)
    assert np.array_equal(trs.idx, trf.idx[rows])
    kv_app = om.KVCache(1, d.n_kv_heads, d.head_dim)
    kv_app.k[0], kv_app.v[0] = kv.k[0].copy(), kv.v[0].copy()
    m.layer(0, x, kv_app, causal, append=True)
    _, _, k_new, v_new = m.layer_rows(0, x, kv, causal, rows, return_kv=True)
    np.testing.assert_array_equal(k_new, kv_app.k[0][:, 9:])
    np.testing.assert_array_equal(v_new, kv_app.v[0][:, 9:])


def test_rmsnorm_constant_input():
    for c in (0.5, -3.0, 1e-4):
        g = np.linspace(0.5, 2.0, 10)
        y = om.rmsnorm(np.full((1, 10), c), g, 1e-6)
        np.testing.assert_allclose(y[0], g * c / math.sqrt(c * c + 1e-6), rtol=1e-14)


# ----------------------------------------------------------------------------- routing and MoE

def test_route_brute_force_and_ties():
    rng = np.random.default_rng(4)
    xn = rng.normal(size=(20, 6))
    wr = rng.normal(size=(10, 6))
    idx, w, r, gap = om.route(xn, wr, 3)
    for t in range(20):
        order = sorted(range(10), key=lambda e: (-r[t, e], e))[:3]
        assert list(idx[t]) == order
        sel = [r[t, e] for e in order]
        z = sum(math.exp(s - sel[0]) for s in sel)
        np.testing.assert_allclose(w[t], [math.exp(s - sel[0]) / z for s in sel], rtol=1e-12)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)
    assert np.all(gap >= 0)
    idx, w, _, gap = om.route(np.zeros((4, 6)), wr, 3)
    assert np.all(idx == [0, 1, 2]) and np.allclose(w, 1 / 3) and np.all(gap == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_moe_identical_experts_is_dense_ffn(dtype):
    """All experts equal -> the routed sum equals one dense SwiGLU FFN, whatever the routing."""
    rnd = numerics.rounder(dtype)
    rng = np.random.default_rng(5)
    d, f, E, k = 12, 10, 6, 2
    gu = rnd(rng.normal(size=(2 * f, d)) * 0.3)
    dn = rnd(rng.normal(size=(d, f)) * 0.3)
    xn = rnd(rng.normal(size=(9, d)))
    idx, w, _, _ = om.route(xn, rng.normal(size=(E, d)), k)
    got = om.moe_routed(xn, idx, w, np.broadcast_to(gu, (E, 2 * f, d)), np.broadcast_to(dn, (E, d, f)), rnd)
    gate = xn @ gu[:f].T
    up = xn @ gu[f:].T
    dense = rnd(rnd(gate / (1 + np.exp(-gate)) * up) @ dn.T)
    np.testing.assert_allclose(got, dense, rtol=1e-13, atol=1e-13)


def test_moe_all_experts_is_dense_mixture():
    rng = np.random.default_rng(6)
    d, f, E = 8, 6, 4
    gu = rng.normal(size=(E, 2 * f, d))
    dn = rng.normal(size=(E, d, f))
    xn = rng.normal(size=(5, d))
    wr = rng.normal(size=(E, d))
    idx, w, r, _ = om.route(xn, wr, E)
    got = om.moe_routed(xn, idx, w, gu, dn, lambda a: a)
    p = np.exp(r - r.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ref = np.zeros((5, d))
    for t in range(5):
        for e in range(E):
            g = xn[t] @ gu[e, :f].T
            u = xn[t] @ gu[e, f:].T
            ref[t] += p[t, e] * ((g / (1 + np.exp(-g)) * u) @ dn[e].T)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- keep / update

def test_keep_schedule_page_constants():
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        pc = json.load(f)
    S, T = pc["canvas_slots"]["value"], pc["timing_steps_T"]["value"]
    n_new = -(-S // T)
    assert n_new == 26 == recipe.C3.n_new
    ks = [osm.keep_count(t, n_new, S) for t in range(1, T + 1)]
    assert ks == [26, 52, 78, 104, 130, 156, 182, 208, 234, 256]
    assert osm.keep_count(4, recipe.C0.n_new, recipe.C0.dims.canvas) == 16


def test_canvas_update_invariants():
    rng = np.random.default_rng(7)
    S, V = 256, 262144
    pred = rng.integers(0, V, S)
    conf = rng.random(S).astype(np.float32).astype(np.float64)
    conf[10] = conf[20] = conf[30] = 0.99  # ties at the top
    conf[40] = np.nan
    for t, k in [(1, 26), (5, 130), (9, 234), (10, 256)]:
        canvas, mask = osm.canvas_update(pred, conf, k, 1, 3, t, V)
        assert canvas.shape == (S,) and mask.sum() == k
        assert np.all(canvas[mask] == pred[mask])
        fresh = philox.uniform_tokens(1, 3, t, np.arange(S), V)
        assert np.all(canvas[~mask] == fresh[~mask])
        assert canvas.min() >= 0 and canvas.max() < V
        if k < S:
            assert not mask[40]
        kept_conf = np.where(np.isnan(conf), -np.inf, conf)
        assert kept_conf[mask].min() >= kept_conf[~mask].max() if k < S else True
    # ties resolve to the lower slot
    mask = osm.keep_mask(np.ones(8), 3)
    assert list(np.nonzero(mask)[0]) == [0, 1, 2]


def test_initial_canvas_is_philox_step0():
    c = osm.initial_canvas(1, 2, 32, 4096)
    assert np.array_equal(c, philox.uniform_tokens(1, 2, 0, np.arange(32), 4096))


# ----------------------------------------------------------------------------- whole-pass invariants

def _tiny_model(seed_shift=0, **kw):
    d = small_dims(**kw)
    st = dg_inputs.model_weights_host(d, seed=recipe.WEIGHT_SEED + seed_shift)
    return d, oracle_model(d, st)


def test_pass_is_permutation_equivariant():
    """No positional term and a per-slot head: permuting the canvas permutes pred/conf/ent."""
    d, m = _tiny_model(n_layers=2)
    kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    osm.prefill(m, kv, dg_inputs.prompt_tokens(5, d.vocab))
    canvas = np.array([3, 9, 27, 1, 50, 60, 2, 33])
    perm = np.array([5, 2, 7, 0, 1, 6, 3, 4])
    a, _ = osm.denoise_pass(m, kv, canvas)
    b, _ = osm.denoise_pass(m, kv, canvas[perm])
    assert np.array_equal(a.pred[perm], b.pred)
    np.testing.assert_allclose(a.conf[perm], b.conf, rtol=1e-12)
    np.testing.assert_allclose(a.ent[perm], b.ent, rtol=1e-12)


def test_prefill_is_chunk_invariant():
    """Causal prefill in one call equals two consecutive calls (catches a wrong causal offset)."""
    d, m = _tiny_model()
    toks = dg_inputs.prompt_tokens(12, d.vocab)
    kv1 = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    osm.prefill(m, kv1, toks)
    kv2 = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    osm.prefill(m, kv2, toks[:5])
    osm.prefill(m, kv2, toks[5:])
    for l in range(d.n_layers):
        np.testing.assert_allclose(kv1.k[l], kv2.k[l], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(kv1.v[l], kv2.v[l], rtol=1e-12, atol=1e-12)


def test_canvas_keys_do_not_persist_until_commit():
    d, m = _tiny_model()
    kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    osm.prefill(m, kv, dg_inputs.prompt_tokens(4, d.vocab))
    osm.denoise_pass(m, kv, np.arange(8))
    assert kv.length == 4
    osm.commit(m, kv, np.arange(8))
    assert kv.length == 12


# ----------------------------------------------------------------------------- stop rule (E1-E4)

def _c0_like(n_layers=1, **kw):
    d = recipe.C0.dims
    from dataclasses import replace
    d = replace(d, n_layers=n_layers, **kw)
    return d


def test_stop_e1_uniform_logits_stable_at_two():
    d = _c0_like()
    st = dg_inputs.model_weights_host(d)
    st["embed"] = np.zeros_like(st["embed"])
    m = oracle_model(d, st)
    kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    res = osm.generate_block(m, kv, osm.Sampler(n_new=4), block=0, do_commit=False)
    assert res.reason == osm.STOP_STABLE and res.steps == 2
    np.testing.assert_allclose(res.mean_entropy, math.log(d.vocab), rtol=1e-12)
    assert np.all(res.tokens == 0)


def test_stop_e2_self_retrieval_entropy_at_one():
    d = _c0_like()
    st = dg_inputs.model_weights_host(d)
    for layer in st["layers"]:
        layer["wo"] = np.zeros_like(layer["wo"])
        layer["w_down"] = np.zeros_like(layer["w_down"])
        layer["ws_down"] = np.zeros_like(layer["ws_down"])
    st["final_norm"] = dg_inputs.const(st["final_norm"].shape, 10.0, d.dtype)
    m = oracle_model(d, st)
    kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    res = osm.generate_block(m, kv, osm.Sampler(n_new=4), block=0, do_commit=False)
    assert res.reason == osm.STOP_ENTROPY and res.steps == 1
    assert np.array_equal(res.tokens, res.passes[0].canvas)


def test_stop_fixed_and_cap_rules():
    s = osm.Sampler(n_new=26, fixed_steps=10)
    p = np.arange(4)
    assert osm.stop_reason(9, 0.0, p, p, s) == osm.STOP_NONE
    assert osm.stop_reason(10, 9.0, p, p + 1, s) == osm.STOP_FIXED
    s = osm.Sampler(n_new=26)
    assert osm.stop_reason(1, 0.01, p, None, s) == osm.STOP_ENTROPY
    assert osm.stop_reason(1, 1.0, p, None, s) == osm.STOP_NONE
    assert osm.stop_reason(2, 1.0, p, p.copy(), s) == osm.STOP_STABLE
    assert osm.stop_reason(47, 1.0, p, p + 1, s) == osm.STOP_NONE
    assert osm.stop_reason(48, 1.0, p, p + 1, s) == osm.STOP_CAP


def test_c0_block_never_exceeds_cap():
    d = recipe.C0.dims
    m = oracle_model(d)
    kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    osm.prefill(m, kv, dg_inputs.prompt_tokens(recipe.C0.prefix, d.vocab))
    res = osm.generate_block(m, kv, osm.Sampler(n_new=4), block=0)
    assert 1 <= res.steps <= 48
    assert res.reason in (osm.STOP_ENTROPY, osm.STOP_STABLE, osm.STOP_CAP)
    assert kv.length == recipe.C0.prefix + d.canvas
    for rec in res.passes:
        assert np.all(rec.ent >= 0) and np.all(rec.ent <= math.log(d.vocab) + 1e-9)


def test_model_size_consistent_with_pages():
    total, active = recipe.param_count(recipe.C3.dims)
    assert abs(total / 25.2e9 - 1) < 0.1
    assert abs(active / 3.8e9 - 1) < 0.15


# ----------------------------------------------------------------------------- sampler variants

EULER_GAMMA = 0.5772156649015329


def test_gumbel_noise_moments_and_range():
    """Standard Gumbel: mean = Euler's constant, variance = pi^2 / 6; u never 0 or 1."""
    g = philox.gumbel_noise(7, 2, 3, np.arange(64), 16384).ravel()  # 1M draws
    assert np.isfinite(g).all()
    assert abs(g.mean() - EULER_GAMMA) < 6e-3
    assert abs(g.var() - math.pi ** 2 / 6) < 2.5e-2
    lo, hi = -math.log(-math.log(2.0 ** -24)), -math.log(-math.log(1 - 2.0 ** -24))
    assert g.min() >= lo - 1e-12 and g.max() <= hi + 1e-12
    # the CDF at three points: P(G <= x) = exp(-exp(-x))
    for x in (-1.0, 0.0, 2.0):
        assert abs((g <= x).mean() - math.exp(-math.exp(-x))) < 3e-3


def test_gumbel_noise_counter_layout():
    """Token v of slot s takes word v mod 4 of the counter (v div 4, s + 2^16 t, block, 1)."""
    seed, block, step = (5 << 32) | 11, 9, 4
    g = philox.gumbel_noise(seed, block, step, np.array([3, 7]), 10)
    for i, s in enumerate((3, 7)):
        for v in range(10):
            w = philox.philox4x32_10((v // 4, s + (step << 16), block, 1), (11, 5))[v % 4]
            u = (2 * (int(w) >> 9) + 1) / 2.0 ** 24
            assert g[i, v] == -math.log(-math.log(u))
    # distinct from the canvas stream and from the neighbouring step / block
    assert not np.array_equal(g, philox.gumbel_noise(seed, block, step + 1, np.array([3, 7]), 10))
    assert not np.array_equal(g, philox.gumbel_noise(seed, block + 1, step, np.array([3, 7]), 10))


@pytest.mark.parametrize("beta", [1.0, 2.5])
def test_gumbel_max_draws_from_the_tempered_softmax(beta):
    """argmax(beta l + G) over 40960 (slot, step) draws: frequencies match softmax(beta l)."""
    l = np.log(np.array([1.0, 2.0, 3.0, 4.0]))
    counts = np.zeros(4)
    for step in range(1, 11):
        g = philox.gumbel_noise(3, 0, step, np.arange(4096), 4)
        counts += np.bincount(np.argmax(beta * l + g, axis=1), minlength=4)
    n = counts.sum()
    p = np.exp(beta * l) / np.exp(beta * l).sum()
    sd = np.sqrt(n * p * (1 - p))
    assert np.all(np.abs(counts - n * p) < 5 * sd), (counts / n, p)


def test_head_gumbel_confidence_is_probability_of_the_draw():
    """Textbook softmax by loops on a tiny vocabulary: conf = p[pred], pred = argmax(beta l + G)."""
    rng = np.random.default_rng(11)
    V, d, n, beta = 37, 8, 6, 1.25
    x = rng.normal(size=(n, d))
    E = rng.normal(size=(V, d)) * 0.7
    pred, conf, ent, margin = om.head_stats(x, np.ones(d), E, beta, 0.0, lambda t: t, gumbel=(4, 1, 2))
    g = philox.gumbel_noise(4, 1, 2, np.arange(n), V)
    plain = om.head_stats(x, np.ones(d), E, beta, 0.0, lambda t: t)
    for i in range(n):
        r = math.sqrt(sum(v * v for v in x[i]) / d)
        lg = [beta * sum((x[i][c] / r) * E[v][c] for c in range(d)) for v in range(V)]
        score = [lg[v] + g[i][v] for v in range(V)]
        best = max(range(V), key=lambda v: (score[v], -v))
        m = max(lg)
        z = sum(math.exp(a - m) for a in lg)
        assert pred[i] == best
        assert abs(conf[i] - math.exp(lg[best] - m) / z) < 1e-12
        assert conf[i] <= plain[1][i] + 1e-15
        assert abs(ent[i] - plain[2][i]) < 1e-12  # the entropy does not depend on the draw
    assert (pred != plain[0]).any()  # at this temperature some draws leave the argmax


def test_head_gumbel_reduces_to_argmax_when_one_logit_dominates():
    """A logit gap above the Gumbel range (|G| < 17 for u in (0, 1) on the 2^-24 grid) makes the
    draw the argmax, and conf = max p."""
    V, d = 512, 2
    E = np.zeros((V, d))
    E[77] = [20.0, 20.0]
    x = np.ones((3, d))
    pred, conf, _, _ = om.head_stats(x, np.ones(d), E, 1.0, 0.0, lambda t: t, gumbel=(1, 0, 1))
    ref = om.head_stats(x, np.ones(d), E, 1.0, 0.0, lambda t: t)
    assert np.all(pred == 77) and np.array_equal(pred, ref[0])
    np.testing.assert_allclose(conf, ref[1], rtol=1e-14)


def test_anneal_schedule_page_values():
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        pc = json.load(f)
    t0, t1 = pc["anneal_temperature_first"]["value"], pc["anneal_temperature_last"]["value"]
    cap = pc["max_denoising_steps"]["value"]
    s = osm.Sampler(n_new=26, anneal=(t0, t1))
    temps = [1.0 / osm.pass_inv_temperature(s, t) for t in range(1, cap + 1)]
    assert abs(temps[0] - 0.8) < 1e-15 and abs(temps[-1] - 0.4) < 1e-15
    steps = np.diff(temps)
    np.testing.assert_allclose(steps, -0.4 / 47, rtol=1e-12)  # linear in T, falling
    s10 = osm.Sampler(n_new=26, anneal=(t0, t1), fixed_steps=pc["timing_steps_T"]["value"])
    assert abs(1.0 / osm.pass_inv_temperature(s10, 10) - 0.4) < 1e-15
    assert abs(1.0 / osm.pass_inv_temperature(s10, 1) - 0.8) < 1e-15
    assert osm.pass_inv_temperature(osm.Sampler(n_new=1, inv_temperature=2.5), 7) == 2.5


def test_entropy_rank_equals_confidence_rank_for_two_level_slots():
    """One boosted token over a uniform rest: entropy falls as the confidence grows, so both
    keep rules select the same slots; hand cases pin the ties and NaN."""
    V, d, n = 300, 2, 24
    rng = np.random.default_rng(5)
    a = rng.permutation(np.linspace(0.5, 9.0, n))  # the boosted logit of each slot
    E = np.zeros((V, d))
    E[5] = [1.0, 0.0]
    x = np.array([[1.0, 1.0]])  # normalised to itself
    stats = [om.head_stats(x, np.ones(d), E * ai, 1.0, 0.0, lambda t: t) for ai in a]
    conf = np.array([st[1][0] for st in stats])
    ent = np.array([st[2][0] for st in stats])
    assert np.all(np.argsort(conf) == np.argsort(-ent))
    for k in (1, 5, 12, 24):
        assert np.array_equal(osm.select_keep(osm.rank_key(conf, ent, True), k), osm.keep_mask(conf, k))
    key = osm.rank_key(None, np.array([0.3, np.nan, 0.1, 0.1, 0.2]), True)
    assert list(np.nonzero(osm.select_keep(key, 3))[0]) == [2, 3, 4]
    assert list(np.nonzero(osm.select_keep(key, 4))[0]) == [0, 2, 3, 4]


def test_lock_update_hand_case():
    """Locked slots stay kept with their token; new locks fill up to k by the key; the rest redraw."""
    S, V = 6, 1000
    pred = np.array([10, 11, 12, 13, 14, 15])
    conf = np.array([0.9, 0.1, 0.8, 0.7, 0.95, 0.2])
    canvas = np.array([100, 101, 102, 103, 104, 105])
    locked = np.array([False, True, False, False, False, True])
    out, mask = osm.canvas_update(pred, conf, 4, 1, 0, 3, V, None, False, locked, canvas)
    assert list(np.nonzero(mask)[0]) == [0, 1, 4, 5]
    assert list(out[[0, 1, 4, 5]]) == [10, 101, 14, 105]
    fresh = philox.uniform_tokens(1, 0, 3, np.arange(S), V)
    assert list(out[[2, 3]]) == list(fresh[[2, 3]])
    # k below the locked count: nothing new locks, nothing unlocks
    out2, mask2 = osm.canvas_update(pred, conf, 1, 1, 0, 3, V, None, False, locked, canvas)
    assert np.array_equal(mask2, locked) and list(out2[[1, 5]]) == [101, 105]


def test_lock_block_invariants_c0():
    """The lock variant on the tiny model: k_t slots locked after pass t, a locked token never
    changes again, and the committed block keeps every locked token."""
    d = recipe.C0.dims
    m = oracle_model(d)
    kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    osm.prefill(m, kv, dg_inputs.prompt_tokens(recipe.C0.prefix, d.vocab))
    s = osm.Sampler(n_new=4, fixed_steps=10, lock=True, gumbel=True, anneal=(0.8, 0.4))
    res = osm.generate_block(m, kv, s, block=0, do_commit=False)
    assert res.steps == 10 and res.reason == osm.STOP_FIXED
    locked_tok = {}
    for t, rec in enumerate(res.passes, start=1):
        for slot, tok in locked_tok.items():
            assert rec.canvas[slot] == tok and rec.pred[slot] == tok
        if rec.keep is not None:
            assert rec.keep.sum() == min(d.canvas, 4 * t)
            for slot in np.nonzero(rec.keep)[0]:
                locked_tok.setdefault(int(slot), int(res.passes[t].canvas[slot]))
    assert all(res.tokens[s_] == tok for s_, tok in locked_tok.items())


def test_stop_and_rule_cases():
    p = np.arange(4)
    s_or = osm.Sampler(n_new=26, entropy_threshold=0.005)
    s_and = osm.Sampler(n_new=26, entropy_threshold=0.005, stop_and=True)
    assert osm.stop_reason(3, 0.001, p, p + 1, s_or) == osm.STOP_ENTROPY
    assert osm.stop_reason(3, 0.001, p, p + 1, s_and) == osm.STOP_NONE       # low but unsettled
    assert osm.stop_reason(3, 2.0, p, p.copy(), s_or) == osm.STOP_STABLE
    assert osm.stop_reason(3, 2.0, p, p.copy(), s_and) == osm.STOP_NONE      # stable but uncertain
    assert osm.stop_reason(3, 0.001, p, p.copy(), s_and) == osm.STOP_SETTLED
    assert osm.stop_reason(1, 0.001, p, None, s_and) == osm.STOP_NONE        # stability needs two passes
    assert osm.stop_reason(48, 2.0, p, p + 1, s_and) == osm.STOP_CAP
    s_fix = osm.Sampler(n_new=26, fixed_steps=10, stop_and=True)
    assert osm.stop_reason(10, 2.0, p, p + 1, s_fix) == osm.STOP_FIXED


def test_recommended_sampler_block_c0():
    """All variants together with the pages' thresholds (0.005 and 0.1): random weights never reach
    them, so with the AND rule the block runs to the cap or to two settled passes."""
    d = recipe.C0.dims
    m = oracle_model(d)
    for thr in (0.005, 0.1):
        kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
        osm.prefill(m, kv, dg_inputs.prompt_tokens(recipe.C0.prefix, d.vocab))
        s = osm.Sampler(n_new=4, entropy_threshold=thr, gumbel=True, anneal=(0.8, 0.4), rank_entropy=True,
                        lock=True, stop_and=True)
        res = osm.generate_block(m, kv, s, block=0, do_commit=False)
        assert res.reason in (osm.STOP_CAP, osm.STOP_SETTLED) and 1 <= res.steps <= 48
        if res.reason == osm.STOP_CAP:
            assert res.steps == 48
        for rec in res.passes:
            assert np.all(rec.ent >= 0) and np.all(rec.ent <= math.log(d.vocab) + 1e-9)



# ----------------------------------------------------------------------------- self-speculative verify

def _self_retrieval_model():
    """Attention and expert outputs zeroed: each row's hidden state is its own embedding, so the greedy causal
    prediction of a row is its own token (a copy model)."""
    d = _c0_like()
    st = dg_inputs.model_weights_host(d)
    for layer in st["layers"]:
        layer["wo"] = np.zeros_like(layer["wo"])
        layer["w_down"] = np.zeros_like(layer["w_down"])
        layer["ws_down"] = np.zeros_like(layer["ws_down"])
    st["final_norm"] = dg_inputs.const(st["final_norm"].shape, 10.0, d.dtype)
    return d, oracle_model(d, st)


def test_verify_copy_model_accepts_runs():
    """With a copy model a_i = d_i, so d_i is accepted while it repeats its predecessor: the accepted count is the
    length of the leading run, and the next token repeats the run's token."""
    d, m = _self_retrieval_model()
    S = d.canvas
    for draft, n_expect in [([5] * S, S), ([5, 5, 5, 7] + [7] * (S - 4), 3), ([9, 8] + [8] * (S - 2), 1)]:
        kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
        osm.prefill(m, kv, dg_inputs.prompt_tokens(6, d.vocab))
        r = osm.verify_block(m, kv, draft)
        assert np.array_equal(r.ar_pred, draft)
        assert r.accepted == n_expect and r.next_token == draft[n_expect - 1]
        assert kv.length == 6 + n_expect


def test_verify_rows_equal_commit_rows():
    """The verify pass is the commit's causal forward: its kept cache rows equal a commit of the accepted tokens,
    and a draft made of the causal pass's own greedy continuation is accepted whole."""
    d = recipe.C0.dims
    m = oracle_model(d)
    prompt = dg_inputs.prompt_tokens(recipe.C0.prefix, d.vocab)
    kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    osm.prefill(m, kv, prompt)
    # greedy continuation of the prompt, one causal step at a time
    x = m.embed(prompt)
    kv_g = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    h, _ = m.body(x, kv_g, causal=True, append=True)
    tok = int(m.head(h[-1:])[0][0])
    greedy = []
    for _ in range(8):
        greedy.append(tok)
        h, _ = m.body(m.embed([tok]), kv_g, causal=True, append=True)
        tok = int(m.head(h)[0][0])
    draft = np.array(greedy + list(dg_inputs.prompt_tokens(d.canvas - 8, d.vocab, seed=9)))
    r = osm.verify_block(m, kv, draft)
    assert r.accepted >= 8 and np.array_equal(r.ar_pred[:7], draft[1:8])
    assert r.next_token == r.ar_pred[r.accepted - 1]
    kv_c = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    osm.prefill(m, kv_c, prompt)
    osm.commit(m, kv_c, draft[:r.accepted])
    for l in range(d.n_layers):
        np.testing.assert_allclose(kv.k[l], kv_c.k[l], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(kv.v[l], kv_c.v[l], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- self-speculative decoding loop

def test_speculative_equals_greedy_autoregressive_decoding():
    """The speculative loop outputs exactly greedy autoregressive decoding from the known first token (computed
    here one causal step at a time, a different route through the same model): the drafts only decide how many
    tokens each verify confirms.  Catches: emitting an unverified draft token, a wrong next-token carry, a cache
    that keeps rejected rows."""
    d, m = _speculative_model()
    prompt = dg_inputs.prompt_tokens(16, d.vocab)
    kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    osm.prefill(m, kv, prompt)
    kv_ar = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    osm.prefill(m, kv_ar, prompt)
    first = 7
    res = osm.generate_speculative(m, kv, osm.Sampler(n_new=2, fixed_steps=3), block0=0, first_token=first,
                                   n_tokens=16)
    ar = osm.greedy_autoregressive(m, kv_ar, first, 16)
    assert np.array_equal(res.tokens, ar)
    assert len(set(ar.tolist())) > 3          # a chain that moves, so a wrong carry or token shows
    assert max(res.accepted) > 1              # and some draft tokens were confirmed
    assert sum(res.accepted) >= 16 and all(a >= 1 for a in res.accepted)
    assert kv.length == 16 + sum(res.accepted)
    for l in range(d.n_layers):   # the kept cache rows are the autoregressive ones
        np.testing.assert_allclose(kv.k[l][:, :16 + 15], kv_ar.k[l][:, :16 + 15], rtol=1e-12, atol=1e-12)


def _speculative_model():
    """A one-layer fp32 model whose output projections are scaled up 30 times, so that the layer, not the
    embedding, decides the head's argmax: its greedy chain moves from token to token (at the seeded random init
    the tied head mostly returns a row's own token) and some diffusion drafts agree with it."""
    d = replace(recipe.C0.dims, canvas=8, n_layers=1, vocab=64)
    st = dg_inputs.model_weights_host(d)
    for layer in st["layers"]:
        for n in ("wo", "w_down", "ws_down"):
            layer[n] = (layer[n] * 30.0).astype(np.float32)
    return d, oracle_model(d, st)


def test_speculative_uniform_model_accepts_whole_blocks():
    """Zero embeddings give uniform logits, so diffusion and causal passes both predict token 0 everywhere: every
    verify accepts the whole draft (the known token, then S - 1 zeros) and the output is [t, 0, 0, ...]."""
    d = replace(recipe.C0.dims, canvas=8, n_layers=1)
    st = dg_inputs.model_weights_host(d)
    st["embed"] = np.zeros_like(st["embed"])
    m = oracle_model(d, st)
    kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    osm.prefill(m, kv, dg_inputs.prompt_tokens(5, d.vocab))
    res = osm.generate_speculative(m, kv, osm.Sampler(n_new=2, fixed_steps=2), block0=3, first_token=9, n_tokens=20)
    assert res.accepted == [8, 8, 8]
    assert list(res.tokens) == [9] + [0] * 19
    assert kv.length == 5 + 24
