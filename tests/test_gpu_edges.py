"""GPU edge cases against the oracle: ragged row counts, the degenerate routing where every token picks
the same experts, and empty calls.

Ragged rows exercise the padded tails of the fragment-tiled activations (row tiles of 16), the partial
query tiles of the attention kernel and the partial key chunks; the all-tied router puts every token on
the same k experts, the maximum load one expert can receive (a tile list of M / 32 tiles per expert).
"""
from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import block_diffusion_decoding_step_amd as dg  # noqa: E402
import dg_inputs  # noqa: E402
from dg_inputs import device as gdev  # noqa: E402
from dg_inputs import recipe  # noqa: E402
from oracle import model as om  # noqa: E402
from oracle import numerics  # noqa: E402
from oracle import sampler as osm  # noqa: E402
from tests._gpu import Session, allclose_report, compare_routing, to_f64  # noqa: E402
from tests._helpers import oracle_dims, oracle_model  # noqa: E402

F32_TOL = (1e-4, 1e-4)
BF16_TOL = (2e-2, 2e-2)
MARGIN = 1e-2


def log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("n,chunk_rows", [(77, 24), (33, 40), (5, 16)])
def test_prefill_ragged_chunks(n, chunk_rows):
    """A prompt whose length and chunking leave partial 16-row tiles: same cache as the oracle."""
    d = recipe.C0.dims
    storage = dg_inputs.model_weights_host(d)
    sess = Session(d, capacity=128, max_tokens=max(d.canvas, chunk_rows), weights=gdev.from_host(storage, d.dtype))
    ws_small = dg.dg_workspace_size(sess.cfg, chunk_rows)
    prompt = dg_inputs.prompt_tokens(n, d.vocab)
    dg.dg_prefill_kv(sess.cfg, sess.weights, sess.kv, torch.from_numpy(prompt).cuda(), n, sess.ws, ws_small)
    torch.cuda.synchronize()
    model = oracle_model(d, storage)
    kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    osm.prefill(model, kv, prompt)
    assert sess.kv.len == kv.length == n
    for l in range(d.n_layers):
        gk, gv = sess.kv_numpy(l, n)
        assert allclose_report(gk, kv.k[l], *F32_TOL)[0], ("K", l)
        assert allclose_report(gv, kv.v[l], *F32_TOL)[0], ("V", l)


@pytest.mark.parametrize("S", [20, 33])
def test_pass_ragged_canvas(S):
    """A canvas that is not a multiple of 16 slots, over a ragged 45-token prompt: pass against the oracle."""
    d = replace(recipe.C0.dims, canvas=S)
    storage = dg_inputs.model_weights_host(d)
    P = 45
    sess = Session(d, capacity=P + 2 * S, max_tokens=64, weights=gdev.from_host(storage, d.dtype))
    model = oracle_model(d, storage)
    kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    prompt = dg_inputs.prompt_tokens(P, d.vocab)
    sess.prefill(prompt)
    osm.prefill(model, kv, prompt)
    canvas = osm.initial_canvas(recipe.INPUT_SEED, 0, S, d.vocab)
    pred, conf, ent = sess.denoise(canvas)
    torch.cuda.synchronize()
    rec, _ = osm.denoise_pass(model, kv, canvas)
    sel = rec.margin > MARGIN
    assert np.array_equal(pred.cpu().numpy()[sel], rec.pred[sel])
    assert allclose_report(to_f64(ent), rec.ent, *F32_TOL)[0]
    assert allclose_report(to_f64(conf), rec.conf, 1e-7, 1e-4)[0]


def _layer_pair(d, storage_layer, x_host, P, k_host, v_host, causal):
    w = gdev.from_host({"embed": dg_inputs.zeros((8, d.d_model), d.dtype), "final_norm": dg_inputs.ones(d.d_model, d.dtype),
                        "layers": [storage_layer]}, d.dtype)
    M = x_host.shape[0]
    sess = Session(d, capacity=P + M, max_tokens=M, weights=w)
    dt = torch.bfloat16 if d.dtype == "bf16" else torch.float32

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if d.dtype == "bf16" else np.ascontiguousarray(a))
        return t.cuda().view(dt) if d.dtype == "bf16" else t.cuda()

    if P:
        sess.k[0, :, :P, :] = up(k_host)
        sess.v[0, :, :, :P] = up(v_host.transpose(0, 2, 1))
        sess.kv.len = P
    x_dev = up(x_host)
    y_dev = torch.empty_like(x_dev)
    ridx = torch.empty((M, d.top_k), dtype=torch.int32, device="cuda")
    rw = torch.empty((M, d.top_k), dtype=torch.float32, device="cuda")
    rlog = torch.empty((M, d.n_experts), dtype=torch.float32, device="cuda")
    dg.dg_layer_forward(sess.cfg, sess.weights, 0, sess.kv, x_dev, y_dev, M, causal,
                        {"route_idx": ridx, "route_w": rw, "router_logits": rlog}, sess.ws, sess.ws_bytes)
    torch.cuda.synchronize()
    model = om.Model(oracle_dims(d), {"embed": None, "final_norm": None,
                                      "layers": [{n: numerics.from_storage(a, d.dtype)
                                                  for n, a in storage_layer.items()}]})
    kv = om.KVCache(1, d.n_kv_heads, d.head_dim)
    if P:
        kv.k[0] = numerics.from_storage(k_host, d.dtype)
        kv.v[0] = numerics.from_storage(v_host, d.dtype)
    y_ref, tr = model.layer(0, numerics.from_storage(x_host, d.dtype), kv, bool(causal), append=False)
    return to_f64(y_dev), y_ref, tr, ridx.cpu().numpy(), rw.cpu().numpy(), rlog.cpu().numpy()


@pytest.mark.parametrize("dims,tol,M,P", [(replace(recipe.C0.dims, n_layers=1), F32_TOL, 64, 40),
                                          (replace(recipe.C0.dims, n_layers=1), F32_TOL, 71, 40),
                                          (replace(recipe.C1.dims, n_layers=1), BF16_TOL, 256, 96),
                                          (replace(recipe.C1.dims, n_layers=1), BF16_TOL, 200, 96)])
def test_all_tokens_route_to_the_same_experts(dims, tol, M, P):
    """Zero router weights: every logit is 0, so every token picks experts 0..k-1 (ties to the lower id)
    with weight 1/k, and those k experts each take all M tokens (the busiest possible routing).  M = 71
    and 200 leave each busy expert a short last tile (3 tiles ending in 7 rows, 7 ending in 8)."""
    d = dims
    host = dg_inputs.layer_weights_host(d, 0)
    host["w_router"] = np.zeros_like(host["w_router"])
    x_host = dg_inputs.hidden((M, d.d_model), d.dtype)
    k_host = dg_inputs.normal((d.n_kv_heads, P, d.head_dim), recipe.INPUT_SEED, recipe.STREAM_PREFIX_K, 1.0, d.dtype)
    v_host = dg_inputs.normal((d.n_kv_heads, P, d.head_dim), recipe.INPUT_SEED, recipe.STREAM_PREFIX_V, 1.0, d.dtype)
    y, y_ref, tr, ridx, rw, rlog = _layer_pair(d, host, x_host, P, k_host, v_host, 0)
    expect = np.broadcast_to(np.arange(d.top_k), (M, d.top_k))
    assert np.array_equal(ridx, expect)
    assert np.array_equal(tr.idx, expect)
    assert np.allclose(rw, 1.0 / d.top_k, atol=1e-7)
    assert np.all(rlog == 0)
    ok, worst, at = allclose_report(y, y_ref, *tol)
    assert ok, (worst, at)


def test_layer_ragged_rows_causal():
    """37 causal rows after a 19-key prefix (partial row tiles, partial key chunks), fp32."""
    d = replace(recipe.C0.dims, n_layers=1)
    host = dg_inputs.layer_weights_host(d, 0)
    M, P = 37, 19
    x_host = dg_inputs.hidden((M, d.d_model), d.dtype)
    k_host = dg_inputs.normal((d.n_kv_heads, P, d.head_dim), recipe.INPUT_SEED, recipe.STREAM_PREFIX_K, 1.0, d.dtype)
    v_host = dg_inputs.normal((d.n_kv_heads, P, d.head_dim), recipe.INPUT_SEED, recipe.STREAM_PREFIX_V, 1.0, d.dtype)
    y, y_ref, tr, ridx, rw, rlog = _layer_pair(d, host, x_host, P, k_host, v_host, 1)
    same = compare_routing(ridx, rw, rlog, tr.router_logits, tr.idx, F32_TOL)
    ok, worst, at = allclose_report(y[same], y_ref[same], *F32_TOL)
    assert ok, (worst, at)


def test_empty_prefill_is_a_no_op():
    d = recipe.C0.dims
    sess = Session(d, capacity=64, max_tokens=d.canvas, weights=gdev.from_host(dg_inputs.model_weights_host(d), d.dtype))
    before = sess.k.clone()
    dg.dg_prefill_kv(sess.cfg, sess.weights, sess.kv, None, 0, sess.ws, sess.ws_bytes)
    torch.cuda.synchronize()
    assert sess.kv.len == 0
    assert torch.equal(before, sess.k)


@pytest.mark.parametrize("E,k", [(160, 8), (24, 12), (256, 16)])
def test_layer_router_slices_and_wide_top_k(E, k):
    """Expert counts past one 64-expert router slice (two slices of 128 when E > 128, the second one
    partly empty) and top-k past 8: one causal fp32 layer against the oracle."""
    d = replace(recipe.C0.dims, n_layers=1, n_experts=E, top_k=k)
    host = dg_inputs.layer_weights_host(d, 0)
    M, P = 40, 24
    x_host = dg_inputs.hidden((M, d.d_model), d.dtype)
    k_host = dg_inputs.normal((d.n_kv_heads, P, d.head_dim), recipe.INPUT_SEED, recipe.STREAM_PREFIX_K, 1.0, d.dtype)
    v_host = dg_inputs.normal((d.n_kv_heads, P, d.head_dim), recipe.INPUT_SEED, recipe.STREAM_PREFIX_V, 1.0, d.dtype)
    log(f"router slices: E={E} k={k}")
    y, y_ref, tr, ridx, rw, rlog = _layer_pair(d, host, x_host, P, k_host, v_host, 1)
    same = compare_routing(ridx, rw, rlog, tr.router_logits, tr.idx, F32_TOL)
    assert same.sum() >= M - 1
    ok, worst, at = allclose_report(y[same], y_ref[same], *F32_TOL)
    assert ok, (worst, at)
