"""GPU parity of each stage of the denoising step against the oracle, through the C ABI.

Inputs come from the seeded generator (dg_inputs) on both sides; nothing the
GPU computes is fed to the oracle.  Bars: bit-exact for integer work (canvas
update, routing, argmax where the fp32 top-2 margin exceeds the threshold);
|gpu - oracle| <= 2e-2 + 2e-2|oracle| in bf16 and 1e-4 + 1e-4|oracle| in fp32.
"""
from __future__ import annotations

import math
import sys
from dataclasses import replace

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import block_diffusion_decoding_step_amd as dg  # noqa: E402
import dg_inputs  # noqa: E402
from dg_inputs import device as gdev  # noqa: E402
from dg_inputs import recipe  # noqa: E402
from oracle import model as om  # noqa: E402
from oracle import numerics  # noqa: E402
from oracle import philox  # noqa: E402
from oracle import sampler as osm  # noqa: E402
from tests._gpu import Session, allclose_report, compare_routing, to_f64  # noqa: E402
from tests._helpers import oracle_dims, oracle_model  # noqa: E402

TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 2e-2)}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ----------------------------------------------------------------------------- generator

def test_device_generator_matches_host():
    for dtype in ("bf16", "f32"):
        t = gdev.normal_tensor((1000, 37), 5, 9, 0.02, dtype)
        h = dg_inputs.normal((1000, 37), 5, 9, 0.02, dtype)
        got = t.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" else t.cpu().numpy()
        assert np.array_equal(got, h)
    u = gdev.uniform_tensor(5000, 1, 1, 262144)
    assert np.array_equal(u.cpu().numpy(), dg_inputs.uniform_int(5000, 1, 1, 262144))


# ----------------------------------------------------------------------------- weight layout

@pytest.mark.parametrize("dtype,batch,rows,cols", [("bf16", 1, 48, 64), ("f32", 2, 40, 96), ("bf16", 3, 8, 32)])
def test_pack_matrix_layout(dtype, batch, rows, cols):
    """Fragment-tiled layout: element (r, c) of each matrix at ((r/16)*(C/32) + c/32)*512 + ((r%16) + 16*((c%32)/8))*8
    + c%8, padded rows zero."""
    src = gdev.normal_tensor((batch, rows, cols), 3, 7, 1.0, dtype)
    out = dg.pack_tensor(src if batch > 1 else src[0])
    torch.cuda.synchronize()
    a = src.float().cpu().numpy()
    got = out.float().cpu().numpy()
    rows_p = (rows + 15) // 16 * 16
    per = rows_p * cols
    assert got.size == batch * per
    exp = np.zeros(batch * per, dtype=np.float32)
    for b in range(batch):
        for r in range(rows):
            for c in range(cols):
                i = ((r // 16) * (cols // 32) + c // 32) * 512 + ((r % 16) + 16 * ((c % 32) // 8)) * 8 + c % 8
                exp[b * per + i] = a[b, r, c]
    assert np.array_equal(got, exp)


# ----------------------------------------------------------------------------- canvas update

@pytest.mark.parametrize("S,V", [(32, 4096), (256, 262144), (200, 1000)])
def test_canvas_update_bit_exact(S, V):
    d = replace(recipe.C0.dims, canvas=S, vocab=V)
    cfg = dg.make_config(d)
    pred_h = dg_inputs.uniform_int(S, 3, 11, V)
    # confidences on a coarse grid so that ties occur; one NaN
    conf_h = (dg_inputs.uniform_int(S, 3, 12, 16).astype(np.float32) / 16.0).astype(np.float32)
    conf_h[S // 3] = np.nan
    pred = torch.from_numpy(pred_h).cuda()
    conf = torch.from_numpy(conf_h).cuda()
    out = torch.empty(S, dtype=torch.int32, device="cuda")
    mask = torch.empty(S, dtype=torch.uint8, device="cuda")
    for step, keep in [(0, 0), (1, 4), (3, 26), (7, S - 1), (9, S)]:
        dg.dg_canvas_update(cfg, pred if keep else None, conf if keep else None, keep, 1, 5, step, out, mask)
        torch.cuda.synchronize()
        if keep == 0:
            exp = philox.uniform_tokens(1, 5, step, np.arange(S), V)
            exp_mask = np.zeros(S, dtype=bool)
        else:
            exp, exp_mask = osm.canvas_update(pred_h, conf_h.astype(np.float64), keep, 1, 5, step, V)
        assert np.array_equal(out.cpu().numpy(), exp), (S, step, keep)
        assert np.array_equal(mask.cpu().numpy().astype(bool), exp_mask), (S, step, keep)
    # initial canvas of another block and a 64-bit seed
    dg.dg_canvas_update(cfg, None, None, 0, (7 << 32) | 3, 2, 0, out, None)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), osm.initial_canvas((7 << 32) | 3, 2, S, V))


def test_canvas_update_rejects_bad_keep():
    cfg = dg.make_config(recipe.C0.dims)
    out = torch.empty(32, dtype=torch.int32, device="cuda")
    with pytest.raises(dg.DGError):
        dg.dg_canvas_update(cfg, None, None, 33, 1, 0, 0, out)
    with pytest.raises(dg.DGError):
        dg.dg_canvas_update(cfg, None, None, 3, 1, 0, 0, out)  # keep > 0 needs pred and conf


# ----------------------------------------------------------------------------- stop check

def test_stop_check_engineered():
    d = recipe.C0.dims
    cfg = dg.make_config(d)
    S = d.canvas
    st = torch.zeros(4, dtype=torch.int32, device="cuda")
    prev = torch.zeros(S, dtype=torch.int32, device="cuda")
    pred = torch.arange(S, dtype=torch.int32, device="cuda")
    low = torch.full((S,), 0.01, device="cuda")
    high = torch.full((S,), 3.0, device="cuda")

    def run(step, ent, p, sampler):
        dg.dg_stop_check(cfg, sampler, step, ent, p, prev, st)
        torch.cuda.synchronize()
        a = st.cpu().numpy()
        return int(a[0]), int(a[1]), float(a[2:3].view(np.float32)[0]), int(a[3])

    s = dg.make_sampler(4)
    assert run(1, low, pred, s)[1] == dg.DG_STOP_ENTROPY
    assert run(1, high, pred, s)[1] == dg.DG_STOP_NONE       # prev <- pred
    assert run(2, high, pred, s)[1] == dg.DG_STOP_STABLE     # unchanged over two passes
    assert run(3, high, pred + 1, s)[1] == dg.DG_STOP_NONE
    assert run(48, high, pred, s)[1] == dg.DG_STOP_CAP
    steps, reason, mean, flags = run(10, high, pred + 5, dg.make_sampler(4, fixed_steps=10))
    assert (steps, reason, flags) == (10, dg.DG_STOP_FIXED, 0) and abs(mean - 3.0) < 1e-6
    bad = high.clone()
    bad[3] = float("nan")
    assert run(5, bad, pred, s)[3] & dg.DG_WARN_NUMERIC


# ----------------------------------------------------------------------------- vocab head

def _head_session(d, embed_host=None):
    w = {"embed": gdev.normal_tensor((d.vocab, d.d_model), 0, recipe.STREAM_EMBED, 0.02, d.dtype)
         if embed_host is None else torch.from_numpy(embed_host).cuda(),
         "final_norm": torch.ones(d.d_model, dtype=gdev.torch_dtype(d.dtype), device="cuda"), "layers": []}
    return Session(replace(d, n_layers=0), capacity=32, weights=w)


def _run_head(sess, x_dev, n, beta=1.0):
    pred, conf, ent = sess.i32(n), sess.f32(n), sess.f32(n)
    dg.dg_vocab_head(sess.cfg, sess.weights, x_dev, n, beta, pred, conf, ent, sess.ws, sess.ws_bytes)
    torch.cuda.synchronize()
    return pred.cpu().numpy(), conf.cpu().numpy().astype(np.float64), ent.cpu().numpy().astype(np.float64)


def test_head_uniform_logits_closed_form():
    d = recipe.C0.dims
    sess = _head_session(d, embed_host=np.zeros((d.vocab, d.d_model), np.float32))
    x = gdev.normal_tensor((d.canvas, d.d_model), 1, recipe.STREAM_HIDDEN, 1.0, "f32")
    pred, conf, ent = _run_head(sess, x, d.canvas)
    assert np.all(pred == 0)
    np.testing.assert_allclose(ent, math.log(d.vocab), rtol=2e-6)
    np.testing.assert_allclose(conf, 1.0 / d.vocab, rtol=2e-6)


def test_head_two_level_closed_form():
    """One token's logit raised by a, the rest 0: closed-form Z, confidence and entropy."""
    d = replace(recipe.C0.dims, canvas=4)
    E = np.zeros((d.vocab, d.d_model), np.float32)
    targets = [5, 4000, 64, 1]
    amps = [3.0, 7.5, 0.5, 12.0]
    x = np.zeros((4, d.d_model), np.float32)
    for i, (v, a) in enumerate(zip(targets, amps)):
        x[i, i] = 1.0                      # rms(x) = 1/sqrt(d): normalised row has sqrt(d) at column i
        E[v, i] = a / math.sqrt(d.d_model)  # logit of token v = a (eps aside)
    sess = _head_session(d, embed_host=E)
    pred, conf, ent = _run_head(sess, torch.from_numpy(x).cuda(), 4)
    for i, (v, a) in enumerate(zip(targets, amps)):
        a_eff = a / math.sqrt(1.0 + 1e-6 * d.d_model)
        Z = math.exp(a_eff) + d.vocab - 1
        assert pred[i] == v
        assert abs(conf[i] - math.exp(a_eff) / Z) <= 1e-5 * conf[i]
        assert abs(ent[i] - (math.log(Z) - a_eff * math.exp(a_eff) / Z)) <= 1e-4


def test_head_ties_lowest_id_across_tiles():
    d = replace(recipe.C0.dims, canvas=2)
    E = np.zeros((d.vocab, d.d_model), np.float32)
    E[[70, 3000, 1000], 0] = 1.0   # equal maxima in different 64-token tiles and work groups
    x = np.zeros((2, d.d_model), np.float32)
    x[:, 0] = 1.0
    sess = _head_session(d, embed_host=E)
    pred, _, _ = _run_head(sess, torch.from_numpy(x).cuda(), 2)
    assert list(pred) == [70, 70]


def _compare_head(d, x_host, x_dev, rows, pred, conf, ent, E64):
    atol, rtol = TOL[d.dtype]
    xs = numerics.from_storage(x_host[rows], d.dtype)
    opred, oconf, oent, margin = om.head_stats(xs, np.ones(d.d_model), E64, 1.0, d.rms_eps,
                                               numerics.rounder(d.dtype))
    sel = margin > 1e-2
    assert np.array_equal(pred[rows][sel], opred[sel])
    ok, worst, at = allclose_report(conf[rows], oconf, atol * 0 + 1e-6, rtol)
    assert ok, ("conf", worst, at)
    ok, worst, at = allclose_report(ent[rows], oent, atol, rtol)
    assert ok, ("ent", worst, at)
    return int(sel.sum())


def test_head_c0_fp32_all_slots():
    d = recipe.C0.dims
    sess = _head_session(d)
    x_host = dg_inputs.hidden((d.canvas, d.d_model), "f32")
    x_dev = torch.from_numpy(x_host).cuda()
    pred, conf, ent = _run_head(sess, x_dev, d.canvas)
    E64 = numerics.from_storage(dg_inputs.embed_host(d), "f32")
    n = _compare_head(d, x_host, x_dev, np.arange(d.canvas), pred, conf, ent, E64)
    assert n >= d.canvas - 2


def test_head_c2_bf16_sampled_slots():
    """Full C2 size: 256 slots x 262144 vocab x 2816; every slot's output depends on its row only, so a sample
    of slots is checked exactly against the oracle and the rest by invariants."""
    d = recipe.C2.dims
    sess = _head_session(d)
    x_host = dg_inputs.hidden((d.canvas, d.d_model), "bf16")
    x_dev = torch.from_numpy(x_host.view(np.int16)).cuda().view(torch.bfloat16)
    pred, conf, ent = _run_head(sess, x_dev, d.canvas)
    assert np.all((pred >= 0) & (pred < d.vocab))
    assert np.all(ent >= 0) and np.all(ent <= math.log(d.vocab) + 1e-4)
    assert np.all((conf > 0) & (conf <= 1))
    log("head C2: generating E on host for the oracle")
    E64 = numerics.from_storage(dg_inputs.embed_host(d), "bf16")
    rows = np.array([0, 1, 37, 100, 128, 200, 254, 255])
    n = _compare_head(d, x_host, x_dev, rows, pred, conf, ent, E64)
    log(f"head C2: {n}/{len(rows)} argmax decisions compared")


# ----------------------------------------------------------------------------- one layer

def _prefix_kv(d, P):
    k = dg_inputs.normal((d.n_kv_heads, P, d.head_dim), recipe.INPUT_SEED, recipe.STREAM_PREFIX_K, 1.0, d.dtype)
    v = dg_inputs.normal((d.n_kv_heads, P, d.head_dim), recipe.INPUT_SEED, recipe.STREAM_PREFIX_V, 1.0, d.dtype)
    return k, v


def _upload_prefix(sess, layer, k, v, dtype):
    P = k.shape[1]
    tk = torch.from_numpy(k.view(np.int16) if dtype == "bf16" else k).cuda()
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(0, 2, 1)).view(np.int16) if dtype == "bf16"
                          else np.ascontiguousarray(v.transpose(0, 2, 1))).cuda()
    if dtype == "bf16":
        tk, tv = tk.view(torch.bfloat16), tv.view(torch.bfloat16)
    sess.k[layer, :, :P, :] = tk
    sess.v[layer, :, :, :P] = tv
    sess.kv.len = P


def _layer_case(d, P, causal, weights_dev, layer_host):
    S = d.canvas
    sess = Session(d, capacity=P + S, weights=weights_dev)
    k, v = _prefix_kv(d, P)
    _upload_prefix(sess, 0, k, v, d.dtype)
    x_host = dg_inputs.hidden((S, d.d_model), d.dtype)
    x_dev = torch.from_numpy(x_host.view(np.int16) if d.dtype == "bf16" else x_host).cuda()
    if d.dtype == "bf16":
        x_dev = x_dev.view(torch.bfloat16)
    y_dev = torch.empty_like(x_dev)
    ridx = torch.empty((S, d.top_k), dtype=torch.int32, device="cuda")
    rw = torch.empty((S, d.top_k), dtype=torch.float32, device="cuda")
    rlog = torch.empty((S, d.n_experts), dtype=torch.float32, device="cuda")
    dg.dg_layer_forward(sess.cfg, sess.weights, 0, sess.kv, x_dev, y_dev, S, causal,
                        {"route_idx": ridx, "route_w": rw, "router_logits": rlog}, sess.ws, sess.ws_bytes)
    torch.cuda.synchronize()
    log(f"layer {d.dtype} P={P} causal={causal}: oracle")
    model = om.Model(oracle_dims(d), {"embed": None, "final_norm": None,
                                      "layers": [{n: numerics.from_storage(a, d.dtype) for n, a in layer_host.items()}]})
    kv = om.KVCache(1, d.n_kv_heads, d.head_dim)
    kv.k[0] = numerics.from_storage(k, d.dtype)
    kv.v[0] = numerics.from_storage(v, d.dtype)
    y_ref, tr = model.layer(0, numerics.from_storage(x_host, d.dtype), kv, bool(causal), append=False)
    same = compare_routing(ridx.cpu().numpy(), rw.cpu().numpy(), rlog.cpu().numpy(), tr.router_logits, tr.idx,
                           TOL[d.dtype])
    atol, rtol = TOL[d.dtype]
    y = to_f64(y_dev)
    ok, worst, at = allclose_report(y[same], y_ref[same], atol, rtol)
    assert ok, ("hidden", worst, at)
    # the canvas keys/values written to the cache match the oracle's projections
    kk, vv = sess.kv_numpy(0, P + S)
    xn = numerics.rounder(d.dtype)(om.rmsnorm(numerics.from_storage(x_host, d.dtype),
                                              model.w["layers"][0]["attn_norm"], d.rms_eps))
    qkv = xn @ model.w["layers"][0]["wqkv"].T
    hq, hkv, dh = d.n_heads, d.n_kv_heads, d.head_dim
    k_ref = numerics.rounder(d.dtype)(qkv[:, hq * dh:(hq + hkv) * dh]).reshape(S, hkv, dh).transpose(1, 0, 2)
    v_ref = numerics.rounder(d.dtype)(qkv[:, (hq + hkv) * dh:]).reshape(S, hkv, dh).transpose(1, 0, 2)
    assert allclose_report(kk[:, P:], k_ref, atol, rtol)[0]
    assert allclose_report(vv[:, P:], v_ref, atol, rtol)[0]
    assert np.array_equal(kk[:, :P], kv.k[0]) and np.array_equal(vv[:, :P], kv.v[0])
    return int((~same).sum())


@pytest.mark.parametrize("causal", [0, 1])
def test_layer_c0_fp32(causal):
    d = replace(recipe.C0.dims, n_layers=1)
    host = dg_inputs.layer_weights_host(d, 0)
    w = gdev.from_host({"embed": np.zeros((8, d.d_model), np.float32), "final_norm": np.ones(d.d_model, np.float32),
                        "layers": [host]}, "f32")
    flips = _layer_case(d, recipe.C0.prefix, causal, w, host)
    assert flips == 0


def test_layer_c1_bf16_full_size():
    d = recipe.C1.dims
    log("layer C1: device weights")
    w = {"embed": torch.zeros((8, d.d_model), dtype=torch.bfloat16, device="cuda"),
         "final_norm": torch.ones(d.d_model, dtype=torch.bfloat16, device="cuda"),
         "layers": [gdev.layer_weights_device(d, 0)]}
    log("layer C1: host weights for the oracle")
    host = dg_inputs.layer_weights_host(d, 0)
    flips = _layer_case(d, recipe.C1.prefix, 0, w, host)
    log(f"layer C1: routing near-tie flips {flips}")
    assert flips <= d.canvas // 20   # every flip is already checked to sit at a tie
