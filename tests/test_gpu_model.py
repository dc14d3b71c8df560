"""End-to-end GPU parity: prefill, denoising passes, the block loop and commit, against the oracle.

Free-running comparisons: both sides start from the seeded inputs and evolve
on their own (the GPU's canvas never feeds the oracle).  Where an argmax or a
routing decision sits within the documented tolerance of a tie, the
comparison stops at that point and says so.
"""
from __future__ import annotations

import math
import sys
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
from tests._helpers import oracle_model  # noqa: E402

F32_TOL = (1e-4, 1e-4)
BF16_TOL = (2e-2, 2e-2)
MARGIN = 1e-2     # argmax decisions compared where the fp32 top-2 margin exceeds this


def log(msg):
    print(msg, flush=True)


def _c0_pair(d=None, storage=None, prefix=None):
    d = d or recipe.C0.dims
    storage = storage if storage is not None else dg_inputs.model_weights_host(d)
    prefix = recipe.C0.prefix if prefix is None else prefix
    sess = Session(d, capacity=prefix + 4 * d.canvas, max_tokens=max(d.canvas, 64),
                   weights=gdev.from_host(storage, d.dtype))
    model = oracle_model(d, storage)
    kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    prompt = dg_inputs.prompt_tokens(prefix, d.vocab)
    if prefix:
        sess.prefill(prompt)
        osm.prefill(model, kv, prompt)
    return sess, model, kv


def _check_kv(sess, kv, tol, keep_rows=None):
    """Cache parity; keep_rows[l] (optional) selects the rows compared at layer l."""
    torch.cuda.synchronize()
    assert sess.kv.len == kv.length
    for l in range(sess.d.n_layers):
        gk, gv = sess.kv_numpy(l, kv.length)
        ok = np.ones(kv.length, dtype=bool) if keep_rows is None else keep_rows[l]
        rk = allclose_report(gk[:, ok], kv.k[l][:, ok], *tol)
        rv = allclose_report(gv[:, ok], kv.v[l][:, ok], *tol)
        assert rk[0], f"K layer {l}: worst excess {rk[1]:.3e} at {rk[2]} (rows compared {int(ok.sum())})"
        assert rv[0], f"V layer {l}: worst excess {rv[1]:.3e} at {rv[2]} (rows compared {int(ok.sum())})"


def _near_tie_rows(traces, thr):
    """keep_rows[l]: rows with no routing gap below thr at any layer before l (a near-tie upstream makes
    the two sides legitimately route that token differently)."""
    n = traces[0].gap.shape[0]
    keep = [np.ones(n, dtype=bool)]
    for tr in traces[:-1]:
        keep.append(keep[-1] & (tr.gap >= thr))
    return keep


def test_c0_prefill_matches_oracle():
    sess, model, kv = _c0_pair()
    _check_kv(sess, kv, F32_TOL)


def test_c0_prefill_chunked_equals_single_call():
    """A workspace sized for 16 rows forces 4 chunks of the 64-token prompt: same cache as the oracle."""
    d = recipe.C0.dims
    storage = dg_inputs.model_weights_host(d)
    sess = Session(d, capacity=128, max_tokens=d.canvas, weights=gdev.from_host(storage, d.dtype))
    small = dg.dg_workspace_size(sess.cfg, 16)
    prompt = dg_inputs.prompt_tokens(64, d.vocab)
    t = torch.from_numpy(prompt).cuda()
    dg.dg_prefill_kv(sess.cfg, sess.weights, sess.kv, t, 64, sess.ws, small)
    model = oracle_model(d, storage)
    kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    osm.prefill(model, kv, prompt)
    _check_kv(sess, kv, F32_TOL)


def test_c0_pass_matches_oracle_layer_by_layer():
    d = recipe.C0.dims
    sess, model, kv = _c0_pair()
    canvas = osm.initial_canvas(recipe.INPUT_SEED, 0, d.canvas, d.vocab)
    dbg = _dbg(d, torch.float32)
    pred, conf, ent = sess.denoise(canvas, dbg=dbg)
    torch.cuda.synchronize()
    hid, ridx, rw, rlog = dbg["hidden"], dbg["route_idx"], dbg["route_w"], dbg["router_logits"]
    rec, _ = osm.denoise_pass(model, kv, canvas, keep_traces=True)
    for l, tr in enumerate(rec.traces):
        compare_routing(ridx[l].cpu().numpy(), rw[l].cpu().numpy(), rlog[l].cpu().numpy(), tr.router_logits,
                        tr.idx, F32_TOL)
        ok, worst, at = allclose_report(to_f64(hid[l]), tr.hidden, *F32_TOL)
        assert ok, (l, worst, at)
    sel = rec.margin > MARGIN
    assert np.array_equal(pred.cpu().numpy()[sel], rec.pred[sel])
    assert allclose_report(to_f64(ent), rec.ent, *F32_TOL)[0]
    assert allclose_report(to_f64(conf), rec.conf, 1e-7, 1e-4)[0]
    assert kv.length == sess.kv.len == recipe.C0.prefix   # a pass does not commit


def _dbg(d, dtype):
    L, S = d.n_layers, d.canvas
    return {"hidden": torch.empty((L, S, d.d_model), dtype=dtype, device="cuda"),
            "route_idx": torch.empty((L, S, d.top_k), dtype=torch.int32, device="cuda"),
            "route_w": torch.empty((L, S, d.top_k), dtype=torch.float32, device="cuda"),
            "router_logits": torch.empty((L, S, d.n_experts), dtype=torch.float32, device="cuda")}


def _gpu_block_loop(sess, sampler_args, block):
    """The block loop driven step by step through the C ABI; returns per-pass records."""
    S, V = sess.S, sess.d.vocab
    sp = dg.make_sampler(**sampler_args)
    canvas = sess.i32(S)
    dg.dg_canvas_update(sess.cfg, None, None, 0, sp.seed, block, 0, canvas)
    prev = torch.zeros(S, dtype=torch.int32, device="cuda")
    st = torch.zeros(4, dtype=torch.int32, device="cuda")
    recs = []
    t = 0
    while True:
        t += 1
        c_now = canvas.cpu().numpy().copy()
        pred, conf, ent = sess.denoise(canvas)
        dg.dg_stop_check(sess.cfg, sp, t, ent, pred, prev, st)
        torch.cuda.synchronize()
        a = st.cpu().numpy()
        recs.append((c_now, pred.cpu().numpy(), to_f64(conf), to_f64(ent), int(a[1])))
        if a[1] != dg.DG_STOP_NONE:
            return recs, pred
        keep = min(S, t * sp.n_new)
        new = sess.i32(S)
        dg.dg_canvas_update(sess.cfg, pred, conf, keep, sp.seed, block, t, new)
        canvas = new


def _compare_trajectory(recs, res, tol):
    for t, ((g_c, g_p, g_conf, g_ent, _), o) in enumerate(zip(recs, res.passes), start=1):
        assert np.array_equal(g_c, o.canvas), f"canvas differs at pass {t}"
        if np.any(o.margin <= MARGIN) and not np.array_equal(g_p, o.pred):
            log(f"argmax near-tie at pass {t} (min margin {o.margin.min():.2e}); trajectory comparison stops")
            return False
        assert np.array_equal(g_p, o.pred), f"prediction differs at pass {t}"
        assert allclose_report(g_ent, o.ent, *tol)[0], f"entropy at pass {t}"
        assert allclose_report(g_conf, o.conf, 1e-7, tol[1])[0], f"confidence at pass {t}"
    return True


def test_c0_block_free_running_matches_oracle():
    d = recipe.C0.dims
    sess, model, kv = _c0_pair()
    res = osm.generate_block(model, kv, osm.Sampler(n_new=recipe.C0.n_new), block=0)
    recs, last_pred = _gpu_block_loop(sess, dict(n_new=recipe.C0.n_new), 0)
    log(f"C0 block: oracle {res.steps} passes reason {res.reason}; GPU {len(recs)} passes reason {recs[-1][4]}")
    if _compare_trajectory(recs, res, F32_TOL):
        assert len(recs) == res.steps and recs[-1][4] == res.reason
        assert np.array_equal(last_pred.cpu().numpy(), res.tokens)
        # commit the block: causal forward of the final predictions into the cache
        ws = sess.ws
        dg.dg_commit_block(sess.cfg, sess.weights, sess.kv, last_pred, ws, sess.ws_bytes)
        _check_kv(sess, kv, F32_TOL)


def test_c0_generate_block_equals_step_loop_and_oracle():
    """dg_generate_block (adaptive) equals the step-by-step loop bit for bit, and the oracle; then a second
    block starts from the committed cache (block-autoregressive)."""
    d = recipe.C0.dims
    sess, model, kv = _c0_pair()
    recs, loop_pred = _gpu_block_loop(sess, dict(n_new=recipe.C0.n_new), 0)
    sess2, _, _ = _c0_pair()
    out = sess2.i32(d.canvas)
    st = dg.dg_generate_block(sess2.cfg, sess2.weights, sess2.kv, dg.make_sampler(recipe.C0.n_new), 0, out,
                              sess2.ws, sess2.ws_bytes)
    assert st.steps == len(recs) and st.reason == recs[-1][4]
    assert np.array_equal(out.cpu().numpy(), loop_pred.cpu().numpy())
    assert abs(st.mean_entropy - recs[-1][3].mean()) < 1e-6 and st.flags == 0
    assert sess2.kv.len == recipe.C0.prefix + d.canvas
    res0 = osm.generate_block(model, kv, osm.Sampler(n_new=recipe.C0.n_new), block=0)
    assert (res0.steps, res0.reason) == (st.steps, st.reason)
    assert np.array_equal(res0.tokens, out.cpu().numpy())
    _check_kv(sess2, kv, F32_TOL)
    out1 = sess2.i32(d.canvas)
    st1 = dg.dg_generate_block(sess2.cfg, sess2.weights, sess2.kv, dg.make_sampler(recipe.C0.n_new), 1, out1,
                               sess2.ws, sess2.ws_bytes)
    res1 = osm.generate_block(model, kv, osm.Sampler(n_new=recipe.C0.n_new), block=1)
    log(f"C0 block 1: GPU {st1.steps} ({st1.reason}), oracle {res1.steps} ({res1.reason})")
    assert (res1.steps, res1.reason) == (st1.steps, st1.reason)
    assert np.array_equal(res1.tokens, out1.cpu().numpy())
    _check_kv(sess2, kv, F32_TOL)


def test_c0_overlapped_commits_equal_oracle_blocks():
    """Three blocks, each block's commit overlapped on the next block's first pass (that forward carries the
    committed rows causally and the canvas rows bidirectionally); the last block commits at its end.  Same
    steps, tokens and cache as the oracle's three plain blocks."""
    d = recipe.C0.dims
    sess, model, kv = _c0_pair()
    outs = [sess.i32(d.canvas) for _ in range(3)]
    pending = None
    for b in range(3):
        st = dg.dg_generate_block_overlapped(sess.cfg, sess.weights, sess.kv, dg.make_sampler(recipe.C0.n_new), b,
                                             pending, 1 if b < 2 else 0, outs[b], sess.ws, sess.ws_bytes)
        res = osm.generate_block(model, kv, osm.Sampler(n_new=recipe.C0.n_new), block=b)
        log(f"C0 overlapped block {b}: GPU {st.steps} ({st.reason}), oracle {res.steps} ({res.reason})")
        assert (res.steps, res.reason) == (st.steps, st.reason)
        assert np.array_equal(res.tokens, outs[b].cpu().numpy())
        assert sess.kv.len == recipe.C0.prefix + d.canvas * (b if b < 2 else 3)
        pending = outs[b]
    _check_kv(sess, kv, F32_TOL)


def test_bf16_overlapped_commits_against_oracle():
    """bf16 at the benchmark's widths (d 2816, 128 experts top-8, 262144 vocabulary, canvas 256; two layers):
    three blocks of one pass each, each block's commit carried by the next block's first pass (512 rows: the
    committed block causal, the canvas bidirectional over it), the last block committed at its end.  Every
    block is checked against the oracle on the GPU's context (teacher-forced): its tokens where the oracle's
    top-2 margin exceeds 1e-2 and its mean entropy, then each committed block's cache rows, every layer, at the
    bf16 bar."""
    from tests._gpu import check_commit_on_gpu_cache, check_pass_on_gpu_cache, check_prompt_cache, gpu_cache_as_oracle
    d = replace(recipe.C3.dims, n_layers=2)
    P, S = 384, d.canvas
    sess = Session(d, capacity=P + 4 * S, max_tokens=2 * S)
    prompt = dg_inputs.prompt_tokens(P, d.vocab)
    sess.prefill(prompt)
    model = oracle_model(d)
    log(f"prompt cache: {check_prompt_cache(sess, model, prompt, BF16_TOL)} rows near a routing tie left out")
    sp = dg.make_sampler(26, fixed_steps=1)
    outs = [sess.i32(S) for _ in range(3)]
    pending = None
    for b in range(3):
        st = dg.dg_generate_block_overlapped(sess.cfg, sess.weights, sess.kv, sp, b, pending, 1 if b < 2 else 0,
                                             outs[b], sess.ws, sess.ws_bytes, side=sess.side)
        torch.cuda.synchronize()
        assert (st.steps, st.reason) == (1, dg.DG_STOP_FIXED)
        toks = outs[b].cpu().numpy()
        if pending is not None:  # the previous block, committed inside this block's first pass
            check_commit_on_gpu_cache(model, gpu_cache_as_oracle(sess, P + (b - 1) * S), outs[b - 1].cpu().numpy(),
                                      sess, BF16_TOL)
        n = check_pass_on_gpu_cache(model, gpu_cache_as_oracle(sess, P + b * S),
                                    osm.initial_canvas(sp.seed, b, S, d.vocab), toks, st.mean_entropy, BF16_TOL)
        log(f"overlapped block {b}: {n}/{S} tokens compared, mean entropy {st.mean_entropy:.4f}")
        pending = outs[b]
    assert sess.kv.len == P + 3 * S
    check_commit_on_gpu_cache(model, gpu_cache_as_oracle(sess, P + 2 * S), outs[2].cpu().numpy(), sess, BF16_TOL)


def test_c0_fixed_T_block():
    d = recipe.C0.dims
    sess, model, kv = _c0_pair()
    out = sess.i32(d.canvas)
    st = dg.dg_generate_block(sess.cfg, sess.weights, sess.kv, dg.make_sampler(recipe.C0.n_new, fixed_steps=10), 0,
                              out, sess.ws, sess.ws_bytes)
    res = osm.generate_block(model, kv, osm.Sampler(n_new=recipe.C0.n_new, fixed_steps=10), block=0)
    assert st.steps == 10 and st.reason == dg.DG_STOP_FIXED == res.reason and res.steps == 10
    assert np.array_equal(out.cpu().numpy(), res.tokens)


def test_stop_e1_uniform_logits_gpu():
    d = replace(recipe.C0.dims, n_layers=1)
    st_h = dg_inputs.model_weights_host(d)
    st_h["embed"] = np.zeros_like(st_h["embed"])
    sess, _, _ = _c0_pair(d, st_h, prefix=0)
    out = sess.i32(d.canvas)
    st = dg.dg_generate_block(sess.cfg, sess.weights, sess.kv, dg.make_sampler(4), 0, out, sess.ws, sess.ws_bytes)
    assert (st.steps, st.reason) == (2, dg.DG_STOP_STABLE)
    assert abs(st.mean_entropy - math.log(d.vocab)) < 1e-4
    assert np.all(out.cpu().numpy() == 0)


def test_stop_e2_self_retrieval_gpu():
    d = replace(recipe.C0.dims, n_layers=1)
    st_h = dg_inputs.model_weights_host(d)
    for layer in st_h["layers"]:
        for n in ("wo", "w_down", "ws_down"):
            layer[n] = np.zeros_like(layer[n])
    st_h["final_norm"] = dg_inputs.const(st_h["final_norm"].shape, 10.0, d.dtype)
    sess, _, _ = _c0_pair(d, st_h, prefix=0)
    out = sess.i32(d.canvas)
    st = dg.dg_generate_block(sess.cfg, sess.weights, sess.kv, dg.make_sampler(4), 0, out, sess.ws, sess.ws_bytes)
    assert (st.steps, st.reason) == (1, dg.DG_STOP_ENTROPY)
    assert np.array_equal(out.cpu().numpy(), osm.initial_canvas(recipe.INPUT_SEED, 0, d.canvas, d.vocab))


def test_deterministic_bitwise():
    """Repeated passes are bit-identical, and so is a pass whose shared expert runs on the caller's stream
    (no dg_side) instead of the side stream."""
    d = replace(recipe.C3.dims, n_layers=2)
    sess = Session(d, capacity=512)
    canvas = gdev.uniform_tensor(d.canvas, 9, 9, d.vocab)
    a = [x.clone() for x in sess.denoise(canvas)]
    b = [x.clone() for x in sess.denoise(canvas)]
    c = [sess.i32(d.canvas), sess.f32(d.canvas), sess.f32(d.canvas)]
    dg.dg_denoise_step(sess.cfg, sess.weights, sess.kv, canvas, 1.0, *c, None, sess.ws, sess.ws_bytes, side=None)
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(x, z)


def test_full_width_two_layers_end_to_end():
    """Two layers at the full widths (d 2816, 16 q / 8 KV heads of 128, 262144 vocab, bf16) with a 256-token
    prompt, every row compared: prefill cache (free-running, both layers), layer 0 of the pass (free-running),
    layer 1 of the pass teacher-forced (the oracle's layer 1 takes the GPU's layer-0 rows and the GPU's layer-1
    cache), routing and sampled head outputs, all at the bf16 bar.

    Routing here selects all 16 of 16 experts (the dense-mixture end of the router; top-8 of 128 is compared
    layer by layer, teacher-forced, at the benchmarked configuration in test_gpu_teacher_forced.py)."""
    d = replace(recipe.C3.dims, n_layers=2, n_experts=16, top_k=16)
    P = 256
    log("full-width: device weights")
    sess = Session(d, capacity=P + d.canvas, max_tokens=d.canvas)
    prompt = dg_inputs.prompt_tokens(P, d.vocab)
    sess.prefill(prompt)
    canvas = osm.initial_canvas(recipe.INPUT_SEED, 0, d.canvas, d.vocab)
    dbg = _dbg(d, torch.bfloat16)
    pred, conf, ent = sess.denoise(canvas, dbg=dbg)
    torch.cuda.synchronize()
    hid, ridx, rw, rlog = dbg["hidden"], dbg["route_idx"], dbg["route_w"], dbg["router_logits"]
    log("full-width: host weights + oracle")
    model = oracle_model(d)
    kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    osm.prefill(model, kv, prompt)
    _check_kv(sess, kv, BF16_TOL)
    x = model.embed(canvas)
    for l in range(d.n_layers):
        if l > 0:  # teacher-forced: the GPU's input rows and the GPU's cache of this layer
            x = to_f64(hid[l - 1])
            gk, gv = sess.kv_numpy(l, P)
            kv.k[l], kv.v[l] = gk, gv
        x, tr = model.layer(l, x, kv, causal=False, append=False)
        same = compare_routing(ridx[l].cpu().numpy(), rw[l].cpu().numpy(), rlog[l].cpu().numpy(),
                               tr.router_logits, tr.idx, BF16_TOL)
        assert same.all()
        ok, worst, at = allclose_report(to_f64(hid[l]), tr.hidden, *BF16_TOL)
        log(f"full-width layer {l}: worst excess {worst:+.2e}")
        assert ok, (l, worst, at)
    x = to_f64(hid[d.n_layers - 1])
    rows = np.array([0, 3, 77, 128, 255])
    opred, oconf, oent, margin = om.head_stats(x[rows], model.w["final_norm"], model.w["embed"], 1.0, d.rms_eps,
                                               numerics.bf16_round)
    sel = margin > MARGIN
    assert np.array_equal(pred.cpu().numpy()[rows][sel], opred[sel])
    assert allclose_report(to_f64(ent)[rows], oent, *BF16_TOL)[0]
    log(f"full-width: {int(sel.sum())}/{len(rows)} argmax compared")


def test_prefill_equals_layer_by_layer_replay():
    """dg_prefill_kv and a causal dg_layer_forward replay of the same prompt write identical caches (bf16,
    full widths, top-8 of 128)."""
    d = replace(recipe.C3.dims, n_layers=2)
    P = 256
    sess = Session(d, capacity=P + d.canvas, max_tokens=d.canvas)
    prompt = dg_inputs.prompt_tokens(P, d.vocab)
    sess.prefill(prompt)
    sess2 = Session(d, capacity=P + d.canvas, max_tokens=d.canvas, weights=sess.w, packed=True)
    x = torch.from_numpy(dg_inputs.embed_host(d, rows=prompt).view(np.int16)).cuda().view(torch.bfloat16)
    for l in range(d.n_layers):
        y = torch.empty_like(x)
        dg.dg_layer_forward(sess2.cfg, sess2.weights, l, sess2.kv, x, y, P, 1, None, sess2.ws, sess2.ws_bytes)
        x = y
    torch.cuda.synchronize()
    for l in range(d.n_layers):
        assert torch.equal(sess2.k[l, :, :P], sess.k[l, :, :P])
        assert torch.equal(sess2.v[l, :, :, :P], sess.v[l, :, :, :P])


def test_c3_bench_configuration_layer0_and_properties():
    """The benchmarked configuration itself (30 layers, 4096-token prompt, bf16): layer 0 of a pass against
    the oracle (layer 0 depends only on the embeddings of the prompt and canvas), output ranges, and a
    fixed T=10 block with its commit."""
    wl = recipe.C3
    d = wl.dims
    log("C3: device weights (49.6 GB)")
    sess = Session(d, capacity=wl.prefix + 2 * d.canvas, max_tokens=d.canvas)
    prompt = dg_inputs.prompt_tokens(wl.prefix, d.vocab)
    log("C3: prefill 4096")
    sess.prefill(prompt)
    canvas = osm.initial_canvas(recipe.INPUT_SEED, 0, d.canvas, d.vocab)
    dbg = _dbg(d, torch.bfloat16)
    pred, conf, ent = sess.denoise(canvas, dbg=dbg)
    torch.cuda.synchronize()
    hid, ridx, rw, rlog = dbg["hidden"], dbg["route_idx"], dbg["route_w"], dbg["router_logits"]
    e = to_f64(ent)
    assert np.all(np.isfinite(to_f64(hid)))
    assert np.all(e >= 0) and np.all(e <= math.log(d.vocab) + 1e-4)
    assert np.all((pred.cpu().numpy() >= 0) & (pred.cpu().numpy() < d.vocab))
    # layer 0 against the oracle: prefix keys/values of layer 0 are projections of the prompt embeddings
    log("C3: oracle layer 0")
    d1 = replace(d, n_layers=1)
    lw = {n: numerics.from_storage(a, "bf16") for n, a in dg_inputs.layer_weights_host(d, 0).items()}
    rows = np.concatenate([prompt, canvas])
    E_rows = numerics.from_storage(dg_inputs.embed_host(d, rows=rows), "bf16")
    model = om.Model(om.Dims(**{f: getattr(d1, f) for f in om.Dims.__dataclass_fields__}),
                     {"embed": None, "final_norm": None, "layers": [lw]})
    xn = numerics.bf16_round(om.rmsnorm(E_rows[:wl.prefix], lw["attn_norm"], d.rms_eps))
    hq, hkv, dh = d.n_heads, d.n_kv_heads, d.head_dim
    kvp = xn @ lw["wqkv"][hq * dh:].T
    kv = om.KVCache(1, hkv, dh)
    kv.k[0] = numerics.bf16_round(kvp[:, :hkv * dh]).reshape(-1, hkv, dh).transpose(1, 0, 2)
    kv.v[0] = numerics.bf16_round(kvp[:, hkv * dh:]).reshape(-1, hkv, dh).transpose(1, 0, 2)
    gk, gv = sess.kv_numpy(0, wl.prefix)
    assert allclose_report(gk, kv.k[0], *BF16_TOL)[0] and allclose_report(gv, kv.v[0], *BF16_TOL)[0]
    x0, tr = model.layer(0, E_rows[wl.prefix:], kv, causal=False, append=False)
    same = compare_routing(ridx[0].cpu().numpy(), rw[0].cpu().numpy(), rlog[0].cpu().numpy(), tr.router_logits,
                           tr.idx, BF16_TOL)
    assert allclose_report(to_f64(hid[0])[same], x0[same], *BF16_TOL)[0]
    # fixed T=10 block + commit
    out = sess.i32(d.canvas)
    st = dg.dg_generate_block(sess.cfg, sess.weights, sess.kv, dg.make_sampler(wl.n_new, fixed_steps=10), 0, out,
                              sess.ws, sess.ws_bytes)
    assert (st.steps, st.reason) == (10, dg.DG_STOP_FIXED)
    assert sess.kv.len == wl.prefix + d.canvas
    o = out.cpu().numpy()
    assert np.all((o >= 0) & (o < d.vocab))
    log(f"C3: mean entropy after 10 passes {st.mean_entropy:.4f} (ln V = {math.log(d.vocab):.4f})")
