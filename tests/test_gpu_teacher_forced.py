"""Teacher-forced parity at the benchmarked configuration, every layer.

The benchmarked workload is the 30-layer bf16 model (d 2816, 16 query / 8 KV heads of 128, top-8 of 128
experts + 1 shared, 262144-token tied vocabulary) over a 4096-token prompt.  A free-running comparison of
30 bf16 layers stops meaning anything after the first near-tie, so each layer is compared on the GPU's own
input ([P2] "DiffusionGemma 26B: How Google's Text Diffusion Model Generates Tokens in Parallel", "How
Diffusion Changes the Equation": every pass predicts every slot through the whole stack):

  * prefill: the prompt runs layer by layer through dg_layer_forward (two causal chunks of 2048 rows, the
    same arithmetic as dg_prefill_kv); for layer l the oracle takes the GPU's input rows of that layer and
    forms every prompt row's keys and values (compared with the GPU's cache rows, all of them) and the
    layer's output on sampled rows (compared where the routing agrees);
  * the canvas pass: dg_denoise_step dumps every layer's output; for layer l the oracle takes the GPU's
    layer input and the GPU's cache of that layer and computes the layer over all 256 canvas rows
    (hidden states where the routing agrees, the canvas keys/values, all rows);
  * the head: the oracle's fused-head statistics on the GPU's final hidden rows, all 256 slots.

Bars: hidden states, keys and values |gpu - oracle| <= 2e-2 + 2e-2 |oracle| (bf16); routing by
compare_routing; argmax where the oracle's top-2 margin exceeds 1e-2; entropy 2e-2, confidence 2e-2.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
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
from tests._helpers import oracle_dims  # noqa: E402

BF16_TOL = (2e-2, 2e-2)
MARGIN = 1e-2
CHUNK = 2048


def log(msg):
    print(msg, flush=True)


def _dbg_rows(d, n, with_hidden_layers=0):
    out = {"route_idx": torch.empty((max(with_hidden_layers, 1), n, d.top_k), dtype=torch.int32, device="cuda"),
           "route_w": torch.empty((max(with_hidden_layers, 1), n, d.top_k), dtype=torch.float32, device="cuda"),
           "router_logits": torch.empty((max(with_hidden_layers, 1), n, d.n_experts), dtype=torch.float32,
                                        device="cuda")}
    if with_hidden_layers:
        out["hidden"] = torch.empty((with_hidden_layers, n, d.d_model), dtype=torch.bfloat16, device="cuda")
    else:
        out = {k: v[0] for k, v in out.items()}
    return out


@pytest.fixture(scope="module")
def c3_run():
    """The GPU side, once: the prompt run layer by layer through dg_layer_forward (each layer's input rows kept),
    then one canvas pass with per-layer dumps."""
    wl = recipe.C3
    d = wl.dims
    P, S, L = wl.prefix, d.canvas, d.n_layers
    log(f"C3 teacher-forced: device weights ({L} layers)")
    sess = Session(d, capacity=P + 2 * S, max_tokens=CHUNK)
    prompt = dg_inputs.prompt_tokens(P, d.vocab)
    emb_nat = gdev.normal_tensor((d.vocab, d.d_model), recipe.WEIGHT_SEED, recipe.STREAM_EMBED, recipe.WEIGHT_SIGMA,
                                 "bf16")
    x = emb_nat[torch.from_numpy(prompt.astype(np.int64)).cuda()].contiguous()
    del emb_nat
    # prefill layer by layer: pre_in[l] are the prompt rows entering layer l
    sample = np.array([0, 1, 2, 63, 64, 1000, 2046, 2047, 2048, 2049, 3000, 4094, 4095])
    pre_in, pre_out, pre_route = [], [], []
    for l in range(L):
        y = torch.empty_like(x)
        route = {k: [] for k in ("route_idx", "route_w", "router_logits")}
        for c0 in range(0, P, CHUNK):
            dbg = _dbg_rows(d, CHUNK)
            sess.kv.len = c0
            dg.dg_layer_forward(sess.cfg, sess.weights, l, sess.kv, x[c0:c0 + CHUNK], y[c0:c0 + CHUNK], CHUNK, 1, dbg,
                                sess.ws, sess.ws_bytes, side=sess.side)
            for k in route:
                route[k].append(dbg[k].cpu().numpy())
        torch.cuda.synchronize()
        pre_in.append(x.cpu())
        pre_out.append(y[torch.from_numpy(sample).cuda()].cpu())
        pre_route.append({k: np.concatenate(v)[sample] for k, v in route.items()})
        x = y
    sess.kv.len = P
    del x, y
    log("C3 teacher-forced: one canvas pass with per-layer dumps")
    canvas = osm.initial_canvas(recipe.INPUT_SEED, 0, S, d.vocab)
    dbg = _dbg_rows(d, S, with_hidden_layers=L)
    pred, conf, ent = sess.denoise(canvas, dbg=dbg)
    torch.cuda.synchronize()
    run = dict(d=d, P=P, S=S, L=L, sample=sample, pre_in=pre_in, pre_out=pre_out, pre_route=pre_route,
               hid=dbg["hidden"].cpu(), ridx=dbg["route_idx"].cpu().numpy(), rw=dbg["route_w"].cpu().numpy(),
               rlog=dbg["router_logits"].cpu().numpy(), kv_np=[sess.kv_numpy(l, P + S) for l in range(L)],
               emb_rows=numerics.from_storage(dg_inputs.embed_host(d, rows=canvas), "bf16"),
               pred=pred.cpu().numpy(), conf=to_f64(conf), ent=to_f64(ent))
    del sess
    torch.cuda.empty_cache()
    return run


def _check_layer(run, l):
    d, P, S, sample = run["d"], run["P"], run["S"], run["sample"]
    lw = {n: numerics.from_storage(a, "bf16") for n, a in dg_inputs.layer_weights_host(d, l).items()}
    model = om.Model(oracle_dims(replace(d, n_layers=1)), {"embed": None, "final_norm": None, "layers": [lw]})
    rep = {"layer": l}
    # prefill: every prompt row's keys/values, sampled rows' outputs, on the GPU's input rows of this layer
    x_in = run["pre_in"][l].float().numpy().astype(np.float64)
    empty = om.KVCache(1, d.n_kv_heads, d.head_dim)
    y_ref, tr, k_ref, v_ref = model.layer_rows(0, x_in, empty, True, sample, return_kv=True)
    gk, gv = run["kv_np"][l]
    rep["prefill_k"] = allclose_report(gk[:, :P], k_ref, *BF16_TOL)
    rep["prefill_v"] = allclose_report(gv[:, :P], v_ref, *BF16_TOL)
    r = run["pre_route"][l]
    same = compare_routing(r["route_idx"], r["route_w"], r["router_logits"], tr.router_logits, tr.idx, BF16_TOL)
    y = run["pre_out"][l].float().numpy().astype(np.float64)
    rep["prefill_out"] = allclose_report(y[same], y_ref[same], *BF16_TOL)
    rep["prefill_routing_flips"] = int((~same).sum())
    del x_in, k_ref, v_ref
    # canvas pass on the GPU's layer input and the GPU's cache of this layer
    xc = run["emb_rows"] if l == 0 else run["hid"][l - 1].float().numpy().astype(np.float64)
    kv = om.KVCache(1, d.n_kv_heads, d.head_dim)
    kv.k[0], kv.v[0] = gk[:, :P], gv[:, :P]
    xo, tr = model.layer(0, xc, kv, causal=False, append=True)
    same = compare_routing(run["ridx"][l], run["rw"][l], run["rlog"][l], tr.router_logits, tr.idx, BF16_TOL)
    g = run["hid"][l].float().numpy().astype(np.float64)
    rep["canvas_out"] = allclose_report(g[same], xo[same], *BF16_TOL)
    rep["canvas_routing_flips"] = int((~same).sum())
    rep["canvas_k"] = allclose_report(gk[:, P:P + S], kv.k[0][:, P:], *BF16_TOL)
    rep["canvas_v"] = allclose_report(gv[:, P:P + S], kv.v[0][:, P:], *BF16_TOL)
    return rep


@pytest.mark.parametrize("first", [0, 10, 20], ids=["layers_0_9", "layers_10_19", "layers_20_29"])
def test_c3_teacher_forced_layers(c3_run, first):
    """Ten layers of the benchmarked configuration, each on the GPU's own inputs (prefill and canvas pass)."""
    layers = range(first, min(first + 10, c3_run["L"]))
    failures = []
    with ThreadPoolExecutor(max_workers=min(5, os.cpu_count() or 1)) as ex:
        for rep in ex.map(lambda l: _check_layer(c3_run, l), layers):
            bad = [k for k, v in rep.items() if isinstance(v, tuple) and not v[0]]
            log(f"layer {rep['layer']:2d}: routing flips prefill {rep['prefill_routing_flips']}/{len(c3_run['sample'])} "
                f"canvas {rep['canvas_routing_flips']}/{c3_run['S']}; worst excess "
                + " ".join(f"{k} {v[1]:+.2e}" for k, v in rep.items() if isinstance(v, tuple))
                + (f"  FAIL {bad}" if bad else ""))
            if bad:
                failures.append((rep["layer"], bad))
            assert rep["canvas_routing_flips"] <= 4 and rep["prefill_routing_flips"] <= 1, rep
    assert not failures, failures


def test_c3_teacher_forced_head(c3_run):
    """The head's statistics on the GPU's final hidden rows, every slot."""
    d, L, S = c3_run["d"], c3_run["L"], c3_run["S"]
    E = numerics.from_storage(dg_inputs.embed_host(d), "bf16")
    opred, oconf, oent, margin = om.head_stats(c3_run["hid"][L - 1].float().numpy().astype(np.float64),
                                               np.ones(d.d_model), E, 1.0, d.rms_eps, numerics.bf16_round)
    sel = margin > MARGIN
    assert np.array_equal(c3_run["pred"][sel], opred[sel])
    ok_e = allclose_report(c3_run["ent"], oent, *BF16_TOL)
    ok_c = allclose_report(c3_run["conf"], oconf, *BF16_TOL)
    log(f"head: {int(sel.sum())}/{S} argmax compared; worst excess entropy {ok_e[1]:+.2e} conf {ok_c[1]:+.2e}")
    assert ok_e[0] and ok_c[0]
