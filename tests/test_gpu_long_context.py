"""Long-context parity: one MoE layer of the 30-layer model over a 131072-token cache, against the oracle.

The long-context workload differs from the others only in the length of the key range, which is
where the attention kernel's chunking, key splits and tail handling matter.  The oracle evaluates
the same layer for a sample of rows (every row's keys and values still enter the attention), on
the cache drawn N(0,1) in bf16 (the single-layer workload's reading of a prefix cache), for

  * a denoising pass: the 256 canvas rows attend to all 131072 + 256 keys, no mask;
  * the last prefill chunk: 2048 rows at positions 129024..131071 attend causally.
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
from tests._gpu import Session, allclose_report, compare_routing, to_f64  # noqa: E402
from tests._helpers import oracle_dims  # noqa: E402

BF16_TOL = (2e-2, 2e-2)


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def layer0():
    d = replace(recipe.C4.dims, n_layers=1)
    log("long context: device weights of one layer")
    w = {"embed": torch.zeros((8, d.d_model), dtype=torch.bfloat16, device="cuda"),
         "final_norm": torch.ones(d.d_model, dtype=torch.bfloat16, device="cuda"),
         "layers": [gdev.layer_weights_device(d, 0)]}
    log("long context: host weights for the oracle")
    host = dg_inputs.layer_weights_host(d, 0)
    model = om.Model(oracle_dims(d), {"embed": None, "final_norm": None,
                                      "layers": [{n: numerics.from_storage(a, "bf16") for n, a in host.items()}]})
    return d, w, model


def _bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _run(d, w, model, P, M, causal, rows):
    sess = Session(d, capacity=P + M, max_tokens=M, weights=w)
    log(f"long context: prefix cache of {P} keys")
    k = dg_inputs.normal((d.n_kv_heads, P, d.head_dim), recipe.INPUT_SEED, recipe.STREAM_PREFIX_K, 1.0, "bf16")
    v = dg_inputs.normal((d.n_kv_heads, P, d.head_dim), recipe.INPUT_SEED, recipe.STREAM_PREFIX_V, 1.0, "bf16")
    sess.k[0, :, :P, :] = _bf16_dev(k)
    sess.v[0, :, :, :P] = _bf16_dev(v.transpose(0, 2, 1))
    sess.kv.len = P
    x_host = dg_inputs.hidden((M, d.d_model), "bf16")
    x_dev = _bf16_dev(x_host)
    y_dev = torch.empty_like(x_dev)
    ridx = torch.empty((M, d.top_k), dtype=torch.int32, device="cuda")
    rw = torch.empty((M, d.top_k), dtype=torch.float32, device="cuda")
    rlog = torch.empty((M, d.n_experts), dtype=torch.float32, device="cuda")
    print(f"long context: layer forward P={P} M={M} causal={causal}", flush=True)
    dg.dg_layer_forward(sess.cfg, sess.weights, 0, sess.kv, x_dev, y_dev, M, causal,
                        {"route_idx": ridx, "route_w": rw, "router_logits": rlog}, sess.ws, sess.ws_bytes)
    torch.cuda.synchronize()
    assert sess.kv.len == P
    log("long context: oracle on sampled rows")
    kv = om.KVCache(1, d.n_kv_heads, d.head_dim)
    kv.k[0] = numerics.from_storage(k, "bf16")
    kv.v[0] = numerics.from_storage(v, "bf16")
    x64 = numerics.from_storage(x_host, "bf16")
    y_ref, tr = model.layer_rows(0, x64, kv, bool(causal), rows)
    same = compare_routing(ridx.cpu().numpy()[rows], rw.cpu().numpy()[rows], rlog.cpu().numpy()[rows],
                           tr.router_logits, tr.idx, BF16_TOL)
    y = to_f64(y_dev)[rows]
    ok, worst, at = allclose_report(y[same], y_ref[same], *BF16_TOL)
    assert ok, ("hidden", worst, at)
    # the new rows' keys/values in the cache, all of them
    lw = model.w["layers"][0]
    hq, hkv, dh = d.n_heads, d.n_kv_heads, d.head_dim
    xn = numerics.bf16_round(om.rmsnorm(x64, lw["attn_norm"], d.rms_eps))
    kvp = xn @ lw["wqkv"][hq * dh:].T
    k_ref = numerics.bf16_round(kvp[:, :hkv * dh]).reshape(M, hkv, dh).transpose(1, 0, 2)
    v_ref = numerics.bf16_round(kvp[:, hkv * dh:]).reshape(M, hkv, dh).transpose(1, 0, 2)
    kk = sess.k[0, :, P:P + M, :].float().cpu().numpy().astype(np.float64)
    vv = sess.v[0, :, :, P:P + M].float().cpu().numpy().astype(np.float64).transpose(0, 2, 1)
    assert allclose_report(kk, k_ref, *BF16_TOL)[0]
    assert allclose_report(vv, v_ref, *BF16_TOL)[0]
    return int((~same).sum())


def test_long_context_canvas_layer_sampled_rows(layer0):
    d, w, model = layer0
    rows = np.array([0, 1, 77, 128, 200, 254, 255])
    flips = _run(d, w, model, recipe.C4.prefix, d.canvas, 0, rows)
    assert flips <= 1


def test_long_context_last_prefill_chunk_sampled_rows(layer0):
    d, w, model = layer0
    M = 2048
    rows = np.array([0, 1, 31, 32, 1000, 2046, 2047])
    flips = _run(d, w, model, recipe.C4.prefix - M, M, 1, rows)
    assert flips <= 1
