"""GPU parity of the self-speculative verify (dg_verify_block) against the oracle: the causal pass's greedy
predictions, the accepted count, the next token and the kept cache rows.

fp32: predictions bit-exact (every margin here is far above rounding), caches within 1e-4; bf16: predictions
compared where the oracle's top-2 margin exceeds 1e-2, the accepted count checked against the rule on the GPU's
own predictions.
"""
from __future__ import annotations

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
from oracle import sampler as osm  # noqa: E402
from tests._gpu import Session, allclose_report  # noqa: E402
from tests._helpers import oracle_model  # noqa: E402

F32_TOL = (1e-4, 1e-4)
BF16_TOL = (2e-2, 2e-2)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _pair(d, storage, prefix):
    sess = Session(d, capacity=prefix + 2 * d.canvas, weights=gdev.from_host(storage, d.dtype))
    model = oracle_model(d, storage)
    kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    prompt = dg_inputs.prompt_tokens(prefix, d.vocab)
    sess.prefill(prompt)
    osm.prefill(model, kv, prompt)
    return sess, model, kv, prompt


def _verify(sess, draft):
    ar = sess.i32(sess.S)
    t = torch.from_numpy(np.asarray(draft, dtype=np.int32)).cuda()
    n, nxt = dg.dg_verify_block(sess.cfg, sess.weights, sess.kv, t, ar, sess.ws, sess.ws_bytes)
    torch.cuda.synchronize()
    return n, nxt, ar.cpu().numpy()


def _greedy(model, prompt, count):
    kv = om.KVCache(model.d.n_layers, model.d.n_kv_heads, model.d.head_dim)
    h, _ = model.body(model.embed(prompt), kv, causal=True, append=True)
    tok = int(model.head(h[-1:])[0][0])
    out = []
    for _ in range(count):
        out.append(tok)
        h, _ = model.body(model.embed([tok]), kv, causal=True, append=True)
        tok = int(model.head(h)[0][0])
    return out


@pytest.mark.parametrize("kind", ["diffusion_draft", "greedy_prefix"])
def test_c0_verify_equals_oracle(kind):
    """A diffusion draft (the oracle's block with the commit deferred) and a draft opening with 8 tokens of the
    causal model's own greedy continuation: predictions, count, next token and cache equal the oracle's."""
    d = recipe.C0.dims
    storage = dg_inputs.model_weights_host(d)
    sess, model, kv, prompt = _pair(d, storage, recipe.C0.prefix)
    if kind == "diffusion_draft":
        draft = osm.generate_block(model, kv, osm.Sampler(n_new=recipe.C0.n_new), block=0, do_commit=False).tokens
    else:
        draft = np.array(_greedy(model, prompt, 8) + list(dg_inputs.prompt_tokens(d.canvas - 8, d.vocab, seed=9)))
    n, nxt, ar = _verify(sess, draft)
    ref = osm.verify_block(model, kv, draft)
    log(f"{kind}: accepted GPU {n}, oracle {ref.accepted}; min margin {ref.margin.min():.2e}")
    assert np.array_equal(ar, ref.ar_pred)
    assert (n, nxt) == (ref.accepted, ref.next_token)
    if kind == "greedy_prefix":
        assert n >= 8
    assert sess.kv.len == kv.length == recipe.C0.prefix + n
    for l in range(d.n_layers):
        gk, gv = sess.kv_numpy(l, kv.length)
        assert allclose_report(gk, kv.k[l], *F32_TOL)[0] and allclose_report(gv, kv.v[l], *F32_TOL)[0], l


def test_copy_model_accepts_leading_run():
    """Attention and expert outputs zeroed, final gain 10: each row predicts its own token, so the accepted count
    is the length of the draft's leading run (the whole canvas, part of it, or only the first token)."""
    d = recipe.C0.dims
    st = dg_inputs.model_weights_host(d)
    for layer in st["layers"]:
        layer["wo"] = np.zeros_like(layer["wo"])
        layer["w_down"] = np.zeros_like(layer["w_down"])
        layer["ws_down"] = np.zeros_like(layer["ws_down"])
    st["final_norm"] = dg_inputs.const(st["final_norm"].shape, 10.0, d.dtype)
    S = d.canvas
    for draft, n_expect in [([5] * S, S), ([5] * 11 + [7] * (S - 11), 11), ([9] + [8] * (S - 1), 1)]:
        sess, _, _, _ = _pair(d, st, 6)
        n, nxt, ar = _verify(sess, draft)
        assert np.array_equal(ar, draft)
        assert (n, nxt) == (n_expect, draft[n_expect - 1])
        assert sess.kv.len == 6 + n_expect


def test_bf16_verify_rule_and_cache():
    d = replace(recipe.C0.dims, dtype="bf16")
    storage = dg_inputs.model_weights_host(d)
    sess, model, kv, prompt = _pair(d, storage, recipe.C0.prefix)
    draft = np.array(_greedy(model, prompt, 6) + list(dg_inputs.prompt_tokens(d.canvas - 6, d.vocab, seed=4)))
    n, nxt, ar = _verify(sess, draft)
    # the rule on the GPU's own predictions
    m = 1
    while m < d.canvas and ar[m - 1] == draft[m]:
        m += 1
    assert (n, nxt) == (m, ar[m - 1])
    ref = osm.verify_block(model, kv, draft)
    sel = ref.margin > 1e-2
    assert np.array_equal(ar[sel], ref.ar_pred[sel])
    if np.all(sel[:max(n, ref.accepted)]):
        assert n == ref.accepted
    keep = min(n, ref.accepted)
    for l in range(d.n_layers):
        gk, gv = sess.kv_numpy(l, recipe.C0.prefix + keep)
        assert allclose_report(gk, kv.k[l][:, :recipe.C0.prefix + keep], *BF16_TOL)[0]
        assert allclose_report(gv, kv.v[l][:, :recipe.C0.prefix + keep], *BF16_TOL)[0]


def test_c0_ragged_canvas_verify():
    d = replace(recipe.C0.dims, canvas=71)
    storage = dg_inputs.model_weights_host(d)
    sess, model, kv, prompt = _pair(d, storage, 45)
    draft = np.array(_greedy(model, prompt, 5) + list(dg_inputs.prompt_tokens(d.canvas - 5, d.vocab, seed=3)))
    n, nxt, ar = _verify(sess, draft)
    ref = osm.verify_block(model, kv, draft)
    assert np.array_equal(ar, ref.ar_pred) and (n, nxt) == (ref.accepted, ref.next_token) and n >= 5
    for l in range(d.n_layers):
        gk, gv = sess.kv_numpy(l, kv.length)
        assert allclose_report(gk, kv.k[l], *F32_TOL)[0] and allclose_report(gv, kv.v[l], *F32_TOL)[0], l


# ----------------------------------------------------------------------------- the self-speculative loop

def _moving_chain_storage(d):
    """Seeded weights with the output projections scaled up 30 times: the layer, not the embedding, decides the
    head's argmax, so the greedy chain moves from token to token and some diffusion drafts agree with it."""
    st = dg_inputs.model_weights_host(d)
    for layer in st["layers"]:
        for n in ("wo", "w_down", "ws_down"):
            layer[n] = (layer[n] * 30.0).astype(np.float32)
    return st


@pytest.mark.parametrize("canvas,vocab", [(8, 64), (32, 4096)])
def test_c0_speculative_loop_equals_oracle(canvas, vocab):
    """dg_generate_speculative against the oracle's loop (fp32): the same tokens (greedy autoregressive decoding
    from the known first token), the same accepted count per round, the same committed cache."""
    d = replace(recipe.C0.dims, canvas=canvas, vocab=vocab, n_layers=1)
    storage = _moving_chain_storage(d)
    n_tokens, first = 3 * canvas // 2, 7
    sess = Session(d, capacity=16 + n_tokens + canvas + 32, weights=gdev.from_host(storage, d.dtype))
    model = oracle_model(d, storage)
    kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
    prompt = dg_inputs.prompt_tokens(16, d.vocab)
    sess.prefill(prompt)
    osm.prefill(model, kv, prompt)
    sp = dg.make_sampler(max(1, canvas // 4), fixed_steps=3)
    out = sess.i32(n_tokens)
    st, acc = dg.dg_generate_speculative(sess.cfg, sess.weights, sess.kv, sp, 5, first, n_tokens, out, sess.ws,
                                         sess.ws_bytes, side=sess.side)
    torch.cuda.synchronize()
    ref = osm.generate_speculative(model, kv, osm.Sampler(n_new=max(1, canvas // 4), fixed_steps=3), block0=5,
                                   first_token=first, n_tokens=n_tokens)
    log(f"speculative S={canvas}: GPU rounds {st.rounds} accepted {acc}; oracle {ref.accepted}")
    assert np.array_equal(out.cpu().numpy(), ref.tokens)
    assert acc == ref.accepted and st.rounds == len(ref.accepted) and st.accepted == sum(ref.accepted)
    assert st.tokens == n_tokens and sess.kv.len == kv.length
    for l in range(d.n_layers):
        gk, gv = sess.kv_numpy(l, kv.length)
        assert allclose_report(gk, kv.k[l], 1e-4, 1e-4)[0] and allclose_report(gv, kv.v[l], 1e-4, 1e-4)[0]
