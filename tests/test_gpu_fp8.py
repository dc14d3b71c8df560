"""GPU parity of the FP8 routed experts and the FP8 vocab head (OCP E4M3 weights, one float scale per output
channel or vocabulary row, bf16 activations) against the oracle's FP8 model.

The pages' headline figures run FP8 weights ([P2] "DiffusionGemma 26B: How Google's Text Diffusion Model
Generates Tokens in Parallel", "Benchmark Numbers").  Checked here:
  * the quantiser: codes and scales bit-exact against the oracle's quantiser, on crafted rows (every E4M3 tie,
    zero rows, saturation) and on seeded expert weights at the full widths;
  * one full-size MoE layer (d 2816, 128 experts top-8 + shared, 2048-key prefix) with FP8 experts;
  * a four-layer FP8 model at the full widths: one canvas pass teacher-forced layer by layer, and the head, with
    the tied embedding / vocab head in bf16 and in FP8 (one scale per vocabulary row);
  * the FP8 head over ragged vocabularies, every slot;
  * a small FP8 model through the block calls: a prompt prefilled with 64-row expert tiles, then blocks whose
    commits ride in the next block's first pass, for one sequence and for three sequences per call.
Bars as for bf16: 2e-2 abs/rel on hidden states and keys/values, routing by compare_routing, argmax where the
oracle's top-2 margin exceeds 1e-2.
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

BF16_TOL = (2e-2, 2e-2)
MARGIN = 1e-2


def log(msg):
    print(msg, flush=True)


def _untile(codes: np.ndarray, batch: int, rows: int, cols: int) -> np.ndarray:
    """FP8 pair-tiled bytes -> row-major [batch, rows, cols] codes (the layout dg_quantize_e4m3 documents)."""
    rp = (rows + 15) // 16 * 16
    a = codes.reshape(batch, rp // 16, cols // 64, 4, 16, 2, 8)      # b, rt, pair, q, r%16, half, j
    a = a.transpose(0, 1, 4, 2, 5, 3, 6).reshape(batch, rp, cols)   # c = 64 pair + 32 half + 8 q + j
    assert np.all(a[:, rows:] == 0), "padded rows are not zero"
    return a[:, :rows]


def _bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _quantize_on_gpu(w_bits: np.ndarray):
    b, r, c = w_bits.shape
    codes, scale = dg.quantize_tensor_e4m3(_bf16_dev(w_bits))
    torch.cuda.synchronize()
    return _untile(codes.cpu().numpy(), b, r, c), scale.cpu().numpy().reshape(b, r)


def _bf16_bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_quantize_crafted_rows_bit_exact():
    """Rows whose largest magnitude is 448 * 2^-k (so the scale is 2^-k exactly and every quotient is exact): the
    other entries sit on every midpoint between neighbouring E4M3 values (ties to the even mantissa), a hair
    either side of them, on the codes themselves and beyond the largest value; plus an all-zero row and a row
    with one nonzero entry.  Codes and scales equal the oracle's bit for bit; padded rows are zero."""
    pos = numerics.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    vals = np.concatenate([mids, -mids, pos, -pos, mids * (1 + 2 ** -7), mids * (1 - 2 ** -7)])
    vals = numerics.bf16_round(vals)                       # exactly representable rows (bf16 storage)
    cols = 128
    rows = []
    for k, chunk in enumerate(np.array_split(vals, len(vals) // (cols - 1) + 1)):
        s = 2.0 ** -(k % 5)
        row = np.zeros(cols)
        row[0] = 448.0 * s
        row[1:1 + len(chunk)] = np.clip(chunk, -448, 448) * s
        rows.append(row)
    rows.append(np.zeros(cols))
    one = np.zeros(cols)
    one[77] = -3.0e-3
    rows.append(one)
    w = np.stack(rows)[None].astype(np.float32)
    bits = _bf16_bits(w)
    codes, scale = _quantize_on_gpu(bits)
    ref_codes, ref_scale = numerics.quantize_e4m3_rows(numerics.from_storage(bits, "bf16").astype(np.float32))
    assert np.array_equal(scale, ref_scale)
    bad = np.nonzero(codes != ref_codes)
    assert bad[0].size == 0, f"{bad[0].size} codes differ, first at {[(int(i), int(j), int(k)) for i, j, k in zip(*bad)][:5]}"


def test_quantize_seeded_expert_weights_bit_exact():
    """The first four experts of a full-width layer's gate/up weights ([4, 1408, 2816], the seeded N(0, 0.02)
    draw): codes and scales equal the oracle's bit for bit."""
    d = recipe.C3.dims
    shape = (4, 2 * d.ffn_expert, d.d_model)
    bits = dg_inputs.normal(shape, recipe.WEIGHT_SEED, recipe.layer_stream(0, "w_gate_up"), recipe.WEIGHT_SIGMA,
                            "bf16")
    codes, scale = _quantize_on_gpu(bits)
    ref_codes, ref_scale = numerics.quantize_e4m3_rows(numerics.from_storage(bits, "bf16").astype(np.float32))
    assert np.array_equal(scale, ref_scale)
    assert np.array_equal(codes, ref_codes)


def test_fp8_layer_full_size():
    """One full-size MoE layer with FP8 experts: 256 canvas rows over a 2048-key prefix (bidirectional), hidden
    states where the routing agrees and the canvas keys/values against the oracle's FP8 layer."""
    d = replace(recipe.C1.dims, expert_dtype="e4m3")
    S, P = d.canvas, recipe.C1.prefix
    log("fp8 layer: device weights")
    w = {"embed": torch.zeros((8, d.d_model), dtype=torch.bfloat16, device="cuda"),
         "final_norm": torch.ones(d.d_model, dtype=torch.bfloat16, device="cuda"),
         "layers": [gdev.layer_weights_device(d, 0)]}
    sess = Session(d, capacity=P + S, weights=w)
    k = dg_inputs.normal((d.n_kv_heads, P, d.head_dim), recipe.INPUT_SEED, recipe.STREAM_PREFIX_K, 1.0, "bf16")
    v = dg_inputs.normal((d.n_kv_heads, P, d.head_dim), recipe.INPUT_SEED, recipe.STREAM_PREFIX_V, 1.0, "bf16")
    sess.k[0, :, :P, :] = _bf16_dev(k)
    sess.v[0, :, :, :P] = _bf16_dev(v.transpose(0, 2, 1))
    sess.kv.len = P
    x_host = dg_inputs.hidden((S, d.d_model), "bf16")
    x_dev = _bf16_dev(x_host)
    y_dev = torch.empty_like(x_dev)
    dbg = {"route_idx": torch.empty((S, d.top_k), dtype=torch.int32, device="cuda"),
           "route_w": torch.empty((S, d.top_k), dtype=torch.float32, device="cuda"),
           "router_logits": torch.empty((S, d.n_experts), dtype=torch.float32, device="cuda")}
    dg.dg_layer_forward(sess.cfg, sess.weights, 0, sess.kv, x_dev, y_dev, S, 0, dbg, sess.ws, sess.ws_bytes,
                        side=sess.side)
    torch.cuda.synchronize()
    log("fp8 layer: oracle")
    lw = om.fp8_expert_layer({n: numerics.from_storage(a, "bf16") for n, a in dg_inputs.layer_weights_host(d, 0).items()})
    model = om.Model(oracle_dims(d), {"embed": None, "final_norm": None, "layers": [lw]})
    kv = om.KVCache(1, d.n_kv_heads, d.head_dim)
    kv.k[0], kv.v[0] = numerics.from_storage(k, "bf16"), numerics.from_storage(v, "bf16")
    y_ref, tr = model.layer(0, numerics.from_storage(x_host, "bf16"), kv, False, append=True)
    same = compare_routing(dbg["route_idx"].cpu().numpy(), dbg["route_w"].cpu().numpy(),
                           dbg["router_logits"].cpu().numpy(), tr.router_logits, tr.idx, BF16_TOL)
    ok, worst, at = allclose_report(to_f64(y_dev)[same], y_ref[same], *BF16_TOL)
    log(f"fp8 layer: {int((~same).sum())} routing flips at ties; worst excess {worst:+.2e}")
    assert ok, ("hidden", worst, at)
    assert int((~same).sum()) <= S // 20
    gk, gv = sess.kv_numpy(0, P + S)
    assert allclose_report(gk[:, P:], kv.k[0][:, P:], *BF16_TOL)[0]
    assert allclose_report(gv[:, P:], kv.v[0][:, P:], *BF16_TOL)[0]
    # the FP8 layer is a different computation from the bf16 one: its outputs move by more than the bf16 bar
    lw16 = {n: numerics.from_storage(a, "bf16") for n, a in dg_inputs.layer_weights_host(d, 0).items()}
    kv16 = om.KVCache(1, d.n_kv_heads, d.head_dim)
    kv16.k[0], kv16.v[0] = kv.k[0][:, :P], kv.v[0][:, :P]
    y16, _ = om.Model(oracle_dims(replace(d, expert_dtype="")), {"embed": None, "final_norm": None,
                                                                  "layers": [lw16]}).layer(
        0, numerics.from_storage(x_host, "bf16"), kv16, False, append=False)
    assert np.max(np.abs(y16 - y_ref)) > 1e-2


@pytest.mark.parametrize("head_dtype", ["", "e4m3"], ids=["bf16_head", "fp8_head"])
def test_fp8_four_layers_teacher_forced_and_head(head_dtype):
    """A four-layer FP8 model at the full widths over a 512-token prompt: one canvas pass, each layer compared on
    the GPU's input rows and cache (the prompt's layer-0 keys/values checked free-running), and the head on every
    slot of the 262,144-token vocabulary.  With the FP8 head the tied embedding is E4M3 too: the prompt's and the
    canvas's embedding rows (compared through layer 0, whose input the oracle builds from its own dequantised
    rows) and the head's row-scaled logits."""
    from tests._gpu import check_prompt_cache
    d = replace(recipe.C3.dims, n_layers=4, expert_dtype="e4m3", head_dtype=head_dtype)
    P, S = 512, d.canvas
    log("fp8 4 layers: device weights")
    sess = Session(d, capacity=P + S, max_tokens=S)
    prompt = dg_inputs.prompt_tokens(P, d.vocab)
    sess.prefill(prompt)
    canvas = osm.initial_canvas(recipe.INPUT_SEED, 0, S, d.vocab)
    L = d.n_layers
    dbg = {"hidden": torch.empty((L, S, d.d_model), dtype=torch.bfloat16, device="cuda"),
           "route_idx": torch.empty((L, S, d.top_k), dtype=torch.int32, device="cuda"),
           "route_w": torch.empty((L, S, d.top_k), dtype=torch.float32, device="cuda"),
           "router_logits": torch.empty((L, S, d.n_experts), dtype=torch.float32, device="cuda")}
    pred, conf, ent = sess.denoise(canvas, dbg=dbg)
    torch.cuda.synchronize()
    log("fp8 4 layers: oracle")
    model = oracle_model(d, log=log)
    left = check_prompt_cache(sess, model, prompt, BF16_TOL)
    log(f"fp8 4 layers: prompt cache checked ({left} rows near a routing tie left out)")
    hid = [to_f64(dbg["hidden"][l]) for l in range(L)]
    x = model.embed(canvas)
    for l in range(L):
        if l:
            x = hid[l - 1]
        kv = om.KVCache(L, d.n_kv_heads, d.head_dim)
        kv.k[l], kv.v[l] = sess.kv_numpy(l, P)
        xo, tr = model.layer(l, x, kv, causal=False, append=False)
        same = compare_routing(dbg["route_idx"][l].cpu().numpy(), dbg["route_w"][l].cpu().numpy(),
                               dbg["router_logits"][l].cpu().numpy(), tr.router_logits, tr.idx, BF16_TOL)
        ok, worst, at = allclose_report(hid[l][same], xo[same], *BF16_TOL)
        log(f"fp8 layer {l}: routing flips {int((~same).sum())}; worst excess {worst:+.2e}")
        assert ok, (l, worst, at)
        assert int((~same).sum()) <= 4
    opred, oconf, oent, margin = om.head_stats(hid[L - 1], model.w["final_norm"], model.w["embed"], 1.0, d.rms_eps,
                                               numerics.bf16_round)
    sel = margin > MARGIN
    assert np.array_equal(pred.cpu().numpy()[sel], opred[sel])
    assert allclose_report(to_f64(ent), oent, *BF16_TOL)[0]
    assert allclose_report(to_f64(conf), oconf, *BF16_TOL)[0]
    log(f"fp8 4 layers: head {int(sel.sum())}/{S} argmax compared")


@pytest.mark.parametrize("vocab", [5000, 4112])
def test_fp8_head_ragged_vocabulary_all_slots(vocab):
    """The FP8 head over a vocabulary that ends inside a 256-token tile (and, at 5000 rows, inside a 16-row
    fragment, whose padding rows the quantiser fills with zeros): every slot against the oracle's row-scaled E4M3
    head (argmax where the top-2 margin exceeds 1e-2, confidence and entropy at the bf16 bar)."""
    from tests._helpers import fp8_embedding
    d = replace(recipe.C2.dims, vocab=vocab, head_dtype="e4m3")
    w = {"embed": gdev.normal_tensor((d.vocab, d.d_model), recipe.WEIGHT_SEED, recipe.STREAM_EMBED,
                                     recipe.WEIGHT_SIGMA, "bf16"),
         "final_norm": torch.ones(d.d_model, dtype=torch.bfloat16, device="cuda"), "layers": []}
    sess = Session(replace(d, n_layers=0), capacity=32, weights=w)
    x_host = dg_inputs.hidden((d.canvas, d.d_model), "bf16")
    x_dev = torch.from_numpy(x_host.view(np.int16)).cuda().view(torch.bfloat16)
    n = d.canvas
    pred, conf, ent = sess.i32(n), sess.f32(n), sess.f32(n)
    dg.dg_vocab_head(sess.cfg, sess.weights, x_dev, n, 1.0, pred, conf, ent, sess.ws, sess.ws_bytes)
    torch.cuda.synchronize()
    E = fp8_embedding(numerics.from_storage(dg_inputs.embed_host(d), "bf16"))
    opred, oconf, oent, margin = om.head_stats(numerics.from_storage(x_host, "bf16"), np.ones(d.d_model), E, 1.0,
                                               d.rms_eps, numerics.bf16_round)
    sel = margin > MARGIN
    log(f"fp8 head V={vocab}: {int(sel.sum())}/{n} argmax compared")
    assert sel.sum() >= n // 2
    assert np.array_equal(pred.cpu().numpy()[sel], opred[sel])
    assert allclose_report(to_f64(conf), oconf, 1e-6, BF16_TOL[1])[0]
    assert allclose_report(to_f64(ent), oent, *BF16_TOL)[0]


def test_fp8_small_widths_overlapped_blocks_against_oracle():
    """FP8 experts and FP8 tied embedding / head at small widths (the tiny model's shapes in bf16: d 256, 8 experts
    top-2 + shared, vocabulary 4096, canvas 32) through the block calls: a 256-token prompt prefilled in one call
    (512 routed pairs, so 64-row expert tiles), then three blocks of one pass each through
    dg_generate_block_overlapped, each block's commit carried by the next block's first pass (64 rows) and the last
    one committed at its end.  Against the FP8 oracle at the bf16 bar: the prompt's layer-0 cache rows
    free-running, every block's tokens (where the oracle's top-2 margin allows) and mean entropy on the GPU's
    context, and each committed block's cache rows."""
    from tests._gpu import check_commit_on_gpu_cache, check_pass_on_gpu_cache, check_prompt_cache, gpu_cache_as_oracle
    d = replace(recipe.C0.dims, dtype="bf16", expert_dtype="e4m3", head_dtype="e4m3")
    P, S = 256, d.canvas
    sess = Session(d, capacity=P + 4 * S, max_tokens=max(P, 2 * S))
    prompt = dg_inputs.prompt_tokens(P, d.vocab)
    sess.prefill(prompt)
    model = oracle_model(d)
    log(f"fp8 small: prompt cache checked ({check_prompt_cache(sess, model, prompt, BF16_TOL)} rows near a "
        f"routing tie left out)")
    sp = dg.make_sampler(recipe.C0.n_new, fixed_steps=1)
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
        log(f"fp8 small block {b}: {n}/{S} tokens compared, mean entropy {st.mean_entropy:.4f}")
        assert n >= S // 4  # slots near a top-2 or routing tie of this small model are left out
        pending = outs[b]
    assert sess.kv.len == P + 3 * S
    check_commit_on_gpu_cache(model, gpu_cache_as_oracle(sess, P + 2 * S), outs[2].cpu().numpy(), sess, BF16_TOL)


def test_fp8_small_widths_batched_blocks_against_oracle():
    """The small FP8 model (FP8 experts and tied embedding / head) with three sequences per call through
    dg_generate_blocks_overlapped: two calls of one pass each, the second call's pass also carrying the first
    call's three blocks.  Every sequence against the FP8 oracle on its own GPU context: tokens where the oracle's
    top-2 margin allows, mean entropy, and each committed block's cache rows at the bf16 bar."""
    from tests._gpu import check_commit_on_gpu_cache, check_pass_on_gpu_cache, gpu_cache_as_oracle
    d = replace(recipe.C0.dims, dtype="bf16", expert_dtype="e4m3", head_dtype="e4m3")
    S = d.canvas
    prefixes, calls = [64, 100, 0], [[2, 7, 1], [8, 2, 8]]
    sessions = []
    for b, p in enumerate(prefixes):  # one cache per sequence over the first session's device weights
        s = Session(d, capacity=p + 3 * S, weights=sessions[0].w if sessions else None, packed=bool(sessions))
        if p:
            s.prefill(dg_inputs.prompt_tokens(p, d.vocab, seed=b + 1))
        sessions.append(s)
    model = oracle_model(d)
    n = len(sessions)
    ws_bytes = dg.dg_workspace_size(sessions[0].cfg, 2 * n * S)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    sp = dg.make_sampler(recipe.C0.n_new, fixed_steps=1)
    outs = [torch.empty((n, S), dtype=torch.int32, device="cuda") for _ in calls]
    for c, blocks in enumerate(calls):
        st = dg.dg_generate_blocks_overlapped(sessions[0].cfg, sessions[0].weights, [s.kv for s in sessions], sp,
                                              blocks, outs[c - 1] if c else None, 1 if c + 1 < len(calls) else 0,
                                              outs[c], ws, ws_bytes, side=sessions[0].side)
        torch.cuda.synchronize()
        assert all((x.steps, x.reason) == (1, dg.DG_STOP_FIXED) for x in st)
        for b, (s, p) in enumerate(zip(sessions, prefixes)):
            if c > 0:  # the previous call's block, committed inside this call's pass
                check_commit_on_gpu_cache(model, gpu_cache_as_oracle(s, p + (c - 1) * S), outs[c - 1][b].cpu().numpy(),
                                          s, BF16_TOL)
            m = check_pass_on_gpu_cache(model, gpu_cache_as_oracle(s, p + c * S),
                                        osm.initial_canvas(sp.seed, blocks[b], S, d.vocab), outs[c][b].cpu().numpy(),
                                        st[b].mean_entropy, BF16_TOL)
            log(f"fp8 small batch call {c} seq {b}: {m}/{S} tokens compared")
            assert m >= S // 4  # slots near a top-2 or routing tie of this small model are left out
    for b, (s, p) in enumerate(zip(sessions, prefixes)):
        assert s.kv.len == p + len(calls) * S
        check_commit_on_gpu_cache(model, gpu_cache_as_oracle(s, p + (len(calls) - 1) * S), outs[-1][b].cpu().numpy(),
                                  s, BF16_TOL)
