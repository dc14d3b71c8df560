"""GPU parity of batched blocks (dg_generate_blocks: several independent sequences' canvases in one pass)
against the oracle run sequence by sequence.

Bars as elsewhere: tokens, passes and stop reasons bit-exact in fp32; caches within 1e-4 (fp32) or 2e-2
(bf16) of the oracle; bf16 tokens equal to the oracle's on the GPU's context wherever the oracle's top-2
margin exceeds 1e-2.
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
ALL = dg.DG_SAMPLE_GUMBEL | dg.DG_SAMPLE_ANNEAL | dg.DG_KEEP_ENTROPY | dg.DG_KEEP_LOCK | dg.DG_STOP_AND


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _sessions(d, prefixes, weights=None, packed=False):
    """One session (cache) per sequence over shared device weights (the first session's packed copy); sequence
    b's prompt is drawn with seed b + 1."""
    out = []
    for b, p in enumerate(prefixes):
        if out:
            s = Session(d, capacity=p + 3 * d.canvas, weights=out[0].w, packed=True)
        else:
            s = Session(d, capacity=p + 3 * d.canvas, weights=weights, packed=packed)
        if p:
            s.prefill(dg_inputs.prompt_tokens(p, d.vocab, seed=b + 1))
        out.append(s)
    return out


def _batch(sessions, sp, blocks):
    d = sessions[0].d
    n = len(sessions)
    ws_bytes = dg.dg_workspace_size(sessions[0].cfg, n * d.canvas)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((n, d.canvas), dtype=torch.int32, device="cuda")
    st = dg.dg_generate_blocks(sessions[0].cfg, sessions[0].weights, [s.kv for s in sessions], sp, blocks, out, ws,
                               ws_bytes)
    torch.cuda.synchronize()
    return out.cpu().numpy(), st


@pytest.mark.parametrize("flags,kw", [(0, dict()), (ALL, dict(entropy_threshold=0.1))], ids=["plain", "recommended"])
def test_c0_batch_equals_oracle_per_sequence(flags, kw):
    """Three sequences with different prompts and lengths (64, 40 and 0 tokens) and block ids: each one's
    tokens, passes, stop reason and committed cache equal the oracle's single-sequence block."""
    d = recipe.C0.dims
    storage = dg_inputs.model_weights_host(d)
    prefixes, blocks = [64, 40, 0], [0, 5, 2]
    sessions = _sessions(d, prefixes, weights=gdev.from_host(storage, d.dtype))
    anneal = (float(np.float32(0.8)), float(np.float32(0.4))) if flags & dg.DG_SAMPLE_ANNEAL else None
    sp = dg.make_sampler(recipe.C0.n_new, flags=flags, temperature_first=0.8, temperature_last=0.4, **kw)
    ref = osm.Sampler(n_new=recipe.C0.n_new, gumbel=bool(flags & dg.DG_SAMPLE_GUMBEL), anneal=anneal,
                      rank_entropy=bool(flags & dg.DG_KEEP_ENTROPY), lock=bool(flags & dg.DG_KEEP_LOCK),
                      stop_and=bool(flags & dg.DG_STOP_AND), **kw)
    toks, st = _batch(sessions, sp, blocks)
    if flags == 0:  # the sequences stop at different passes (9, 9 and 15): finished canvases ride along
        assert len({x.steps for x in st}) > 1
    model = oracle_model(d, storage)
    for b, (p, blk) in enumerate(zip(prefixes, blocks)):
        kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
        if p:
            osm.prefill(model, kv, dg_inputs.prompt_tokens(p, d.vocab, seed=b + 1))
        res = osm.generate_block(model, kv, ref, block=blk)
        log(f"seq {b}: GPU {st[b].steps} passes reason {st[b].reason}; oracle {res.steps} reason {res.reason}")
        assert (st[b].steps, st[b].reason) == (res.steps, res.reason), b
        assert np.array_equal(toks[b], res.tokens), b
        s = sessions[b]
        assert s.kv.len == kv.length == p + d.canvas
        for l in range(d.n_layers):
            gk, gv = s.kv_numpy(l, kv.length)
            assert allclose_report(gk, kv.k[l], *F32_TOL)[0] and allclose_report(gv, kv.v[l], *F32_TOL)[0], (b, l)


@pytest.mark.parametrize("overlapped", [False, True], ids=["commit_at_end", "commit_in_next_pass"])
def test_c3_two_layers_batch_against_oracle(overlapped):
    """bf16 at the benchmark's widths (d 2816, 128 experts top-8, 262144 vocabulary, canvas 256) with two layers
    and four sequences per call: 1024 canvas rows per pass (the 64-row expert tiles).  Each call runs one pass;
    with overlapped=True the second call's first pass also carries the first call's four blocks (2048 rows).
    Every sequence is checked against the oracle on the GPU's context (teacher-forced): its tokens where the
    oracle's top-2 margin exceeds 1e-2, its mean entropy, and each committed block's cache rows, every layer,
    at the bf16 bar; the prompt caches are checked free-running."""
    from tests._gpu import check_commit_on_gpu_cache, check_pass_on_gpu_cache, check_prompt_cache, gpu_cache_as_oracle
    d = replace(recipe.C3.dims, n_layers=2)
    S = d.canvas
    prefixes, calls = [512, 300, 64, 700], ([[3, 1, 4, 1], [5, 9, 2, 6]] if overlapped else [[3, 1, 4, 1]])
    log("c3_two_layers: building weights and prompts")
    sessions = _sessions(d, prefixes)
    model = oracle_model(d)
    for b, (s, p) in enumerate(zip(sessions, prefixes)):  # prompt caches, free-running
        out = check_prompt_cache(s, model, dg_inputs.prompt_tokens(p, d.vocab, seed=b + 1), BF16_TOL)
        log(f"seq {b} prompt cache: {out} rows near a routing tie left out")
    n = len(sessions)
    ws_bytes = dg.dg_workspace_size(sessions[0].cfg, (2 if overlapped else 1) * n * S)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    sp = dg.make_sampler(26, fixed_steps=1)
    outs = [torch.empty((n, S), dtype=torch.int32, device="cuda") for _ in calls]
    side = sessions[0].side
    for c, blocks in enumerate(calls):
        if overlapped:
            st = dg.dg_generate_blocks_overlapped(sessions[0].cfg, sessions[0].weights, [s.kv for s in sessions], sp,
                                                  blocks, outs[c - 1] if c else None, 1 if c + 1 < len(calls) else 0,
                                                  outs[c], ws, ws_bytes, side=side)
        else:
            st = dg.dg_generate_blocks(sessions[0].cfg, sessions[0].weights, [s.kv for s in sessions], sp, blocks,
                                       outs[c], ws, ws_bytes, side=side)
        torch.cuda.synchronize()
        assert all((x.steps, x.reason) == (1, dg.DG_STOP_FIXED) for x in st)
        for b, (s, p) in enumerate(zip(sessions, prefixes)):
            if overlapped and c > 0:  # the previous call's block, committed inside this call's first pass
                check_commit_on_gpu_cache(model, gpu_cache_as_oracle(s, p + (c - 1) * S), outs[c - 1][b].cpu().numpy(),
                                          s, BF16_TOL)
            m = check_pass_on_gpu_cache(model, gpu_cache_as_oracle(s, p + c * S),
                                        osm.initial_canvas(sp.seed, blocks[b], S, d.vocab), outs[c][b].cpu().numpy(),
                                        st[b].mean_entropy, BF16_TOL)
            log(f"call {c} seq {b}: {m}/{S} tokens compared, mean entropy {st[b].mean_entropy:.4f}")
    for b, (s, p) in enumerate(zip(sessions, prefixes)):  # each call's own commit at its end
        assert s.kv.len == p + len(calls) * S
        check_commit_on_gpu_cache(model, gpu_cache_as_oracle(s, p + (len(calls) - 1) * S), outs[-1][b].cpu().numpy(),
                                  s, BF16_TOL)


@pytest.mark.parametrize("canvas,prefixes", [(71, [33, 0, 70]), (32, [5, 64, 1, 17, 40, 2, 0, 9])],
                         ids=["ragged_canvas", "eight_sequences"])
def test_c0_batch_edges_equal_oracle(canvas, prefixes):
    """A ragged canvas (71 slots: segment boundaries off the 16-row fragments) and the most sequences per call
    (8): each sequence equals the oracle's single-sequence block at a fixed T."""
    d = replace(recipe.C0.dims, canvas=canvas)
    storage = dg_inputs.model_weights_host(d)
    sessions = _sessions(d, prefixes, weights=gdev.from_host(storage, d.dtype))
    blocks = list(range(7, 7 + len(prefixes)))
    sp = dg.make_sampler(-(-canvas // 4), fixed_steps=4)
    toks, st = _batch(sessions, sp, blocks)
    model = oracle_model(d, storage)
    for b, (p, blk) in enumerate(zip(prefixes, blocks)):
        kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
        if p:
            osm.prefill(model, kv, dg_inputs.prompt_tokens(p, d.vocab, seed=b + 1))
        res = osm.generate_block(model, kv, osm.Sampler(n_new=-(-canvas // 4), fixed_steps=4), block=blk)
        assert (st[b].steps, st[b].reason) == (res.steps, res.reason), b
        assert np.array_equal(toks[b], res.tokens), b
        for l in range(d.n_layers):
            gk, gv = sessions[b].kv_numpy(l, kv.length)
            assert allclose_report(gk, kv.k[l], *F32_TOL)[0] and allclose_report(gv, kv.v[l], *F32_TOL)[0], (b, l)


def test_c0_batch_overlapped_commits_equal_oracle():
    """Three consecutive batched calls of three sequences, each call's blocks committed inside the next call's
    first pass (the last call commits its own): every block and the final caches equal the oracle's blocks
    generated and committed one after another."""
    d = recipe.C0.dims
    storage = dg_inputs.model_weights_host(d)
    prefixes = [64, 40, 0]
    sessions = []
    w = gdev.from_host(storage, d.dtype)
    for b, p in enumerate(prefixes):
        s = Session(d, capacity=p + 5 * d.canvas, weights=w if not sessions else sessions[0].w,
                    packed=bool(sessions))
        if p:
            s.prefill(dg_inputs.prompt_tokens(p, d.vocab, seed=b + 1))
        sessions.append(s)
    n = len(sessions)
    ws_bytes = dg.dg_workspace_size(sessions[0].cfg, 2 * n * d.canvas)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    sp = dg.make_sampler(recipe.C0.n_new)
    outs = [torch.empty((n, d.canvas), dtype=torch.int32, device="cuda") for _ in range(3)]
    gpu = []
    for c in range(3):
        st = dg.dg_generate_blocks_overlapped(sessions[0].cfg, sessions[0].weights, [s.kv for s in sessions], sp,
                                              [10 * c + b for b in range(n)], outs[c - 1] if c else None,
                                              1 if c < 2 else 0, outs[c], ws, ws_bytes)
        torch.cuda.synchronize()
        gpu.append((outs[c].cpu().numpy(), [(x.steps, x.reason) for x in st]))
    model = oracle_model(d, storage)
    for b, p in enumerate(prefixes):
        kv = om.KVCache(d.n_layers, d.n_kv_heads, d.head_dim)
        if p:
            osm.prefill(model, kv, dg_inputs.prompt_tokens(p, d.vocab, seed=b + 1))
        for c in range(3):
            res = osm.generate_block(model, kv, osm.Sampler(n_new=recipe.C0.n_new), block=10 * c + b)
            assert gpu[c][1][b] == (res.steps, res.reason), (b, c)
            assert np.array_equal(gpu[c][0][b], res.tokens), (b, c)
        s = sessions[b]
        assert s.kv.len == kv.length == p + 3 * d.canvas
        for l in range(d.n_layers):
            gk, gv = s.kv_numpy(l, kv.length)
            assert allclose_report(gk, kv.k[l], *F32_TOL)[0] and allclose_report(gv, kv.v[l], *F32_TOL)[0], (b, l)
