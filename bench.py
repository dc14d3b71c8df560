#!/usr/bin/env python3
"""Benchmark of the block-diffusion denoising step on one MI355X.

Workload (N=1, default full_loop_bf16): the 30-layer bf16 MoE model (d 2816,
16 q / 8 KV heads of dim 128, 128 experts top-8 + 1 shared, 262144-token tied
vocabulary) with a 4096-token uniform-random prompt prefilled into the KV
cache, random-init weights from the seeded generator.  One timed step is one
whole 256-slot block at a fixed T=10: the initial random canvas, 10 denoising
passes, 10 stop checks, 9 keep/re-randomise updates, and one block commit into
the KV cache.  Blocks run through dg_generate_block_overlapped: each block's
commit (a causal forward of its 256 tokens) rides in the next block's first
pass, so that forward streams the weights once for both; every step therefore
carries one commit, of the block before it (the cache length is reset to the
prompt before each step, so every step does identical work).  With --workload
long_context_bf16 the prompt is 131072 tokens and one step is 4 consecutive
blocks.  Reported value: canvas tokens per second = 256 * blocks / (step
time); also ms per denoising pass.  --sampler recommended runs the same
workload under the recommended sampler's variants (Gumbel-max draws at a
temperature annealed from 0.8 to 0.4, entropy-ranked locking keep, AND stop
rule; still a fixed T).

Extra objects on the JSON line:
  roofline     — the dominant kernel (routed-expert gate/up projection, HBM
                 bound; attention, matrix-core bound, on the long-context
                 workload): algorithmic bytes or FLOPs per launch / its average
                 duration from HIP events recorded on the launch stream during
                 the timed run of plain passes (every launch there has the
                 canvas shape); traffic from the committed rocprofv3 counter
                 summary when it matches the current kernel source, else null
  cpu_baseline — the CPU oracle timed on a bounded sample (one layer of the
                 pass plus the head on a few slots), extrapolated to a step
  kernels      — per-kernel-class time of one instrumented denoising pass
  mfma, hbm    — achieved bf16 matrix-core TFLOP/s of attention, the expert
                 GEMMs, the dense projections and the vocab GEMM, and HBM GB/s
                 of the expert-weight stream, from that pass, as fractions of
                 MI355X peak (algorithmic FLOPs / bytes)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "canvas tokens/sec at batch 1 (256-slot block, T=10) + ms/denoising step"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILES = {"bf16": os.path.join(ROOT, "profiles", "moe_gate_up_traffic.json"),
                 "e4m3": os.path.join(ROOT, "profiles", "moe_gate_up_f8_traffic.json")}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("k_gemm.hip", "dg_device.h", "dg_wave_gemm.h", "dg_kernels.h"):
        with open(os.path.join(ROOT, "block_diffusion_decoding_step_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def expert_weight_bytes(d) -> float:
    """Bytes per routed-expert weight: 2 (bf16) or 1 (FP8 E4M3 codes; their float scales are counted apart)."""
    return 1.0 if d.expert_dtype == "e4m3" else 2.0


def gate_up_bytes(d, experts_hit: float, pairs: int, rows: int = None) -> float:
    """Algorithmic bytes of one routed gate/up launch: each hit expert's [2*fe, d] weights once (plus, for FP8
    weights, their 2*fe float scales), the normalised rows once, the SwiGLU products written once."""
    w = experts_hit * 2 * d.ffn_expert * (d.d_model * expert_weight_bytes(d) + (4 if d.expert_dtype == "e4m3" else 0))
    x = (d.canvas if rows is None else rows) * d.d_model * 2
    h = pairs * d.ffn_expert * 2
    return w + x + h


def attention_flops(d, keys: int, causal: bool) -> float:
    """Algorithmic FLOPs of one attention launch over the canvas: Q K^T and P V for every visible key."""
    if causal:  # query i (0-based) of the block sees keys - S + i + 1 keys
        visible = d.canvas * (keys - d.canvas) + d.canvas * (d.canvas + 1) / 2
    else:
        visible = d.canvas * keys
    return 4.0 * d.n_heads * d.head_dim * visible


# the shared expert's GEMMs run on a side stream, concurrently with the routing and the routed experts:
# their event-timed spans include the time their workgroups wait for compute units the routed experts hold
SIDE_KERNELS = ("shared_gate_up", "shared_down")
SIDE_NOTE = "side stream, concurrent with the routing and routed experts: event span, not exclusive time"


def pass_flops(d, keys: int, pairs: int) -> dict:
    """Algorithmic FLOPs of one denoising pass by kernel class."""
    S, L = d.canvas, d.n_layers
    qkv = 2 * S * d.d_model * (d.n_heads + 2 * d.n_kv_heads) * d.head_dim
    o = 2 * S * d.n_heads * d.head_dim * d.d_model
    shared = 2 * S * d.d_model * 3 * d.ffn_shared
    router = 2 * S * d.d_model * d.n_experts
    return {"attention": L * attention_flops(d, keys, False),
            "experts": L * 2 * pairs * 3 * d.ffn_expert * d.d_model,
            "dense": L * (qkv + o),
            "shared_expert": L * shared,
            "router": L * router,
            "vocab_head": 2 * S * d.vocab * d.d_model}


def read_traffic(d, kernel: str):
    """Measured HBM bytes per canvas launch of the gate/up kernel from the committed counter summary of this
    expert precision, or None when there is none or the kernel sources changed since it was taken."""
    path = TRAFFIC_FILES["e4m3" if d.expert_dtype == "e4m3" else "bf16"]
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash() or t.get("kernel") != kernel:
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(wl, log_fn) -> dict:
    """Oracle on the host: one layer of a denoising pass over a 4096-key cache plus the head on 16 slots,
    extrapolated to a block (10 passes of 30 layers and 256 head slots, plus a 30-layer commit)."""
    import numpy as np

    import dg_inputs
    from dg_inputs import recipe
    from oracle import model as om
    from oracle import numerics
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    d = wl.dims
    log_fn("cpu baseline: generating one layer + embedding on the host")
    lw = {n: numerics.from_storage(a, "bf16") for n, a in dg_inputs.layer_weights_host(d, 0).items()}
    E = numerics.from_storage(dg_inputs.embed_host(d), "bf16")
    d1 = om.Dims(**{f: getattr(d, f) for f in om.Dims.__dataclass_fields__})
    d1.n_layers = 1
    model = om.Model(d1, {"embed": E, "final_norm": np.ones(d.d_model), "layers": [lw]})
    kv = om.KVCache(1, d.n_kv_heads, d.head_dim)
    kv.k[0] = numerics.from_storage(dg_inputs.normal((d.n_kv_heads, wl.prefix, d.head_dim), 1,
                                                     recipe.STREAM_PREFIX_K, 1.0, "bf16"), "bf16")
    kv.v[0] = numerics.from_storage(dg_inputs.normal((d.n_kv_heads, wl.prefix, d.head_dim), 1,
                                                     recipe.STREAM_PREFIX_V, 1.0, "bf16"), "bf16")
    x = numerics.from_storage(dg_inputs.hidden((d.canvas, d.d_model), "bf16"), "bf16")
    log_fn("cpu baseline: timing the oracle")

    def repeat(fn, budget_s):
        n, t0 = 0, time.perf_counter()
        while True:
            out = fn()
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                return el / n, n, out

    t_layer, n_layer, (xo, _) = repeat(lambda: model.layer(0, x, kv, causal=False, append=False), 8.0)
    head_rows = 32
    t_head, n_head, _ = repeat(lambda: model.head(xo[:head_rows]), 4.0)
    t_pass = d.n_layers * t_layer + (d.canvas / head_rows) * t_head
    t_block = wl.fixed_steps * t_pass + d.n_layers * t_layer
    single = None
    try:  # the same single-layer and head samples on one BLAS thread
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t1_layer, _, _ = repeat(lambda: model.layer(0, x, kv, causal=False, append=False), 2.0)
            t1_head, _, _ = repeat(lambda: model.head(xo[:head_rows]), 2.0)
        single = {"cores": 1, "ms_per_moe_layer_pass": round(t1_layer * 1e3, 1),
                  "ms_per_head_pass": round(t1_head * d.canvas / head_rows * 1e3, 1),
                  "note": (f"one bidirectional MoE layer of the full widths over a {wl.prefix}-key cache and the "
                           f"vocab head over {d.canvas} slots (extrapolated from {head_rows}), one BLAS thread")}
    except Exception:  # pragma: no cover - threadpoolctl missing
        single = None
    return {"value": d.canvas / t_block, "unit": "canvas tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"{n_layer} runs of one bidirectional layer over a {wl.prefix}-key cache "
                       f"({t_layer:.2f} s each) and {n_head} runs of the vocab head on {head_rows} slots "
                       f"({t_head:.2f} s each), float64 numpy; extrapolated to {wl.fixed_steps} passes x "
                       f"{d.n_layers} layers x {d.canvas} head slots + a {d.n_layers}-layer commit"),
            "ms_per_denoising_step": t_pass * 1e3,
            "ms_per_moe_layer_pass": round(t_layer * 1e3, 1),
            "ms_per_head_pass": round(t_head * d.canvas / head_rows * 1e3, 1),
            "single_thread": single}


def run_batch(args, wl) -> int:
    """--batch B: one step is B independent sequences' blocks in one call (each sequence has its own 4096-token
    prompt and cache; T passes over all B canvases and the commit of B blocks, carried by the next call's first
    pass when 2 B canvases fit the routing row limit, else a causal forward at the end).  value = B * 256 / step time.  The roofline kernel is the gate/up projection over the B * 256 rows,
    timed with HIP events over the timed steps (passes and commits have the same row count); at 8 * B * 256
    routed pairs every expert is hit (a given expert is missed with probability (1 - 8/128)^(8 B 256))."""
    import numpy as np
    import torch

    import block_diffusion_decoding_step_amd as dg
    from dg_inputs import device as gdev
    from dg_inputs import recipe

    d, T, B = wl.dims, wl.fixed_steps, args.batch
    if B * d.canvas > 2048 or B > 8:
        print(f"--batch {B}: at most 8 canvases and 2048 rows per pass", file=sys.stderr)
        return 2
    log(f"bench: {wl.name} batch {B}; generating weights on the device")
    side = dg.Side()  # the shared expert's stream and events, owned here
    w = gdev.packed_model_weights_device(d)
    weights = dg.Weights(w["embed"], w["final_norm"], w["layers"], w.get("embed_scale"))
    cfg = dg.make_config(d)
    cap = ((wl.prefix + (wl.blocks + 1) * d.canvas + 31) // 32) * 32
    ws_bytes = dg.dg_workspace_size(cfg, max(2 * B * d.canvas if 2 * B * d.canvas <= 2048 else B * d.canvas, 2048))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    kvs, keep = [], []
    t0 = time.perf_counter()
    for b in range(B):
        k, v = gdev.kv_tensors(d, cap)
        kv = dg.KV(k, v, cap, 0)
        prompt = gdev.uniform_tensor(wl.prefix, recipe.INPUT_SEED + b, recipe.STREAM_PROMPT, d.vocab)
        dg.dg_prefill_kv(cfg, weights, kv, prompt, wl.prefix, ws, ws_bytes, side=side)
        kvs.append(kv)
        keep.append((k, v))
    torch.cuda.synchronize()
    t_prefill = time.perf_counter() - t0
    P = [kv.len for kv in kvs]
    sampler = dg.make_sampler(wl.n_new, fixed_steps=T, seed=recipe.INPUT_SEED)
    toks = torch.empty((B, d.canvas), dtype=torch.int32, device="cuda")

    # with 2 B canvas rows within the routing limit, each block's commit rides in the next call's first pass
    overlap = 2 * B * d.canvas <= 2048
    toks2 = [toks, torch.empty_like(toks)]
    pending = [None]

    def step(i):
        out = []
        for j in range(wl.blocks):
            if j == 0:
                for kv, p in zip(kvs, P):
                    kv.len = p
            ids = [(i * wl.blocks + j) * B + b for b in range(B)]
            if overlap:
                q = (i * wl.blocks + j) % 2
                out += dg.dg_generate_blocks_overlapped(cfg, weights, kvs, sampler, ids, pending[0], 1, toks2[q], ws,
                                                        ws_bytes, side=side)
                pending[0] = toks2[q]
            else:
                out += dg.dg_generate_blocks(cfg, weights, kvs, sampler, ids, toks, ws, ws_bytes, side=side)
        return out

    for i in range(args.warmup):
        step(i)
    if overlap and pending[0] is None:  # no warmup: one untimed call leaves the pending blocks
        step(0)
    torch.cuda.synchronize()
    dg.dg_timing_start(["moe_gate_up"])
    t0 = time.perf_counter()
    statuses = [st for i in range(args.steps) for st in step(i)]
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t0
    tim = dg.dg_timing_stop()
    assert all(s.steps == T and s.reason == dg.DG_STOP_FIXED for s in statuses)
    block_ms = t_total / args.steps * 1e3
    value = B * d.canvas * wl.blocks * args.steps / t_total
    g_ms, g_n = tim["moe_gate_up"]
    g_avg = g_ms / g_n
    M = B * d.canvas
    # launches per call: T passes of M rows and the commit's M rows (as a pass of its own, or inside the first
    # pass of the next call, which then has 2 M rows): every launch averages (T + 1) M / T rows when overlapped
    g_work = gate_up_bytes(d, d.n_experts, M * d.top_k * ((T + 1) / T if overlap else 1), M)
    achieved = g_work / (g_avg * 1e-3) / 1e9
    out = {
        "metric": METRIC.replace("at batch 1", f"at batch {B}"),
        "value": round(value, 2),
        "unit": "canvas tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(block_ms, 4),
        "ms_per_denoising_step": None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if d.expert_dtype != "e4m3" else "bf16+e4m3",
        "data": "synthetic",
        "config": {"workload": wl.name + f"_batch{B}", "description": wl.description, "canvas": d.canvas,
                   "prefix": wl.prefix, "T": T, "batch": B, "blocks_per_step": wl.blocks,
                   "step": (f"{wl.blocks} x (B = {B} blocks in one call: {T} passes over all {M} canvas rows + "
                            f"stop checks + updates + the commit of B blocks, "
                            + ("inside the next call's first pass (dg_generate_blocks_overlapped))" if overlap else
                               "in one causal forward at the end (dg_generate_blocks))")),
                   "ms_per_denoising_step_note": "passes run inside dg_generate_blocks and are not timed alone",
                   "prefill_s": round(t_prefill, 3)},
        "roofline": {"kernel": "k_moe_gate_up", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "bytes_per_launch": g_work, "avg_launch_ms": round(g_avg, 5),
                     "launches": g_n, "rows_per_launch": M},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, log)
    print(json.dumps(out), flush=True)
    return 0


def run_speculative(args, wl) -> int:
    """--speculative N: self-speculative decoding (dg_generate_speculative) of N output tokens after the prompt:
    each round drafts a 256-slot block by diffusion (T passes, the commit deferred) and verifies it with one causal
    forward; value = output tokens per second.  With random-init weights the drafts are random tokens, so a verify
    confirms about one token (the known one carried in): the line measures the loop's cost per round and reports
    the accepted tokens per verify; it says nothing about trained weights."""
    import torch

    import block_diffusion_decoding_step_amd as dg
    from dg_inputs import device as gdev
    from dg_inputs import recipe

    d, T, N = wl.dims, wl.fixed_steps, args.speculative
    side = dg.Side()
    log(f"bench: {wl.name} speculative {N} tokens; generating weights on the device")
    w = gdev.packed_model_weights_device(d)
    weights = dg.Weights(w["embed"], w["final_norm"], w["layers"], w.get("embed_scale"))
    cfg = dg.make_config(d)
    cap = ((wl.prefix + 2 * (N + d.canvas) + 31) // 32) * 32
    k, v = gdev.kv_tensors(d, cap)
    kv = dg.KV(k, v, cap, 0)
    ws_bytes = dg.dg_workspace_size(cfg, 2048)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    prompt = gdev.uniform_tensor(wl.prefix, recipe.INPUT_SEED, recipe.STREAM_PROMPT, d.vocab)
    dg.dg_prefill_kv(cfg, weights, kv, prompt, wl.prefix, ws, ws_bytes, side=side)
    P = kv.len
    sampler = dg.make_sampler(wl.n_new, fixed_steps=T, seed=recipe.INPUT_SEED)
    out = torch.empty(N, dtype=torch.int32, device="cuda")
    first = int(prompt[-1].item())
    for _ in range(args.warmup):
        kv.len = P
        dg.dg_generate_speculative(cfg, weights, kv, sampler, 0, first, N, out, ws, ws_bytes, side=side)
    torch.cuda.synchronize()
    stats, t0 = [], time.perf_counter()
    for i in range(args.steps):
        kv.len = P
        stats.append(dg.dg_generate_speculative(cfg, weights, kv, sampler, 1000 * i, first, N, out, ws, ws_bytes,
                                                side=side))
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t0
    rounds = sum(st.rounds for st, _ in stats)
    accepted = sum(st.accepted for st, _ in stats)
    res = {"metric": "output tokens/sec, self-speculative decoding at batch 1 (diffusion drafts of 256 slots, "
                     "T=10, verified causally)",
           "value": round(N * args.steps / t_total, 3), "unit": "output tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(t_total / args.steps * 1e3, 3), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": wl.name + "_speculative", "prefix": wl.prefix, "canvas": d.canvas, "T": T,
                      "tokens_per_step": N, "step": f"dg_generate_speculative of {N} tokens after the prompt"},
           "accepted_per_verify": round(accepted / rounds, 4), "verifies_per_step": rounds / args.steps,
           "ms_per_round": round(t_total / rounds * 1e3, 3)}
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="full_loop_bf16", choices=["full_loop_bf16", "long_context_bf16",
                                                                     "full_loop_fp8"])
    ap.add_argument("--sampler", default="plain", choices=["plain", "recommended"],
                    help="plain: argmax and confidence-ranked keep; recommended: Gumbel-max draws at a temperature "
                         "annealed 0.8 -> 0.4, entropy-ranked locking keep, AND stop rule (fixed T either way)")
    ap.add_argument("--batch", type=int, default=1,
                    help="canvases per pass (independent sequences, dg_generate_blocks); 1 is the batch-1 workload")
    ap.add_argument("--speculative", type=int, default=0,
                    help="tokens of self-speculative decoding per step (dg_generate_speculative); 0: the block workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (reference for HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one MI355X only: the library runs the whole denoising step on a single GPU "
              f"with no collectives (asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import block_diffusion_decoding_step_amd as dg
    import dg_inputs
    from dg_inputs import device as gdev
    from dg_inputs import recipe

    wl = recipe.WORKLOADS[args.workload]
    d = wl.dims
    T = wl.fixed_steps
    torch.cuda.set_device(0)
    if args.batch > 1:
        return run_batch(args, wl)
    if args.speculative > 0:
        return run_speculative(args, wl)
    stream = torch.cuda.current_stream()
    log(f"bench: {wl.name} on {torch.cuda.get_device_name(0)}; generating weights on the device")
    side = dg.Side()  # the shared expert's stream and events, owned here
    w = gdev.packed_model_weights_device(d)
    weights = dg.Weights(w["embed"], w["final_norm"], w["layers"], w.get("embed_scale"))
    cfg = dg.make_config(d)
    cap = ((wl.prefix + (wl.blocks + 1) * d.canvas + 31) // 32) * 32  # + the canvas rows of an overlapped commit
    k, v = gdev.kv_tensors(d, cap)
    kv = dg.KV(k, v, cap, 0)
    chunk = 2048
    ws_bytes = dg.dg_workspace_size(cfg, max(2 * d.canvas, chunk))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    prompt = gdev.uniform_tensor(wl.prefix, recipe.INPUT_SEED, recipe.STREAM_PROMPT, d.vocab)
    log(f"bench: prefill {wl.prefix} tokens")
    t0 = time.perf_counter()
    dg.dg_prefill_kv(cfg, weights, kv, prompt, wl.prefix, ws, ws_bytes, side=side)
    torch.cuda.synchronize()
    t_prefill = time.perf_counter() - t0
    P = kv.len
    flags = 0
    if args.sampler == "recommended":
        flags = dg.DG_SAMPLE_GUMBEL | dg.DG_SAMPLE_ANNEAL | dg.DG_KEEP_ENTROPY | dg.DG_KEEP_LOCK | dg.DG_STOP_AND
    sampler = dg.make_sampler(wl.n_new, fixed_steps=T, seed=recipe.INPUT_SEED, entropy_threshold=0.005, flags=flags,
                              temperature_first=0.8, temperature_last=0.4)

    def one_pass(dbg=None, t=1):
        if flags == 0 or dbg is not None:
            dg.dg_denoise_step(cfg, weights, kv, canvas, 1.0, pred, conf, ent, dbg, ws, ws_bytes, side=side)
        else:
            dg.dg_denoise_step_sampler(cfg, weights, kv, sampler, 0, t, canvas, pred, conf, ent, ws, ws_bytes, side=side)
    toks = [torch.empty(d.canvas, dtype=torch.int32, device="cuda") for _ in range(2)]
    pending = [None]

    blocks = wl.blocks

    def step(i):
        """One timed step: `blocks` consecutive blocks.  Each block's commit runs inside the next block's first
        pass (dg_generate_block_overlapped), the last one's inside the next step's first block, so every step
        carries `blocks` commits; the cache length is reset to the prompt first, so every step does the same
        work (the pending block is committed at the prompt's end)."""
        kv.len = P
        out = []
        for b in range(blocks):
            j = i * blocks + b
            out.append(dg.dg_generate_block_overlapped(cfg, weights, kv, sampler, j, pending[0], 1, toks[j % 2], ws,
                                                       ws_bytes, side=side))
            pending[0] = toks[j % 2]
        return out

    log(f"bench: warmup {args.warmup} steps of {blocks} block(s)")
    for i in range(args.warmup):
        step(i)
    if pending[0] is None:  # no warmup: one untimed block leaves the pending commit the first timed step carries
        kv.len = P
        dg.dg_generate_block_overlapped(cfg, weights, kv, sampler, 0, None, 1, toks[1], ws, ws_bytes, side=side)
        pending[0] = toks[1]
    torch.cuda.synchronize()

    # timed region: K steps
    dom = "attention" if wl.prefix > 65536 else "moe_gate_up"
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    statuses = [st for i in range(args.steps) for st in step(i)]
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t0
    assert all(s.steps == T and s.reason == dg.DG_STOP_FIXED for s in statuses)
    block_ms = t_total / args.steps * 1e3
    value = d.canvas * blocks * args.steps / t_total

    # ms per denoising pass alone (the same kernels, no update/commit)
    canvas = torch.empty(d.canvas, dtype=torch.int32, device="cuda")
    dg.dg_canvas_update(cfg, None, None, 0, recipe.INPUT_SEED, 0, 0, canvas)
    pred = torch.empty(d.canvas, dtype=torch.int32, device="cuda")
    conf = torch.empty(d.canvas, dtype=torch.float32, device="cuda")
    ent = torch.empty(d.canvas, dtype=torch.float32, device="cuda")
    # (timed region of its own; HIP events around the dominant kernel's launches on the launch stream: every
    # launch here has the canvas shape the roofline's algorithmic bytes describe)
    kv.len = P
    n_pass = args.steps * T
    dg.dg_timing_start([dom])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_pass):
        one_pass(t=i % T + 1)
    torch.cuda.synchronize()
    pass_ms = (time.perf_counter() - t0) / n_pass * 1e3
    tim = dg.dg_timing_stop()

    # routing of one pass: experts hit per layer (for the algorithmic bytes)
    ridx = torch.empty((d.n_layers, d.canvas, d.top_k), dtype=torch.int32, device="cuda")
    one_pass({"route_idx": ridx})
    torch.cuda.synchronize()
    ri = ridx.cpu().numpy()
    experts_hit = float(np.mean([len(np.unique(ri[l])) for l in range(d.n_layers)]))
    counts = [np.bincount(ri[l].ravel(), minlength=d.n_experts) for l in range(d.n_layers)]
    expert_tiles = float(np.mean([np.sum((c + 31) // 32) for c in counts]))  # 32-row tiles (weight reads)
    max_pairs = int(max(c.max() for c in counts))

    if args.copy_calibration_mib > 0:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give the scale of the byte counters
        src = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # per-kernel breakdown from one extra instrumented denoising pass (outside the timed region)
    kv.len = P
    dg.dg_timing_start(list(dg.KERNELS))
    one_pass()
    torch.cuda.synchronize()
    breakdown = dg.dg_timing_stop()

    pairs = d.canvas * d.top_k
    fl = pass_flops(d, P + d.canvas, pairs)
    cls = {"attention": ("attention", "attn_merge"), "experts": ("moe_gate_up", "moe_down"),
           "dense": ("gemm_qkv", "gemm_o"), "router": ("route",),
           "shared_expert": SIDE_KERNELS, "vocab_head": ("vocab_head", "head_merge")}
    mfma = {}
    for name, ks in cls.items():
        ms = sum(breakdown.get(k, (0.0, 0))[0] for k in ks)
        tf = fl[name] / (ms * 1e-3) / 1e12 if ms > 0 else 0.0
        mfma[name] = {"tflops": round(tf, 1), "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "ms_per_pass": round(ms, 4),
                      "kernels": list(ks)}
        if ks == SIDE_KERNELS:
            mfma[name]["note"] = SIDE_NOTE
    ex_ms = sum(breakdown.get(k, (0.0, 0))[0] for k in ("moe_gate_up", "moe_down"))
    ex_bytes = d.n_layers * experts_hit * 3 * d.ffn_expert * d.d_model * expert_weight_bytes(d)
    if d.expert_dtype == "e4m3":  # the scales: 2*fe (gate/up) + d (down) floats per hit expert
        ex_bytes += d.n_layers * experts_hit * (2 * d.ffn_expert + d.d_model) * 4
    hbm = {"experts": {"gbs": round(ex_bytes / (ex_ms * 1e-3) / 1e9, 1),
                       "frac": round(ex_bytes / (ex_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "bytes_per_pass": ex_bytes, "kernels": ["moe_gate_up", "moe_down"]}}

    g_ms, g_n = tim[dom]
    g_avg = g_ms / g_n
    if dom == "moe_gate_up":
        g_work = gate_up_bytes(d, experts_hit, pairs)
        achieved = g_work / (g_avg * 1e-3) / 1e9
        kname = "k_moe_gate_up_f8" if d.expert_dtype == "e4m3" else "k_moe_gate_up"
        roof = {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic(d, kname),
                "bytes_per_launch": g_work}
    else:
        # the timed plain passes: canvas queries over the prompt and the canvas
        g_work = attention_flops(d, P + d.canvas, False)
        achieved = g_work / (g_avg * 1e-3) / 1e12
        roof = {"kernel": "k_attn", "bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                "flops_per_launch": g_work}
    roof.update({"avg_launch_ms": round(g_avg, 5), "launches": g_n, "experts_hit_per_layer": experts_hit,
                 "expert_tiles_per_layer": expert_tiles, "max_pairs_per_expert": max_pairs})
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "canvas tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(block_ms, 4),
        "ms_per_denoising_step": round(pass_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if d.expert_dtype != "e4m3" else "bf16+e4m3",
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description,
                   "canvas": d.canvas, "prefix": wl.prefix, "T": T, "batch": 1, "blocks_per_step": blocks,
                   "sampler": args.sampler,
                   "step": (f"{blocks} block(s), each: {T} passes + stop checks + {T - 1} keep/re-randomise updates "
                            f"+ one commit (of the previous block, inside the first pass)"),
                   "canvas_tokens_per_s_without_commit": round(d.canvas / (T * pass_ms * 1e-3), 2),
                   "prefill_s": round(t_prefill, 3)},
        "roofline": roof,
        "mfma": mfma,
        "hbm": hbm,
        "kernels": {k: dict({"ms_per_pass": round(v[0], 4), "launches_per_pass": v[1]},
                            **({"note": SIDE_NOTE} if k in SIDE_KERNELS else {}))
                    for k, v in sorted(breakdown.items(), key=lambda kv_: -kv_[1][0])},
    }
    if not args.no_cpu_baseline:
        try:
            out["cpu_baseline"] = cpu_baseline(wl, log)
        except MemoryError:  # pragma: no cover
            out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
