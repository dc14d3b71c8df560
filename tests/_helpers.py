"""Helpers shared by the tests: building oracle models from the seeded input recipe."""
from __future__ import annotations

from dataclasses import replace

import numpy as np

import dg_inputs
from dg_inputs import recipe
from oracle import model as om
from oracle import sampler as osm


def oracle_dims(d: recipe.Dims) -> om.Dims:
    return om.Dims(n_layers=d.n_layers, d_model=d.d_model, n_heads=d.n_heads, n_kv_heads=d.n_kv_heads,
                   head_dim=d.head_dim, n_experts=d.n_experts, top_k=d.top_k, ffn_expert=d.ffn_expert,
                   ffn_shared=d.ffn_shared, vocab=d.vocab, canvas=d.canvas, dtype=d.dtype, rms_eps=d.rms_eps)


def oracle_model(d: recipe.Dims, storage=None, log=None) -> om.Model:
    """The oracle model of the seeded weights (or of `storage`); with FP8 experts (or an FP8 head) their matrices
    (or the tied embedding) are quantised by the oracle's own quantiser.  The embedding is quantised in blocks of
    rows (each row has its own scale, so blocks give the same result), with a progress line per block through
    `log` (the full vocabulary takes minutes in float64)."""
    if storage is None:
        storage = dg_inputs.model_weights_host(d)
    w = om.weights_to_f64(storage, d.dtype)
    if d.expert_dtype == "e4m3":
        w["layers"] = [om.fp8_expert_layer(l) for l in w["layers"]]
    if d.head_dtype == "e4m3":
        w["embed"] = fp8_embedding(w["embed"], log)
    return om.Model(oracle_dims(d), w)


def fp8_embedding(e: np.ndarray, log=None) -> np.ndarray:
    """The oracle's FP8 (row-scaled E4M3) dequantised embedding of a float64 matrix, in blocks of rows (each row has
    its own scale, so blocks give the same result) with a progress line per block through `log`."""
    deq = np.empty_like(e)
    step = 16384
    for r0 in range(0, e.shape[0], step):
        deq[r0:r0 + step] = om.fp8_embed({"embed": e[r0:r0 + step]})["embed"]
        if log:
            log(f"oracle FP8 embedding: rows {min(r0 + step, e.shape[0])}/{e.shape[0]}")
    return deq


def oracle_sampler(w: recipe.Workload, **kw) -> osm.Sampler:
    args = dict(n_new=w.n_new, max_steps=w.max_steps, entropy_threshold=w.entropy_threshold,
                fixed_steps=0, seed=recipe.INPUT_SEED)
    args.update(kw)
    return osm.Sampler(**args)


def small_dims(**kw) -> recipe.Dims:
    """A very small fp32 model for fast oracle-only checks."""
    base = recipe.Dims(n_layers=1, d_model=32, n_heads=4, n_kv_heads=2, head_dim=8, n_experts=4, top_k=2,
                       ffn_expert=16, ffn_shared=16, vocab=64, canvas=8, dtype="f32")
    return replace(base, **kw)
