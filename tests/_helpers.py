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


def oracle_model(d: recipe.Dims, storage=None) -> om.Model:
    """The oracle model of the seeded weights (or of `storage`); with FP8 experts their matrices are quantised by
    the oracle's own quantiser."""
    if storage is None:
        storage = dg_inputs.model_weights_host(d)
    w = om.weights_to_f64(storage, d.dtype)
    if d.expert_dtype == "e4m3":
        w["layers"] = [om.fp8_expert_layer(l) for l in w["layers"]]
    return om.Model(oracle_dims(d), w)


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
