"""Device-resident synthetic inputs (torch tensors on the GPU, filled by the device generator).

Same values as the host routines in ``dg_inputs`` (bit-identical), produced on
the GPU so that the 50 GB of bf16 weights of the full model take milliseconds.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import torch

from . import recipe
from . import fill_normal_device, fill_uniform_device
from .recipe import Dims, layer_shapes, layer_stream


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def normal_tensor(shape, seed: int, stream: int, sigma: float, dtype: str, device="cuda") -> torch.Tensor:
    t = torch.empty(tuple(shape), dtype=torch_dtype(dtype), device=device)
    fill_normal_device(t, seed, stream, sigma, dtype, torch.cuda.current_stream().cuda_stream)
    return t


def uniform_tensor(n: int, seed: int, stream: int, bound: int, device="cuda") -> torch.Tensor:
    t = torch.empty(n, dtype=torch.int32, device=device)
    fill_uniform_device(t, seed, stream, bound, torch.cuda.current_stream().cuda_stream)
    return t


def layer_weights_device(d: Dims, layer: int, seed: int = recipe.WEIGHT_SEED,
                         sigma: float = recipe.WEIGHT_SIGMA) -> Dict[str, torch.Tensor]:
    out = {}
    for name, shape in layer_shapes(d).items():
        if name in recipe.NORM_TENSORS:
            out[name] = torch.ones(shape, dtype=torch_dtype(d.dtype), device="cuda")
        else:
            out[name] = normal_tensor(shape, seed, layer_stream(layer, name), sigma, d.dtype)
    return out


def model_weights_device(d: Dims, seed: int = recipe.WEIGHT_SEED, with_embed: bool = True) -> dict:
    return {
        "embed": normal_tensor((d.vocab, d.d_model), seed, recipe.STREAM_EMBED, recipe.WEIGHT_SIGMA, d.dtype)
        if with_embed else None,
        "final_norm": torch.ones(d.d_model, dtype=torch_dtype(d.dtype), device="cuda"),
        "layers": [layer_weights_device(d, l, seed) for l in range(d.n_layers)],
    }


def from_host(storage: dict, dtype: str) -> dict:
    """Upload a storage-form weight dict (uint16 bf16 bits or float32 arrays) to the GPU."""
    def up(a):
        t = torch.from_numpy(a.copy())
        if dtype == "bf16":
            t = t.view(torch.bfloat16)
        return t.cuda()
    return {"embed": up(storage["embed"]), "final_norm": up(storage["final_norm"]),
            "layers": [{k: up(v) for k, v in layer.items()} for layer in storage["layers"]]}


def kv_tensors(d: Dims, capacity: int):
    """Key cache [L, Hkv, cap, Dh] and value cache [L, Hkv, Dh, cap] (positions contiguous)."""
    dt = torch_dtype(d.dtype)
    k = torch.zeros((max(d.n_layers, 1), d.n_kv_heads, capacity, d.head_dim), dtype=dt, device="cuda")
    v = torch.zeros((max(d.n_layers, 1), d.n_kv_heads, d.head_dim, capacity), dtype=dt, device="cuda")
    return k, v


def packed_model_weights_device(d: Dims, seed: int = recipe.WEIGHT_SEED) -> dict:
    """Device weights in the library's fragment-tiled layout, generated and converted one tensor at a time
    so that the peak memory is the packed model plus one natural tensor."""
    import block_diffusion_decoding_step_amd as dg
    emb = normal_tensor((d.vocab, d.d_model), seed, recipe.STREAM_EMBED, recipe.WEIGHT_SIGMA, d.dtype)
    out = {"final_norm": torch.ones(d.d_model, dtype=torch_dtype(d.dtype), device="cuda"), "layers": []}
    if d.head_dtype == "e4m3":
        out["embed"], out["embed_scale"] = dg.quantize_tensor_e4m3(emb)
    else:
        out["embed"] = dg.pack_tensor(emb)
    del emb
    for l in range(d.n_layers):
        layer = {}
        for name, shape in layer_shapes(d).items():
            if name in recipe.NORM_TENSORS:
                layer[name] = torch.ones(shape, dtype=torch_dtype(d.dtype), device="cuda")
            else:
                t = normal_tensor(shape, seed, layer_stream(l, name), recipe.WEIGHT_SIGMA, d.dtype)
                if d.expert_dtype == "e4m3" and name in dg.EXPERT_FIELDS:
                    layer[name], layer[name + "_scale"] = dg.quantize_tensor_e4m3(t)
                else:
                    layer[name] = dg.pack_tensor(t)
                del t
        out["layers"].append(layer)
    return out
