"""Workload shapes, seeds and the synthetic-input recipe.

This module describes *what the inputs are* (dimensions, seeds, which tensor is
drawn from which generator stream and with which scale).  It contains no step
of the block-diffusion method.  Both the GPU path's tests/bench and the oracle's
tests use it so that they see the same inputs.

Dimensions come from the model the pages describe (a 128-expert, 8-active +
1-shared MoE backbone with a 262K vocabulary and a 256-slot canvas; pages
"DiffusionGemma 26B: How Google's Text Diffusion Model Generates Tokens in
Parallel", section "Architecture Details") with the per-layer widths of the
benchmark workloads listed here, since the pages give only parameter totals.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Iterator, Optional, Tuple

WEIGHT_SEED = 0
INPUT_SEED = 1
WEIGHT_SIGMA = 0.02

# generator streams for non-weight inputs (seed INPUT_SEED)
STREAM_PROMPT = 1
STREAM_HIDDEN = 2
STREAM_PREFIX_K = 4
STREAM_PREFIX_V = 5
STREAM_PREFIX_HIDDEN = 6

# per-tensor streams for weights (seed WEIGHT_SEED)
STREAM_EMBED = 0x10
_LAYER_STREAM_BASE = 0x100
_LAYER_STREAM_STRIDE = 0x20
LAYER_TENSORS = ("wqkv", "wo", "w_router", "w_gate_up", "w_down", "ws_gate_up", "ws_down")
NORM_TENSORS = ("attn_norm", "ffn_norm")


@dataclass(frozen=True)
class Dims:
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    ffn_expert: int
    ffn_shared: int
    vocab: int
    canvas: int
    dtype: str  # "f32" or "bf16"
    rms_eps: float = 1e-6
    expert_dtype: str = ""  # "" (as dtype) or "e4m3": routed experts' weights quantised to FP8 per output channel
    head_dtype: str = ""    # "" (as dtype) or "e4m3": the tied embedding / head quantised to FP8 per vocabulary row

    @property
    def qkv_rows(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim


@dataclass(frozen=True)
class Workload:
    name: str
    dims: Dims
    prefix: int            # tokens already in the KV cache when the block starts
    n_new: int             # new slots kept per pass (keep count k_t = min(S, t*n_new))
    fixed_steps: int       # T for timing runs (0 = adaptive only)
    max_steps: int = 48
    entropy_threshold: float = 0.05
    blocks: int = 1
    description: str = ""


C0 = Workload(
    name="tiny_fp32",
    dims=Dims(n_layers=2, d_model=256, n_heads=4, n_kv_heads=2, head_dim=64, n_experts=8, top_k=2,
              ffn_expert=512, ffn_shared=512, vocab=4096, canvas=32, dtype="f32"),
    prefix=64, n_new=4, fixed_steps=0,
    description="2 layers, d 256, 4 q / 2 KV heads of dim 64, 8 experts top-2 + 1 shared (ffn 512), "
                "vocab 4096, prefix 64, canvas 32, keep 4 per pass, fp32",
)

_BIG = Dims(n_layers=30, d_model=2816, n_heads=16, n_kv_heads=8, head_dim=128, n_experts=128, top_k=8,
            ffn_expert=704, ffn_shared=2816, vocab=262144, canvas=256, dtype="bf16")

C1 = Workload(
    name="moe_layer_bf16", dims=replace(_BIG, n_layers=1), prefix=2048, n_new=26, fixed_steps=10,
    description="one MoE layer, d 2816, 16 q / 8 KV heads of dim 128, canvas 256 over a 2048-token prefix, "
                "128 experts top-8 + 1 shared, bf16",
)
C2 = Workload(
    name="head_bf16", dims=replace(_BIG, n_layers=0), prefix=0, n_new=26, fixed_steps=10,
    description="256 slots x 2816 hidden through the tied 262144-vocab head with fused softmax/entropy/"
                "argmax and the keep/re-randomise update, bf16",
)
C3 = Workload(
    name="full_loop_bf16", dims=_BIG, prefix=4096, n_new=26, fixed_steps=10,
    description="30 layers, 4096-token prompt prefilled, 256-slot canvas, T=10, bf16",
)
C4 = Workload(
    name="long_context_bf16", dims=_BIG, prefix=131072, n_new=26, fixed_steps=10, blocks=4,
    description="the 30-layer model over a 131072-token prefix, 4 consecutive committed blocks at T=10, bf16",
)

C3_FP8 = Workload(
    name="full_loop_fp8", dims=replace(_BIG, expert_dtype="e4m3", head_dtype="e4m3"), prefix=4096, n_new=26,
    fixed_steps=10,
    description="the full-loop workload with the routed experts' weights and the tied embedding / vocab head in FP8 "
                "(OCP E4M3, one scale per output channel or vocabulary row, quantised from the same bf16 weights); "
                "everything else bf16",
)

WORKLOADS = {w.name: w for w in (C0, C1, C2, C3, C4, C3_FP8)}


def layer_stream(layer: int, tensor: str) -> int:
    return _LAYER_STREAM_BASE + layer * _LAYER_STREAM_STRIDE + LAYER_TENSORS.index(tensor)


def layer_shapes(d: Dims) -> dict:
    return {
        "attn_norm": (d.d_model,),
        "wqkv": (d.qkv_rows, d.d_model),
        "wo": (d.d_model, d.n_heads * d.head_dim),
        "ffn_norm": (d.d_model,),
        "w_router": (d.n_experts, d.d_model),
        "w_gate_up": (d.n_experts, 2 * d.ffn_expert, d.d_model),
        "w_down": (d.n_experts, d.d_model, d.ffn_expert),
        "ws_gate_up": (2 * d.ffn_shared, d.d_model),
        "ws_down": (d.d_model, d.ffn_shared),
    }


def gen_scale(sigma: float):
    """fp32 multiplier turning the generator's integer sum into a value of std sigma."""
    import numpy as np
    return np.float32(sigma / 75674.38473)


def numel(shape: Tuple[int, ...]) -> int:
    n = 1
    for s in shape:
        n *= s
    return n


def param_count(d: Dims) -> Tuple[int, int]:
    """(total, active per token) parameter counts of the dims, embedding counted once (tied head)."""
    per_layer = sum(numel(s) for s in layer_shapes(d).values())
    expert = numel(layer_shapes(d)["w_gate_up"][1:]) + numel(layer_shapes(d)["w_down"][1:])
    total = d.n_layers * per_layer + d.vocab * d.d_model + d.d_model
    active = total - d.n_layers * (d.n_experts - d.top_k) * expert
    return total, active
