"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle's tests.

The generator itself is written once, in ``dgi.h`` (SplitMix64 in counter mode,
an Irwin-Hall normal and a multiply-shift uniform integer), and compiled twice:
for the host with gcc (``libdgi_host.so``) and for gfx950 with hipcc
(``libdgi_dev.so``).  Host and device values are bit-identical.  Nothing here
computes any step of the block-diffusion method.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

from . import recipe
from .recipe import (C0, C1, C2, C3, C4, WORKLOADS, Dims, Workload, gen_scale, layer_shapes, layer_stream,
                     numel)

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libdgi_host.so")
DEV_LIB = os.path.join(_HERE, "libdgi_dev.so")

_host = None
_dev = None


def build_host() -> str:
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-o", HOST_LIB, os.path.join(_HERE, "gen_host.c")]
    subprocess.run(cmd, check=True)
    return HOST_LIB


def build_dev() -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", DEV_LIB, os.path.join(_HERE, "gen_dev.hip")]
    subprocess.run(cmd, check=True, stderr=subprocess.DEVNULL)
    return DEV_LIB


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            build_host()
        lib = ctypes.CDLL(HOST_LIB)
        i64, u64, f32, vp, u32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p, ctypes.c_uint32
        lib.dgi_host_normal_f32.argtypes = [vp, i64, u64, u64, f32]
        lib.dgi_host_normal_bf16.argtypes = [vp, i64, u64, u64, f32]
        lib.dgi_host_uniform_i32.argtypes = [vp, i64, u64, u64, u32]
        lib.dgi_host_normal_bf16_range.argtypes = [vp, i64, i64, u64, u64, f32]
        lib.dgi_host_normal_f32_range.argtypes = [vp, i64, i64, u64, u64, f32]
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is not built; run __graft_entry__.build() first")
        import torch  # noqa: F401  (bind to the HIP runtime torch has loaded, see the libdg binding)
        lib = ctypes.CDLL(DEV_LIB)
        i64, u64, f32, vp, u32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p, ctypes.c_uint32
        for name in ("dgi_dev_normal_f32", "dgi_dev_normal_bf16"):
            getattr(lib, name).argtypes = [vp, i64, u64, u64, f32, vp]
            getattr(lib, name).restype = ctypes.c_int
        lib.dgi_dev_uniform_i32.argtypes = [vp, i64, u64, u64, u32, vp]
        lib.dgi_dev_uniform_i32.restype = ctypes.c_int
        _dev = lib
    return _dev


# ----------------------------------------------------------------------------- host

def normal(shape, seed: int, stream: int, sigma: float, dtype: str, first: int = 0) -> np.ndarray:
    """Host tensor of generator normals.  dtype "bf16" returns uint16 bit patterns; "f32" returns float32.

    ``first`` selects the flat index the slice starts at, so any slice of a large tensor can be
    produced without generating the rest.
    """
    n = numel(tuple(shape))
    lib = _host_lib()
    sc = gen_scale(sigma)
    if dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        lib.dgi_host_normal_bf16_range(out.ctypes.data, first, n, seed, stream, sc)
    elif dtype == "f32":
        out = np.empty(n, dtype=np.float32)
        lib.dgi_host_normal_f32_range(out.ctypes.data, first, n, seed, stream, sc)
    else:
        raise ValueError(dtype)
    return out.reshape(shape)


def uniform_int(n: int, seed: int, stream: int, bound: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _host_lib().dgi_host_uniform_i32(out.ctypes.data, n, seed, stream, bound)
    return out


def ones(shape, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return np.full(shape, 0x3F80, dtype=np.uint16)
    return np.ones(shape, dtype=np.float32)


def const(shape, value: float, dtype: str) -> np.ndarray:
    a = np.full(shape, value, dtype=np.float32)
    if dtype == "bf16":
        u = a.view(np.uint32)
        return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return a


def zeros(shape, dtype: str) -> np.ndarray:
    return np.zeros(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)


def layer_weights_host(d: Dims, layer: int, seed: int = recipe.WEIGHT_SEED,
                       sigma: float = recipe.WEIGHT_SIGMA) -> dict:
    """One layer's weights in storage form (uint16 bf16 bits or float32), norm gains set to 1."""
    out = {}
    for name, shape in layer_shapes(d).items():
        if name in recipe.NORM_TENSORS:
            out[name] = ones(shape, d.dtype)
        else:
            out[name] = normal(shape, seed, layer_stream(layer, name), sigma, d.dtype)
    return out


def embed_host(d: Dims, seed: int = recipe.WEIGHT_SEED, sigma: float = recipe.WEIGHT_SIGMA,
               rows: Optional[np.ndarray] = None) -> np.ndarray:
    """The tied embedding / head matrix E [vocab, d_model] (or only the given rows)."""
    if rows is None:
        return normal((d.vocab, d.d_model), seed, recipe.STREAM_EMBED, sigma, d.dtype)
    out = [normal((1, d.d_model), seed, recipe.STREAM_EMBED, sigma, d.dtype, first=int(r) * d.d_model)
           for r in rows]
    return np.concatenate(out, axis=0)


def model_weights_host(d: Dims, seed: int = recipe.WEIGHT_SEED) -> dict:
    return {
        "embed": embed_host(d, seed),
        "final_norm": ones((d.d_model,), d.dtype),
        "layers": [layer_weights_host(d, l, seed) for l in range(d.n_layers)],
    }


def prompt_tokens(n: int, vocab: int, seed: int = recipe.INPUT_SEED) -> np.ndarray:
    return uniform_int(n, seed, recipe.STREAM_PROMPT, vocab)


def hidden(shape, dtype: str, seed: int = recipe.INPUT_SEED, stream: int = recipe.STREAM_HIDDEN) -> np.ndarray:
    return normal(shape, seed, stream, 1.0, dtype)


# ----------------------------------------------------------------------------- device

def fill_normal_device(tensor, seed: int, stream: int, sigma: float, dtype: str, hip_stream: int = 0) -> None:
    """Fill a contiguous device tensor (any torch dtype of the right element size) with generator normals."""
    lib = _dev_lib()
    n = tensor.numel()
    sc = gen_scale(sigma)
    fn = lib.dgi_dev_normal_bf16 if dtype == "bf16" else lib.dgi_dev_normal_f32
    rc = fn(ctypes.c_void_p(tensor.data_ptr()), n, seed, stream, sc, ctypes.c_void_p(hip_stream))
    if rc != 0:
        raise RuntimeError(f"device input generator failed with HIP error {rc}")


def fill_uniform_device(tensor, seed: int, stream: int, bound: int, hip_stream: int = 0) -> None:
    rc = _dev_lib().dgi_dev_uniform_i32(ctypes.c_void_p(tensor.data_ptr()), tensor.numel(), seed, stream, bound,
                                        ctypes.c_void_p(hip_stream))
    if rc != 0:
        raise RuntimeError(f"device input generator failed with HIP error {rc}")
