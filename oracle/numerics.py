"""Storage-precision helpers of the oracle (test infrastructure only).

The GPU path stores some tensors in bf16 between kernels; the oracle keeps its
arithmetic in float64 and rounds to bf16 (round to nearest, ties to even) at
exactly those storage points, so the two compute the same quantity.  In fp32
workloads no rounding is applied: the oracle stays in float64 throughout.

Decisions that floating point turns into integers (router top-k, argmax,
confidence ranking) are taken on values rounded to float32, the precision in
which the GPU kernels take them.
"""
from __future__ import annotations

import numpy as np

_MIN_NORMAL_F32 = 2.0 ** -126


def bf16_round(x) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), returned as float64.

    bf16 keeps 7 of float64's 52 fraction bits, so the low 45 bits are rounded
    away directly in the float64 bit pattern (no double rounding through fp32).
    Values below the fp32 normal range go through float32 first.
    """
    x = np.asarray(x, dtype=np.float64)
    u = x.view(np.uint64).copy()
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    u = (u + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    out = u.view(np.float64)
    tiny = np.abs(x) < _MIN_NORMAL_F32
    if np.any(tiny):
        f = x[tiny].astype(np.float32).view(np.uint32)
        f = (f + np.uint32(0x7FFF) + ((f >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
        out = out.copy()
        out[tiny] = f.view(np.float32).astype(np.float64)
    nan = np.isnan(x)
    if np.any(nan):
        out = np.where(nan, np.nan, out)
    return out


def from_bf16_bits(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def from_storage(a, dtype: str) -> np.ndarray:
    """Storage tensor (uint16 bf16 bits, or float32) -> float64 values."""
    if dtype == "bf16":
        return from_bf16_bits(a)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def rounder(dtype: str):
    """The storage rounding applied at bf16 store points; identity in fp32 workloads."""
    if dtype == "bf16":
        return bf16_round
    return lambda x: np.asarray(x, dtype=np.float64)


def f32(x) -> np.ndarray:
    """Round to float32 (the kernels' decision precision), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
