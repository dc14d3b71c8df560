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


# ----------------------------------------------------------------------------- OCP FP8 E4M3
# The 8-bit float of the OCP "8-bit Floating Point Specification" (OFP8), E4M3 variant: one sign bit, four
# exponent bits with bias 7, three mantissa bits.  Exponent field 0 holds the subnormals 0.mmm * 2^-6; the
# exponent field 15 holds normal values except mantissa 111, which is NaN (there are no infinities), so the
# largest finite magnitude is 1.110b * 2^8 = 448 and the smallest subnormal 2^-9.

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_QUANTUM_SUBNORMAL = 2.0 ** -9


def e4m3_decode(codes) -> np.ndarray:
    """uint8 E4M3 codes -> float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * E4M3_QUANTUM_SUBNORMAL, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_round(x) -> np.ndarray:
    """float64 -> the nearest E4M3 value, ties to the even mantissa, magnitudes beyond 448 saturated to 448.

    In the normal range the spacing of E4M3 values in the binade [2^E, 2^(E+1)) is 2^(E-3) (three mantissa
    bits); below 2^-6 it is the subnormal spacing 2^-9.  Dividing by a power of two is exact, so rounding
    |x| / spacing to the nearest even integer (numpy's round) and scaling back is the exact RNE result; a
    carry into the next binade lands on a representable value."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(np.where(a > 0, a, 1.0))       # a = f * 2^e with f in [0.5, 1): binade exponent e - 1
    q = np.where(a >= E4M3_MIN_NORMAL, np.exp2((e - 1 - 3).astype(np.float64)), E4M3_QUANTUM_SUBNORMAL)
    r = np.round(a / q) * q
    r = np.minimum(r, E4M3_MAX)
    out = np.copysign(r, x)
    return np.where(np.isnan(x), np.nan, out)


def e4m3_encode(values) -> np.ndarray:
    """E4M3-representable float64 values (finite) -> their uint8 codes.  A zero keeps its sign: +0 is code 0x00,
    -0 code 0x80 (a negative value that rounds to zero rounds to -0, as in IEEE arithmetic)."""
    v = np.asarray(values, dtype=np.float64)
    table = e4m3_decode(np.arange(256))
    finite = np.nonzero(~np.isnan(table) & ~((np.arange(256) == 0x80)))[0]   # the negative zero is added below
    order = np.argsort(table[finite])
    codes = finite[order][np.searchsorted(table[finite][order], v)]
    assert np.array_equal(table[codes], v), "value not representable in E4M3"
    codes = np.where((v == 0) & np.signbit(v), 0x80, codes)
    return codes.astype(np.uint8)


def round_e4m3_rows(w) -> tuple:
    """Per-row (per-output-channel) E4M3 quantisation of a weight matrix [..., rows, cols], as values.

    The scale of a row is s = amax / 448 in float32 (1 for an all-zero row); each weight is divided by s in
    float32 and rounded to E4M3 (ties to even, saturated).  The row's dequantised weights are value * s.
    Returns (E4M3 values float64 [..., rows, cols], scales float32 [..., rows]).  The decisions are taken in
    float32, the precision the quantiser kernel takes them in."""
    w32 = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w32), axis=-1)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    quot = (w32 / s[..., None]).astype(np.float32)
    return e4m3_round(quot.astype(np.float64)), s


def quantize_e4m3_rows(w) -> tuple:
    """round_e4m3_rows with the values as their codes: (codes uint8 [..., rows, cols], scales float32 [..., rows])."""
    v, s = round_e4m3_rows(w)
    return e4m3_encode(v), s
