"""Pins of the oracle's FP8 (OCP E4M3) weights: decoding, rounding, per-channel quantisation, scaled experts.

The routed experts of the FP8 workload hold E4M3 weights with one float32 scale per output channel, the
precision of the pages' headline figures ([P2] "DiffusionGemma 26B: How Google's Text Diffusion Model
Generates Tokens in Parallel", "Benchmark Numbers": one H100 in FP8 at batch 1; [P1] "DiffusionGemma: When
Text Generation Stops Being Sequential", "Where it actually pays off: local, single-user inference").  The
decoding and rounding are checked against torch's float8_e4m3fn conversions (a library routine written
independently of the oracle) on every code and every tie, and against the format's fixed points.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import model as om
from oracle import numerics

CODES = np.arange(256)


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).float().double().numpy()


def _torch_round(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).float().double().numpy()


def test_decode_every_code():
    """All 256 codes against torch's decoding, plus the format's fixed points: 448 is the largest finite value
    (0x7E), 2^-9 the smallest subnormal (0x01), 2^-6 the smallest normal (0x08), 0x7F / 0xFF are NaN, and the
    positive codes are increasing.  Catches: a bias of 8 (the FNUZ variant), a missing subnormal range, an
    infinity code, a swapped exponent / mantissa split."""
    got = numerics.e4m3_decode(CODES)
    ref = _torch_decode(CODES)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x38] == 1.0
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and np.sum(np.isnan(got)) == 2
    pos = got[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(got[0x80:0xFF], -pos)


def test_round_ties_neighbours_and_codes():
    """Every finite code rounds to itself; the midpoint of two neighbouring codes rounds to the one with the even
    mantissa; a hair either side rounds to the nearer one; all of it equal to torch's conversion.  Catches:
    round-half-up, truncation, a wrong spacing in some binade, the subnormal spacing."""
    pos = numerics.e4m3_decode(CODES[:0x7F])
    assert np.array_equal(numerics.e4m3_round(pos), pos)
    assert np.array_equal(numerics.e4m3_round(-pos), -pos)
    lo, hi = pos[:-1], pos[1:]
    mid = (lo + hi) / 2
    even = np.where((CODES[:0x7E] & 1) == 0, lo, hi)
    assert np.array_equal(numerics.e4m3_round(mid), even)
    assert np.array_equal(numerics.e4m3_round(-mid), -even)
    eps = (hi - lo) * 1e-3
    assert np.array_equal(numerics.e4m3_round(mid - eps), lo)
    assert np.array_equal(numerics.e4m3_round(mid + eps), hi)
    for x in (mid, mid - eps, mid + eps, -mid):
        assert np.array_equal(numerics.e4m3_round(x.astype(np.float32)), _torch_round(x))


def test_round_random_and_saturation():
    """Random float32 magnitudes over the whole range (log-uniform, both signs) equal torch's conversion; beyond
    the largest value the rounding saturates at 448 (torch keeps ties at 448 up to 464 and returns NaN above,
    the reading here is saturation, stated with the quantiser)."""
    rng = np.random.default_rng(3)
    x = (np.exp(rng.uniform(np.log(2.0 ** -12), np.log(464.0), 200_000)) * rng.choice([-1, 1], 200_000))
    x = x.astype(np.float32)
    assert np.array_equal(numerics.e4m3_round(x), _torch_round(x))
    big = np.array([448.0, 460.0, 464.0, 465.0, 1e4, np.float32(3.0e38)])
    assert np.array_equal(numerics.e4m3_round(big), np.full(6, 448.0))
    assert np.array_equal(numerics.e4m3_round(-big), np.full(6, -448.0))
    assert numerics.e4m3_round(2.0 ** -10) == 0.0 and numerics.e4m3_round(2.0 ** -10 * 1.001) == 2.0 ** -9
    assert np.isnan(numerics.e4m3_round(np.nan))


def test_encode_inverts_decode():
    pos = numerics.e4m3_decode(CODES[:0x7F])
    assert np.array_equal(numerics.e4m3_encode(pos), CODES[:0x7F].astype(np.uint8))
    assert np.array_equal(numerics.e4m3_encode(-pos), (CODES[:0x7F] | 0x80).astype(np.uint8))


def test_codes_equal_torch_codes_including_signed_zero():
    """Codes of rounded values, byte for byte against torch's float8_e4m3fn cast, on every tie, the codes, small
    negative values that round to -0 (code 0x80) and zeros of both signs."""
    pos = numerics.e4m3_decode(CODES[:0x7F])
    mids = (pos[:-1] + pos[1:]) / 2
    x = np.concatenate([mids, -mids, pos, -pos, [-0.0, 0.0, -2.0 ** -10, -1e-5, 2.0 ** -11]]).astype(np.float32)
    got = numerics.e4m3_encode(numerics.e4m3_round(x))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    assert got[-5] == 0x80 and got[-4] == 0x00 and got[-3] == 0x80 and got[-2] == 0x80


def test_quantize_rows_closed_forms():
    """A row's largest magnitude maps to the code of +-448 and its scale is amax / 448 in float32; halves of it
    to 224; zero to code 0; an all-zero row keeps scale 1.  Random rows: the dequantised weights lie within half
    an E4M3 spacing of the originals (relative 2^-4 in the normal range, 2^-10 s absolute below it)."""
    a = np.float32(0.0371)
    w = np.array([[a, -a, a / 2, 0.0, -a / 4], [0, 0, 0, 0, 0]], dtype=np.float32)
    codes, s = numerics.quantize_e4m3_rows(w)
    assert s.dtype == np.float32 and s[0] == np.float32(a / np.float32(448.0)) and s[1] == 1.0
    v = numerics.e4m3_decode(codes)
    assert list(v[0]) == [448.0, -448.0, 224.0, 0.0, -112.0] and np.all(v[1] == 0)
    rng = np.random.default_rng(4)
    w = (rng.normal(size=(8, 2816)) * 0.02).astype(np.float32)
    codes, s = numerics.quantize_e4m3_rows(w)
    deq = numerics.e4m3_decode(codes) * s[:, None].astype(np.float64)
    bound = np.maximum(np.abs(w) * 2.0 ** -4, 2.0 ** -10 * s[:, None]) * (1 + 1e-6)
    assert np.all(np.abs(deq - w) <= bound)
    assert np.all(np.max(np.abs(numerics.e4m3_decode(codes)), axis=1) == 448.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fp8_experts_are_the_dequantised_ffn(dtype):
    """The scaled routed experts equal the plain experts of the dequantised weights diag(s) Q, and with every
    expert identical the routed sum is that one dequantised FFN whatever the routing.  Catches: the scale applied
    to the wrong axis (input channel), to the gate only, or after the SwiGLU product."""
    rnd = numerics.rounder(dtype)
    rng = np.random.default_rng(5)
    d, f, E, k = 64, 32, 4, 2
    gu = rng.normal(size=(2 * f, d)) * 0.3
    dn = rng.normal(size=(d, f)) * 0.3
    layer = om.fp8_expert_layer({"w_gate_up": np.broadcast_to(gu, (E, 2 * f, d)).copy(),
                                 "w_down": np.broadcast_to(dn, (E, d, f)).copy()})
    q_gu, s_gu = layer["w_gate_up"][0], layer["w_gate_up_scale"][0]
    q_dn, s_dn = layer["w_down"][0], layer["w_down_scale"][0]
    xn = rnd(rng.normal(size=(9, d)))
    idx, w, _, _ = om.route(xn, rng.normal(size=(E, d)), k)
    got = om.moe_routed(xn, idx, w, layer["w_gate_up"], layer["w_down"], rnd, layer["w_gate_up_scale"],
                        layer["w_down_scale"])
    deq_gu = q_gu * s_gu[:, None]
    deq_dn = q_dn * s_dn[:, None]
    gate, up = xn @ deq_gu[:f].T, xn @ deq_gu[f:].T
    dense = rnd(rnd(gate / (1 + np.exp(-gate)) * up) @ deq_dn.T)
    np.testing.assert_allclose(got, dense, rtol=1e-12, atol=1e-13)
    assert np.max(np.abs(deq_gu - gu)) <= 2.0 ** -4 * np.max(np.abs(gu)) * 1.0001


def test_fp8_embedding_is_the_row_dequantised_matrix():
    """om.fp8_embed replaces the tied embedding by code * row scale (numerics.quantize_e4m3_rows, one scale per
    vocabulary row), which the lookup rounds to the storage type and the head multiplies directly.  Rows made of
    E4M3 values times a power of two (each holding +-448 times it) come back exactly; rows of very different sizes
    each keep the E4M3 relative bound.  Catches: a scale per column instead of per row, a missing scale, a lookup
    that skips the storage rounding."""
    rng = np.random.default_rng(11)
    pos = numerics.e4m3_decode(CODES[:0x7F])
    vals = np.concatenate([pos, -pos])
    rows = rng.choice(vals, size=(6, 128))
    rows[:, 0] = 448.0
    k = np.array([-12, -3, 0, 2, 5, -7], dtype=np.float64)
    exact = rows * np.exp2(k)[:, None]
    assert np.array_equal(om.fp8_embed({"embed": exact})["embed"], exact)
    mags = np.array([1e-3, 0.02, 7.0])[:, None]
    e = (rng.normal(size=(3, 256)) * mags).astype(np.float32).astype(np.float64)
    deq = om.fp8_embed({"embed": e, "final_norm": None})["embed"]
    bound = np.maximum(np.abs(e) * 2.0 ** -4, 2.0 ** -10 * np.max(np.abs(e), axis=1, keepdims=True) / 448.0)
    assert np.all(np.abs(deq - e) <= bound * (1 + 1e-6))
    dims = om.Dims(n_layers=0, d_model=256, n_heads=1, n_kv_heads=1, head_dim=64, n_experts=2, top_k=1,
                   ffn_expert=32, ffn_shared=32, vocab=3, canvas=4, dtype="bf16")
    m = om.Model(dims, {"embed": deq, "final_norm": np.ones(256), "layers": []})
    got = m.embed([2, 0, 1])
    assert np.array_equal(got, numerics.bf16_round(deq[[2, 0, 1]]))
    assert not np.array_equal(got, deq[[2, 0, 1]])   # the dequantised rows are not bf16 values themselves


def test_row_values_are_the_decoded_codes():
    """round_e4m3_rows (the values the FP8 experts and head are built from) and quantize_e4m3_rows (their codes,
    as the quantiser kernel writes them) agree: decoding the codes gives the values bit for bit, signed zeros
    included, and the scales are the same."""
    rng = np.random.default_rng(3)
    w = np.concatenate([rng.normal(size=(64, 512)) * 0.02, rng.normal(size=(4, 512)) * 1e-6,
                        np.zeros((1, 512))]).astype(np.float32)
    w[0, :5] = [-1e-9, 0.0, -0.0, 3.0, -3.0]
    v, s = numerics.round_e4m3_rows(w)
    c, s2 = numerics.quantize_e4m3_rows(w)
    d = numerics.e4m3_decode(c)
    assert np.array_equal(s, s2)
    assert np.array_equal(v, d) and np.array_equal(np.signbit(v), np.signbit(d))
    assert np.signbit(v[0, 0]) and v[0, 0] == 0.0   # a negative weight that rounds to zero keeps its sign
