"""Python binding of libdg, the MI355X block-diffusion denoising library.

Argument marshalling only: every function here forwards to the C ABI declared
in ``include/dg.h`` under the same name, passing device pointers taken from
torch tensors (torch is used for device memory and streams, nothing else) and
raising ``DGError`` on a negative status.  No step of the method runs in
Python, and there is no fallback: if ``libdg.so`` is missing, importing the
package fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
# DG_LIBRARY selects another build of the same library (the host-sanitizer build the CPU tests of the C ABI use)
LIB_PATH = os.environ.get("DG_LIBRARY") or os.path.join(_HERE, "libdg.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() (hipcc, gfx950) first")
# torch brings its own HIP runtime and loads it under a different file name than the
# one libdg records; loading torch first makes libdg bind to that same runtime
# instead of starting a second one in the process.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

DG_OK, DG_ERR_INVALID, DG_ERR_UNSUPPORTED, DG_ERR_KV_FULL, DG_ERR_WORKSPACE, DG_ERR_HIP = 0, -1, -2, -3, -4, -5
DG_F32, DG_BF16, DG_E4M3 = 0, 1, 2
DG_STOP_NONE, DG_STOP_ENTROPY, DG_STOP_STABLE, DG_STOP_CAP, DG_STOP_FIXED, DG_STOP_SETTLED = 0, 1, 2, 3, 4, 5
DG_WARN_NUMERIC = 0x1
# sampler variants (dg_sampler.flags)
DG_SAMPLE_GUMBEL, DG_SAMPLE_ANNEAL, DG_KEEP_ENTROPY, DG_KEEP_LOCK, DG_STOP_AND = 0x1, 0x2, 0x4, 0x8, 0x10
EXPORTED = ("dg_workspace_size", "dg_prefill_kv", "dg_denoise_step", "dg_canvas_update", "dg_commit_block",
            "dg_generate_block", "dg_generate_block_overlapped", "dg_layer_forward", "dg_vocab_head", "dg_stop_check", "dg_status_string",
            "dg_generate_blocks", "dg_generate_blocks_overlapped", "dg_verify_block", "dg_denoise_step_sampler", "dg_canvas_update_sampler", "dg_vocab_head_sampler", "dg_sampler_inv_temperature",
            "dg_last_hip_error", "dg_timing_start", "dg_timing_stop", "dg_packed_elems", "dg_pack_matrix",
            "dg_side_create", "dg_side_destroy", "dg_generate_speculative", "dg_packed_bytes_e4m3", "dg_quantize_e4m3", "dg_denoise_step_noalloc", "dg_noalloc_scratch_bytes")
# kernel classes of dg_timing_* (dg_kernel in dg.h), in enum order
KERNELS = ("embed", "rmsnorm", "gemm_qkv", "attention", "attn_merge", "gemm_o", "route",
           "moe_gate_up", "moe_down", "shared_gate_up", "shared_down", "moe_combine", "vocab_head",
           "head_merge", "stop_check", "canvas_update", "kv_scatter")


class DGError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _lib.dg_status_string(status).decode()
        if status == DG_ERR_HIP:
            msg += f" (hip error {_lib.dg_last_hip_error()})"
        super().__init__(f"{fn}: {msg} [{status}]")
        self.status = status


# ----------------------------------------------------------------------------- structs (mirror dg.h)

class dg_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("ffn_expert", ctypes.c_int32), ("ffn_shared", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("canvas", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float), ("expert_dtype", ctypes.c_int32),
                ("head_dtype", ctypes.c_int32)]


class dg_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("attn_norm", "wqkv", "wo", "ffn_norm", "w_router", "w_gate_up",
                                               "w_down", "ws_gate_up", "ws_down", "w_gate_up_scale",
                                               "w_down_scale")]


class dg_weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("h_layers", ctypes.POINTER(dg_layer_weights)), ("embed_scale", ctypes.c_void_p)]


class dg_kv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("len", ctypes.c_int64),
                ("capacity", ctypes.c_int64)]


class dg_sampler(ctypes.Structure):
    _fields_ = [("n_new", ctypes.c_int32), ("max_steps", ctypes.c_int32), ("fixed_steps", ctypes.c_int32),
                ("entropy_threshold", ctypes.c_float), ("inv_temperature", ctypes.c_float),
                ("flags", ctypes.c_uint32), ("seed", ctypes.c_uint64), ("temperature_first", ctypes.c_float),
                ("temperature_last", ctypes.c_float)]


class dg_block_status(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int32), ("reason", ctypes.c_int32), ("mean_entropy", ctypes.c_float),
                ("flags", ctypes.c_uint32)]


class dg_side(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p), ("fork", ctypes.c_void_p), ("join", ctypes.c_void_p)]


class dg_spec_status(ctypes.Structure):
    _fields_ = [("rounds", ctypes.c_int32), ("tokens", ctypes.c_int32), ("accepted", ctypes.c_int32),
                ("next_token", ctypes.c_int32)]


class dg_debug(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_void_p), ("route_idx", ctypes.c_void_p), ("route_w", ctypes.c_void_p),
                ("router_logits", ctypes.c_void_p)]


_P = ctypes.POINTER
_vp, _i32, _i64, _u32, _u64, _f32, _sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                          ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t)
_SIGS = {
    "dg_workspace_size": [_P(dg_config), _i64, _P(_sz)],
    "dg_prefill_kv": [_P(dg_config), _P(dg_weights), _P(dg_kv), _vp, _i64, _vp, _sz, _P(dg_side), _vp],
    "dg_denoise_step": [_P(dg_config), _P(dg_weights), _P(dg_kv), _vp, _f32, _vp, _vp, _vp, _P(dg_debug), _vp, _sz,
                        _P(dg_side), _vp],
    "dg_canvas_update": [_P(dg_config), _vp, _vp, _i32, _u64, _u32, _u32, _vp, _vp, _vp],
    "dg_commit_block": [_P(dg_config), _P(dg_weights), _P(dg_kv), _vp, _vp, _sz, _P(dg_side), _vp],
    "dg_generate_block": [_P(dg_config), _P(dg_weights), _P(dg_kv), _P(dg_sampler), _u32, _vp, _P(dg_block_status),
                          _vp, _sz, _P(dg_side), _vp],
    "dg_generate_block_overlapped": [_P(dg_config), _P(dg_weights), _P(dg_kv), _P(dg_sampler), _u32, _vp, _i32, _vp,
                                     _P(dg_block_status), _vp, _sz, _P(dg_side), _vp],
    "dg_generate_blocks": [_P(dg_config), _P(dg_weights), _P(dg_kv), _i32, _P(dg_sampler), _P(_u32), _vp,
                           _P(dg_block_status), _vp, _sz, _P(dg_side), _vp],
    "dg_generate_blocks_overlapped": [_P(dg_config), _P(dg_weights), _P(dg_kv), _i32, _P(dg_sampler), _P(_u32), _vp,
                                      _i32, _vp, _P(dg_block_status), _vp, _sz, _P(dg_side), _vp],
    "dg_verify_block": [_P(dg_config), _P(dg_weights), _P(dg_kv), _vp, _vp, _P(_i32), _P(_i32), _vp, _sz, _P(dg_side), _vp],
    "dg_layer_forward": [_P(dg_config), _P(dg_weights), _i32, _P(dg_kv), _vp, _vp, _i64, _i32, _P(dg_debug), _vp,
                         _sz, _P(dg_side), _vp],
    "dg_vocab_head": [_P(dg_config), _P(dg_weights), _vp, _i64, _f32, _vp, _vp, _vp, _vp, _sz, _vp],
    "dg_stop_check": [_P(dg_config), _P(dg_sampler), _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "dg_denoise_step_sampler": [_P(dg_config), _P(dg_weights), _P(dg_kv), _P(dg_sampler), _u32, _i32, _vp, _vp, _vp,
                                _vp, _vp, _sz, _P(dg_side), _vp],
    "dg_canvas_update_sampler": [_P(dg_config), _P(dg_sampler), _u32, _i32, _vp, _vp, _vp, _vp, _vp, _vp],
    "dg_vocab_head_sampler": [_P(dg_config), _P(dg_weights), _P(dg_sampler), _u32, _i32, _vp, _i64, _vp, _vp, _vp,
                              _vp, _sz, _vp],
    "dg_sampler_inv_temperature": [_P(dg_sampler), _i32, _P(ctypes.c_float)],
    "dg_packed_elems": [_i64, _i64, _P(_i64)],
    "dg_pack_matrix": [_vp, _vp, _i64, _i64, _i64, _i32, _vp],
    "dg_side_create": [_P(dg_side)],
    "dg_generate_speculative": [_P(dg_config), _P(dg_weights), _P(dg_kv), _P(dg_sampler), _u32, _i32, _i32, _vp,
                                _P(_i32), _P(dg_spec_status), _vp, _sz, _P(dg_side), _vp],
    "dg_packed_bytes_e4m3": [_i64, _i64, _P(_i64)],
    "dg_quantize_e4m3": [_vp, _vp, _vp, _i64, _i64, _i64, _vp],
    "dg_denoise_step_noalloc": [_P(dg_config), _P(dg_weights), _P(dg_kv), _vp, _f32, _vp, _vp, _vp, _P(dg_side), _vp],
    "dg_noalloc_scratch_bytes": [_P(_sz)],
    "dg_side_destroy": [_P(dg_side)],
}
for _name, _args in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_int
_lib.dg_status_string.argtypes = [ctypes.c_int]
_lib.dg_status_string.restype = ctypes.c_char_p
_lib.dg_last_hip_error.argtypes = []
_lib.dg_last_hip_error.restype = ctypes.c_int
_lib.dg_timing_start.argtypes = [ctypes.c_uint64]
_lib.dg_timing_start.restype = ctypes.c_int
_lib.dg_timing_stop.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
_lib.dg_timing_stop.restype = ctypes.c_int


# ----------------------------------------------------------------------------- marshalling helpers

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _side(side):
    if side is None:
        return None
    return ctypes.byref(side.struct if isinstance(side, Side) else side)


class Side:
    """A caller-owned dg_side: the side stream and fork/join events of the shared expert, made by
    dg_side_create and destroyed by close() (or when the object is collected)."""

    def __init__(self):
        self.struct = dg_side()
        _check("dg_side_create", _lib.dg_side_create(ctypes.byref(self.struct)))

    def close(self) -> None:
        if self.struct.stream:
            _check("dg_side_destroy", _lib.dg_side_destroy(ctypes.byref(self.struct)))

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover - interpreter shutdown
            pass


def _check(fn: str, rc: int) -> None:
    if rc != DG_OK:
        raise DGError(fn, rc)


def make_config(dims, dtype: Optional[str] = None, rms_eps: float = 1e-6) -> dg_config:
    """A dg_config from any object with the dimension attributes of the C struct."""
    dt = dtype or getattr(dims, "dtype", "bf16")
    return dg_config(n_layers=dims.n_layers, d_model=dims.d_model, n_heads=dims.n_heads,
                     n_kv_heads=dims.n_kv_heads, head_dim=dims.head_dim, n_experts=dims.n_experts,
                     top_k=dims.top_k, ffn_expert=dims.ffn_expert, ffn_shared=dims.ffn_shared, vocab=dims.vocab,
                     canvas=dims.canvas, dtype=DG_BF16 if dt == "bf16" else DG_F32,
                     rms_eps=getattr(dims, "rms_eps", rms_eps), rope_theta=0.0,
                     expert_dtype=DG_E4M3 if getattr(dims, "expert_dtype", "") == "e4m3" else 0,
                     head_dtype=DG_E4M3 if getattr(dims, "head_dtype", "") == "e4m3" else 0)


class Weights:
    """dg_weights built from device tensors; keeps the tensors alive."""

    LAYER_FIELDS = ("attn_norm", "wqkv", "wo", "ffn_norm", "w_router", "w_gate_up", "w_down", "ws_gate_up",
                    "ws_down", "w_gate_up_scale", "w_down_scale")

    def __init__(self, embed, final_norm, layers: Sequence[Dict[str, object]], embed_scale=None):
        self._keep = [embed, final_norm, list(layers), embed_scale]
        n = len(layers)
        self._layers = (dg_layer_weights * max(n, 1))()
        for i, lw in enumerate(layers):
            for f in self.LAYER_FIELDS:
                setattr(self._layers[i], f, _ptr(lw.get(f)))
        self.struct = dg_weights(embed=_ptr(embed), final_norm=_ptr(final_norm),
                                 h_layers=ctypes.cast(self._layers, _P(dg_layer_weights)),
                                 embed_scale=_ptr(embed_scale))


class KV:
    """dg_kv over caller-owned key/value tensors; ``len`` tracks the committed length."""

    def __init__(self, k, v, capacity: int, length: int = 0):
        self.k, self.v = k, v
        self.struct = dg_kv(k=_ptr(k), v=_ptr(v), len=length, capacity=capacity)

    @property
    def len(self) -> int:
        return int(self.struct.len)

    @len.setter
    def len(self, value: int) -> None:
        self.struct.len = value


def _w(weights):
    return ctypes.byref(weights.struct if isinstance(weights, Weights) else weights)


def _kv(kv):
    return ctypes.byref(kv.struct if isinstance(kv, KV) else kv)


# ----------------------------------------------------------------------------- C ABI, same names

def dg_workspace_size(cfg: dg_config, max_tokens: int) -> int:
    out = ctypes.c_size_t(0)
    _check("dg_workspace_size", _lib.dg_workspace_size(ctypes.byref(cfg), max_tokens, ctypes.byref(out)))
    return int(out.value)


def dg_prefill_kv(cfg, weights, kv, tokens, n: int, ws, ws_bytes: int, side=None, stream=None) -> None:
    _check("dg_prefill_kv", _lib.dg_prefill_kv(ctypes.byref(cfg), _w(weights), _kv(kv), _ptr(tokens), n, _ptr(ws),
                                               ws_bytes, _side(side), _stream(stream)))


def dg_denoise_step(cfg, weights, kv, canvas, inv_temperature: float, pred, conf, entropy, dbg=None, ws=None,
                    ws_bytes: int = 0, side=None, stream=None) -> None:
    d = _dbg(dbg)
    _check("dg_denoise_step", _lib.dg_denoise_step(ctypes.byref(cfg), _w(weights), _kv(kv), _ptr(canvas),
                                                   inv_temperature, _ptr(pred), _ptr(conf), _ptr(entropy), d,
                                                   _ptr(ws), ws_bytes, _side(side), _stream(stream)))


def dg_denoise_step_noalloc(cfg, weights, kv, canvas, inv_temperature: float, pred, conf, entropy, side=None,
                            stream=None) -> None:
    _check("dg_denoise_step_noalloc",
           _lib.dg_denoise_step_noalloc(ctypes.byref(cfg), _w(weights), _kv(kv), _ptr(canvas), inv_temperature,
                                        _ptr(pred), _ptr(conf), _ptr(entropy), _side(side), _stream(stream)))


def dg_noalloc_scratch_bytes() -> int:
    out = ctypes.c_size_t(0)
    _check("dg_noalloc_scratch_bytes", _lib.dg_noalloc_scratch_bytes(ctypes.byref(out)))
    return int(out.value)


def dg_canvas_update(cfg, pred, conf, keep_count: int, seed: int, block: int, step: int, canvas_out,
                     keep_mask=None, stream=None) -> None:
    _check("dg_canvas_update", _lib.dg_canvas_update(ctypes.byref(cfg), _ptr(pred), _ptr(conf), keep_count, seed,
                                                     block, step, _ptr(canvas_out), _ptr(keep_mask),
                                                     _stream(stream)))


def dg_commit_block(cfg, weights, kv, block_tokens, ws, ws_bytes: int, side=None, stream=None) -> None:
    _check("dg_commit_block", _lib.dg_commit_block(ctypes.byref(cfg), _w(weights), _kv(kv), _ptr(block_tokens),
                                                   _ptr(ws), ws_bytes, _side(side), _stream(stream)))


def dg_generate_block(cfg, weights, kv, sampler: dg_sampler, block: int, tokens_out, ws, ws_bytes: int,
                      side=None, stream=None) -> dg_block_status:
    st = dg_block_status()
    _check("dg_generate_block", _lib.dg_generate_block(ctypes.byref(cfg), _w(weights), _kv(kv),
                                                       ctypes.byref(sampler), block, _ptr(tokens_out),
                                                       ctypes.byref(st), _ptr(ws), ws_bytes, _side(side), _stream(stream)))
    return st


def dg_generate_block_overlapped(cfg, weights, kv, sampler: dg_sampler, block: int, pending, defer_commit: int,
                                 tokens_out, ws, ws_bytes: int, side=None, stream=None) -> dg_block_status:
    st = dg_block_status()
    _check("dg_generate_block_overlapped",
           _lib.dg_generate_block_overlapped(ctypes.byref(cfg), _w(weights), _kv(kv), ctypes.byref(sampler), block,
                                             _ptr(pending), defer_commit, _ptr(tokens_out), ctypes.byref(st),
                                             _ptr(ws), ws_bytes, _side(side), _stream(stream)))
    return st


def dg_generate_blocks(cfg, weights, kvs, sampler: dg_sampler, blocks, tokens_out, ws, ws_bytes: int,
                       side=None, stream=None) -> list:
    """Blocks of len(kvs) sequences at once; tokens_out is [n_seq, canvas]; each KV's len grows on success."""
    n = len(kvs)
    arr = (dg_kv * n)(*[kv.struct for kv in kvs])
    ids = (ctypes.c_uint32 * n)(*[int(b) for b in blocks])
    st = (dg_block_status * n)()
    rc = _lib.dg_generate_blocks(ctypes.byref(cfg), _w(weights), arr, n, ctypes.byref(sampler), ids,
                                 _ptr(tokens_out), st, _ptr(ws), ws_bytes, _side(side), _stream(stream))
    _check("dg_generate_blocks", rc)
    for kv, a in zip(kvs, arr):
        kv.len = int(a.len)
    return list(st)


def dg_generate_blocks_overlapped(cfg, weights, kvs, sampler: dg_sampler, blocks, pending, defer_commit: int,
                                  tokens_out, ws, ws_bytes: int, side=None, stream=None) -> list:
    """dg_generate_blocks with the pending blocks committed inside the first pass (see include/dg.h)."""
    n = len(kvs)
    arr = (dg_kv * n)(*[kv.struct for kv in kvs])
    ids = (ctypes.c_uint32 * n)(*[int(b) for b in blocks])
    st = (dg_block_status * n)()
    rc = _lib.dg_generate_blocks_overlapped(ctypes.byref(cfg), _w(weights), arr, n, ctypes.byref(sampler), ids,
                                            _ptr(pending), defer_commit, _ptr(tokens_out), st, _ptr(ws), ws_bytes,
                                            _side(side), _stream(stream))
    _check("dg_generate_blocks_overlapped", rc)
    for kv, a in zip(kvs, arr):
        kv.len = int(a.len)
    return list(st)


def dg_verify_block(cfg, weights, kv, draft, ar_pred, ws, ws_bytes: int, side=None, stream=None) -> tuple:
    """Self-speculative verify; returns (accepted, next_token); kv.len grows by accepted."""
    n, nxt = _i32(0), _i32(0)
    _check("dg_verify_block", _lib.dg_verify_block(ctypes.byref(cfg), _w(weights), _kv(kv), _ptr(draft),
                                                   _ptr(ar_pred), ctypes.byref(n), ctypes.byref(nxt), _ptr(ws),
                                                   ws_bytes, _side(side), _stream(stream)))
    return int(n.value), int(nxt.value)


def dg_generate_speculative(cfg, weights, kv, sampler: dg_sampler, block0: int, first_token: int, n_tokens: int,
                            tokens_out, ws, ws_bytes: int, side=None, stream=None) -> tuple:
    """Self-speculative decoding; returns (dg_spec_status, accepted count of each round); kv.len grows."""
    st = dg_spec_status()
    acc = (ctypes.c_int32 * max(n_tokens, 1))()
    _check("dg_generate_speculative",
           _lib.dg_generate_speculative(ctypes.byref(cfg), _w(weights), _kv(kv), ctypes.byref(sampler), block0,
                                        first_token, n_tokens, _ptr(tokens_out), acc, ctypes.byref(st), _ptr(ws),
                                        ws_bytes, _side(side), _stream(stream)))
    return st, [int(acc[i]) for i in range(st.rounds)]


def _dbg(dbg):
    if dbg is None:
        return None
    return ctypes.byref(dg_debug(hidden=_ptr(dbg.get("hidden")), route_idx=_ptr(dbg.get("route_idx")),
                                 route_w=_ptr(dbg.get("route_w")), router_logits=_ptr(dbg.get("router_logits"))))


def dg_layer_forward(cfg, weights, layer: int, kv, x_in, x_out, n: int, causal: int, dbg=None, ws=None,
                     ws_bytes: int = 0, side=None, stream=None) -> None:
    _check("dg_layer_forward", _lib.dg_layer_forward(ctypes.byref(cfg), _w(weights), layer, _kv(kv), _ptr(x_in),
                                                     _ptr(x_out), n, causal, _dbg(dbg), _ptr(ws), ws_bytes,
                                                     _side(side), _stream(stream)))


def dg_vocab_head(cfg, weights, x, n: int, inv_temperature: float, pred, conf, entropy, ws, ws_bytes: int,
                  stream=None) -> None:
    _check("dg_vocab_head", _lib.dg_vocab_head(ctypes.byref(cfg), _w(weights), _ptr(x), n, inv_temperature,
                                               _ptr(pred), _ptr(conf), _ptr(entropy), _ptr(ws), ws_bytes,
                                               _stream(stream)))


def dg_stop_check(cfg, sampler: dg_sampler, step: int, entropy, pred, prev_pred, d_status, canvas=None,
                  lock_mask=None, stream=None) -> None:
    _check("dg_stop_check", _lib.dg_stop_check(ctypes.byref(cfg), ctypes.byref(sampler), step, _ptr(entropy),
                                               _ptr(pred), _ptr(prev_pred), _ptr(canvas), _ptr(lock_mask),
                                               _ptr(d_status), _stream(stream)))


def dg_denoise_step_sampler(cfg, weights, kv, sampler: dg_sampler, block: int, step: int, canvas, pred, conf,
                            entropy, ws, ws_bytes: int, side=None, stream=None) -> None:
    _check("dg_denoise_step_sampler",
           _lib.dg_denoise_step_sampler(ctypes.byref(cfg), _w(weights), _kv(kv), ctypes.byref(sampler), block, step,
                                        _ptr(canvas), _ptr(pred), _ptr(conf), _ptr(entropy), _ptr(ws), ws_bytes,
                                        _side(side), _stream(stream)))


def dg_canvas_update_sampler(cfg, sampler: dg_sampler, block: int, step: int, pred, conf, entropy, canvas,
                             lock_mask=None, stream=None) -> None:
    _check("dg_canvas_update_sampler",
           _lib.dg_canvas_update_sampler(ctypes.byref(cfg), ctypes.byref(sampler), block, step, _ptr(pred),
                                         _ptr(conf), _ptr(entropy), _ptr(canvas), _ptr(lock_mask), _stream(stream)))


def dg_vocab_head_sampler(cfg, weights, sampler: dg_sampler, block: int, step: int, x, n: int, pred, conf, entropy,
                          ws, ws_bytes: int, stream=None) -> None:
    _check("dg_vocab_head_sampler",
           _lib.dg_vocab_head_sampler(ctypes.byref(cfg), _w(weights), ctypes.byref(sampler), block, step, _ptr(x), n,
                                      _ptr(pred), _ptr(conf), _ptr(entropy), _ptr(ws), ws_bytes, _stream(stream)))


def dg_sampler_inv_temperature(sampler: dg_sampler, step: int) -> float:
    out = ctypes.c_float()
    _check("dg_sampler_inv_temperature", _lib.dg_sampler_inv_temperature(ctypes.byref(sampler), step,
                                                                         ctypes.byref(out)))
    return float(out.value)


def dg_status_string(status: int) -> str:
    return _lib.dg_status_string(status).decode()


def dg_last_hip_error() -> int:
    return int(_lib.dg_last_hip_error())


def make_sampler(n_new: int, max_steps: int = 48, fixed_steps: int = 0, entropy_threshold: float = 0.05,
                 inv_temperature: float = 1.0, seed: int = 1, flags: int = 0, temperature_first: float = 0.0,
                 temperature_last: float = 0.0) -> dg_sampler:
    return dg_sampler(n_new=n_new, max_steps=max_steps, fixed_steps=fixed_steps,
                      entropy_threshold=entropy_threshold, inv_temperature=inv_temperature, flags=flags, seed=seed,
                      temperature_first=temperature_first, temperature_last=temperature_last)


def dg_timing_start(kernels: Sequence[str]) -> None:
    """Record HIP events around launches of the named kernel classes (see KERNELS)."""
    mask = 0
    for k in kernels:
        mask |= 1 << KERNELS.index(k)
    _check("dg_timing_start", _lib.dg_timing_start(mask))


def dg_timing_stop() -> Dict[str, tuple]:
    """Stop recording; {kernel: (total ms, launches)} for kernels with at least one launch."""
    n = len(KERNELS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check("dg_timing_stop", _lib.dg_timing_stop(ms, cnt))
    return {KERNELS[i]: (float(ms[i]), int(cnt[i])) for i in range(n) if cnt[i]}


def dg_packed_elems(rows: int, cols: int) -> int:
    out = ctypes.c_int64(0)
    _check("dg_packed_elems", _lib.dg_packed_elems(rows, cols, ctypes.byref(out)))
    return int(out.value)


def dg_pack_matrix(src, dst, batch: int, rows: int, cols: int, dtype: int, stream=None) -> None:
    _check("dg_pack_matrix", _lib.dg_pack_matrix(_ptr(src), _ptr(dst), batch, rows, cols, dtype, _stream(stream)))


def dg_packed_bytes_e4m3(rows: int, cols: int) -> int:
    out = ctypes.c_int64(0)
    _check("dg_packed_bytes_e4m3", _lib.dg_packed_bytes_e4m3(rows, cols, ctypes.byref(out)))
    return int(out.value)


def dg_quantize_e4m3(src, dst, scale, batch: int, rows: int, cols: int, stream=None) -> None:
    _check("dg_quantize_e4m3", _lib.dg_quantize_e4m3(_ptr(src), _ptr(dst), _ptr(scale), batch, rows, cols,
                                                     _stream(stream)))


def quantize_tensor_e4m3(t):
    """A 2-D [rows, cols] or 3-D [batch, rows, cols] row-major bf16 device tensor -> (E4M3 codes in the FP8
    pair-tiled layout, uint8 1-D; per-row float32 scales [batch * rows])."""
    import torch
    rows, cols = int(t.shape[-2]), int(t.shape[-1])
    batch = int(t.shape[0]) if t.dim() == 3 else 1
    codes = torch.empty(batch * dg_packed_bytes_e4m3(rows, cols), dtype=torch.uint8, device=t.device)
    scale = torch.empty(batch * rows, dtype=torch.float32, device=t.device)
    dg_quantize_e4m3(t.contiguous(), codes, scale, batch, rows, cols)
    return codes, scale


MATRIX_FIELDS = ("wqkv", "wo", "w_router", "w_gate_up", "w_down", "ws_gate_up", "ws_down")
EXPERT_FIELDS = ("w_gate_up", "w_down")


def pack_tensor(t):
    """A 2-D [rows, cols] or 3-D [batch, rows, cols] row-major device tensor -> its fragment-tiled copy (1-D)."""
    import torch
    rows, cols = int(t.shape[-2]), int(t.shape[-1])
    batch = int(t.shape[0]) if t.dim() == 3 else 1
    dt = DG_BF16 if t.dtype == torch.bfloat16 else DG_F32
    out = torch.empty(batch * dg_packed_elems(rows, cols), dtype=t.dtype, device=t.device)
    dg_pack_matrix(t.contiguous(), out, batch, rows, cols, dt)
    return out


def pack_layer(layer: Dict[str, object], expert_dtype: str = "") -> Dict[str, object]:
    """One layer's weights with every matrix converted to the library's layout (norm gains unchanged); with
    expert_dtype "e4m3" the routed experts' matrices are quantised (codes + "<name>_scale")."""
    out = {}
    for k, v in layer.items():
        if expert_dtype == "e4m3" and k in EXPERT_FIELDS:
            out[k], out[k + "_scale"] = quantize_tensor_e4m3(v)
        elif k in MATRIX_FIELDS:
            out[k] = pack_tensor(v)
        else:
            out[k] = v
    return out


def pack_weights(natural: dict, expert_dtype: str = "", head_dtype: str = "") -> dict:
    """{"embed", "final_norm", "layers": [...]} of row-major device tensors -> the library's layout.  With
    head_dtype "e4m3" the tied embedding is quantised (codes + "embed_scale", one scale per vocabulary row)."""
    out = {"final_norm": natural["final_norm"], "layers": [pack_layer(l, expert_dtype) for l in natural["layers"]]}
    emb = natural.get("embed")
    if emb is None:
        out["embed"] = None
    elif head_dtype == "e4m3":
        out["embed"], out["embed_scale"] = quantize_tensor_e4m3(emb)
    else:
        out["embed"] = pack_tensor(emb)
    return out
