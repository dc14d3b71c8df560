"""The C ABI without a GPU: libdg.so loads, exports every call include/dg.h declares, and rejects bad
arguments with the documented status before touching the device (no compute call is made here)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess
import sys
from dataclasses import replace

import pytest

import block_diffusion_decoding_step_amd as dg
from dg_inputs import recipe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_documented_calls():
    names = _declared()
    for n in ("dg_prefill_kv", "dg_denoise_step", "dg_canvas_update", "dg_commit_block", "dg_generate_block",
              "dg_generate_block_overlapped", "dg_denoise_step_sampler", "dg_canvas_update_sampler",
              "dg_vocab_head_sampler", "dg_sampler_inv_temperature", "dg_generate_blocks", "dg_verify_block",
              "dg_generate_blocks_overlapped",
              "dg_workspace_size", "dg_status_string"):
        assert n in names
    assert set(names) == set(dg.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(dg.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", dg.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (dg_\w+)", out))
    assert set(_declared()) <= exported


def test_header_compiles_as_c():
    src = '#include "dg.h"\nint main(void){dg_config c; (void)c; return dg_status_string(0) == 0;}\n'
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-I", os.path.dirname(HEADER),
                        "-x", "c", "-"], input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_struct_layouts_match_header():
    src = ('#include <stdio.h>\n#include <stddef.h>\n#include "dg.h"\n'
           'int main(void){printf("%zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(dg_config), sizeof(dg_layer_weights),'
           ' sizeof(dg_weights), sizeof(dg_kv), sizeof(dg_sampler), offsetof(dg_sampler, seed),'
           ' sizeof(dg_block_status), sizeof(dg_debug)); printf("%zu\\n", sizeof(dg_side)); return 0;}\n')
    exe = "/tmp/dg_layout_probe"
    r = subprocess.run(["gcc", "-I", os.path.dirname(HEADER), "-x", "c", "-", "-o", exe], input=src,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    got = [int(x) for x in subprocess.run([exe], capture_output=True, text=True).stdout.split()]
    exp = [ctypes.sizeof(dg.dg_config), ctypes.sizeof(dg.dg_layer_weights), ctypes.sizeof(dg.dg_weights),
           ctypes.sizeof(dg.dg_kv), ctypes.sizeof(dg.dg_sampler), dg.dg_sampler.seed.offset,
           ctypes.sizeof(dg.dg_block_status), ctypes.sizeof(dg.dg_debug), ctypes.sizeof(dg.dg_side)]
    assert got == exp


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert dg.dg_status_string(s) and dg.dg_status_string(s) != "unknown status"
    assert dg.dg_status_string(-99) == "unknown status"


def _cfg(**kw):
    return dg.make_config(replace(recipe.C0.dims, **kw))


@pytest.mark.parametrize("kw,status", [
    (dict(d_model=0), dg.DG_ERR_INVALID),
    (dict(top_k=9), dg.DG_ERR_INVALID),
    (dict(n_heads=3), dg.DG_ERR_INVALID),
    (dict(head_dim=96), dg.DG_ERR_UNSUPPORTED),
    (dict(d_model=250), dg.DG_ERR_UNSUPPORTED),
    (dict(ffn_expert=500), dg.DG_ERR_UNSUPPORTED),
    (dict(n_heads=16, n_kv_heads=2), dg.DG_ERR_UNSUPPORTED),
    (dict(canvas=2048), dg.DG_ERR_UNSUPPORTED),
    (dict(n_experts=300, top_k=2), dg.DG_ERR_UNSUPPORTED),
])
def test_workspace_size_rejects_bad_config(kw, status):
    with pytest.raises(dg.DGError) as e:
        dg.dg_workspace_size(_cfg(**kw), 32)
    assert e.value.status == status


def test_rope_is_unsupported():
    c = _cfg()
    c.rope_theta = 10000.0
    with pytest.raises(dg.DGError) as e:
        dg.dg_workspace_size(c, 32)
    assert e.value.status == dg.DG_ERR_UNSUPPORTED


def test_workspace_size_grows_with_rows():
    c = dg.make_config(recipe.C3.dims)
    a = dg.dg_workspace_size(c, 256)
    b = dg.dg_workspace_size(c, 2048)
    assert 0 < a < b
    with pytest.raises(dg.DGError):
        dg.dg_workspace_size(c, 0)
    with pytest.raises(dg.DGError):
        dg.dg_workspace_size(c, 4096)   # above the permutation's row limit for 128 experts


class _Fake:
    """Aligned fake device addresses: validation runs on the host and never dereferences them."""

    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def _fake_weights(n_layers):
    a = _Fake(0x10000)
    return dg.Weights(a, a, [{f: a for f in dg.Weights.LAYER_FIELDS} for _ in range(n_layers)])


def test_calls_validate_before_any_device_work():
    cfg = _cfg()
    w = _fake_weights(cfg.n_layers)
    buf = _Fake(0x20000)
    ws_bytes = dg.dg_workspace_size(cfg, cfg.canvas)
    kv = dg.KV(buf, buf, capacity=96, length=80)  # 80 + 32 > 96
    with pytest.raises(dg.DGError) as e:
        dg.dg_denoise_step(cfg, w, kv, buf, 1.0, buf, buf, buf, None, buf, ws_bytes, stream=0)
    assert e.value.status == dg.DG_ERR_KV_FULL
    kv = dg.KV(buf, buf, capacity=100, length=0)  # capacity not a multiple of 32
    with pytest.raises(dg.DGError) as e:
        dg.dg_denoise_step(cfg, w, kv, buf, 1.0, buf, buf, buf, None, buf, ws_bytes, stream=0)
    assert e.value.status == dg.DG_ERR_INVALID
    kv = dg.KV(buf, buf, capacity=128, length=0)
    with pytest.raises(dg.DGError) as e:
        dg.dg_denoise_step(cfg, w, kv, buf, 1.0, buf, buf, buf, None, buf, ws_bytes - 256, stream=0)
    assert e.value.status == dg.DG_ERR_WORKSPACE
    with pytest.raises(dg.DGError) as e:
        dg.dg_denoise_step(cfg, w, kv, None, 1.0, buf, buf, buf, None, buf, ws_bytes, stream=0)
    assert e.value.status == dg.DG_ERR_INVALID
    with pytest.raises(dg.DGError) as e:
        dg.dg_denoise_step(cfg, w, kv, buf, 0.0, buf, buf, buf, None, buf, ws_bytes, stream=0)
    assert e.value.status == dg.DG_ERR_INVALID
    with pytest.raises(dg.DGError) as e:   # misaligned weight pointer
        dg.dg_denoise_step(cfg, _fake_weights_misaligned(cfg.n_layers), kv, buf, 1.0, buf, buf, buf, None, buf,
                           ws_bytes, stream=0)
    assert e.value.status == dg.DG_ERR_INVALID
    with pytest.raises(dg.DGError) as e:
        dg.dg_prefill_kv(cfg, w, kv, buf, 200, buf, ws_bytes, stream=0)
    assert e.value.status == dg.DG_ERR_KV_FULL
    with pytest.raises(dg.DGError) as e:
        dg.dg_layer_forward(cfg, w, 5, kv, buf, buf, 32, 0, None, buf, ws_bytes, stream=0)
    assert e.value.status == dg.DG_ERR_INVALID
    with pytest.raises(dg.DGError) as e:
        dg.dg_layer_forward(cfg, w, 0, kv, buf, buf, 32, 2, None, buf, ws_bytes, stream=0)
    assert e.value.status == dg.DG_ERR_INVALID
    bad = dg.make_sampler(4)
    bad.max_steps = 0
    with pytest.raises(dg.DGError) as e:
        dg.dg_generate_block(cfg, w, kv, bad, 0, buf, buf, ws_bytes, stream=0)
    assert e.value.status == dg.DG_ERR_INVALID
    with pytest.raises(dg.DGError) as e:
        dg.dg_generate_block_overlapped(cfg, w, kv, dg.make_sampler(4), 0, None, 2, buf, buf, ws_bytes, stream=0)
    assert e.value.status == dg.DG_ERR_INVALID
    kv_short = dg.KV(buf, buf, capacity=64, length=16)  # 16 + 2 * 32 > 64: a pending block needs two canvases
    with pytest.raises(dg.DGError) as e:
        dg.dg_generate_block_overlapped(cfg, w, kv_short, dg.make_sampler(4), 0, buf, 1, buf, buf, ws_bytes, stream=0)
    assert e.value.status == dg.DG_ERR_KV_FULL
    with pytest.raises(dg.DGError) as e:  # the workspace holds one canvas of rows, a pending block needs two
        dg.dg_generate_block_overlapped(cfg, w, kv, dg.make_sampler(4), 0, buf, 1, buf, buf, ws_bytes, stream=0)
    assert e.value.status == dg.DG_ERR_WORKSPACE
    with pytest.raises(dg.DGError) as e:
        dg.dg_stop_check(cfg, dg.make_sampler(4), 0, buf, buf, buf, buf, stream=0)
    assert e.value.status == dg.DG_ERR_INVALID
    with pytest.raises(dg.DGError) as e:
        dg.dg_canvas_update(cfg, buf, buf, cfg.canvas + 1, 1, 0, 1, buf, None, 0)
    assert e.value.status == dg.DG_ERR_INVALID
    with pytest.raises(dg.DGError) as e:
        dg.dg_vocab_head(cfg, w, buf, 0, 1.0, buf, buf, buf, buf, ws_bytes, 0)
    assert e.value.status == dg.DG_ERR_INVALID
    # the failed commit left the committed length alone
    assert kv.len == 0


def _fake_weights_misaligned(n_layers):
    a = _Fake(0x10000)
    layers = [{f: a for f in dg.Weights.LAYER_FIELDS} for _ in range(n_layers)]
    layers[-1]["w_down"] = _Fake(0x10008)
    return dg.Weights(a, a, layers)


def test_packed_elems():
    assert dg.dg_packed_elems(16, 32) == 512
    assert dg.dg_packed_elems(8, 256) == 16 * 256
    assert dg.dg_packed_elems(262144, 2816) == 262144 * 2816
    for rows, cols in ((0, 32), (16, 30), (16, 0)):
        with pytest.raises(dg.DGError):
            dg.dg_packed_elems(rows, cols)


def test_pack_rejects_overlap_and_bad_dtype():
    a = _Fake(0x100000)
    with pytest.raises(dg.DGError):
        dg.dg_pack_matrix(a, _Fake(0x100000 + 64), 1, 16, 32, dg.DG_BF16, 0)
    with pytest.raises(dg.DGError):
        dg.dg_pack_matrix(a, _Fake(0x900000), 1, 16, 32, 7, 0)


# ----------------------------------------------------------------------------- sampler variants

def test_sampler_flag_values_match_header():
    text = open(HEADER).read()
    for name in ("DG_SAMPLE_GUMBEL", "DG_SAMPLE_ANNEAL", "DG_KEEP_ENTROPY", "DG_KEEP_LOCK", "DG_STOP_AND"):
        m = re.search(r"#define %s (0x[0-9A-Fa-f]+)u" % name, text)
        assert m and int(m.group(1), 16) == getattr(dg, name), name
    assert "DG_STOP_SETTLED = 5" in text and dg.DG_STOP_SETTLED == 5


def test_anneal_schedule_equals_oracle():
    """The host schedule of the passes' temperatures against the oracle's (fp32 rounding of 1/T)."""
    from oracle import sampler as osm
    for fixed, cap in ((0, 48), (10, 48), (1, 48), (0, 1)):
        sp = dg.make_sampler(26, max_steps=cap, fixed_steps=fixed, flags=dg.DG_SAMPLE_ANNEAL, temperature_first=0.8,
                             temperature_last=0.4)
        ref = osm.Sampler(n_new=26, max_steps=cap, fixed_steps=fixed, anneal=(float(ctypes.c_float(0.8).value),
                                                                              float(ctypes.c_float(0.4).value)))
        for t in range(1, (fixed or cap) + 1):
            got = dg.dg_sampler_inv_temperature(sp, t)
            assert got == float(ctypes.c_float(osm.pass_inv_temperature(ref, t)).value), (fixed, cap, t)
    sp = dg.make_sampler(4, inv_temperature=2.5)
    assert dg.dg_sampler_inv_temperature(sp, 7) == 2.5


def test_sampler_variants_validate():
    cfg = _cfg()
    w = _fake_weights(cfg.n_layers)
    buf = _Fake(0x20000)
    ws_bytes = dg.dg_workspace_size(cfg, cfg.canvas)
    kv = dg.KV(buf, buf, capacity=128, length=0)
    bad = [dg.make_sampler(4, flags=0x20),                                                # unknown bit
           dg.make_sampler(4, flags=dg.DG_SAMPLE_ANNEAL, temperature_first=0.8),            # last = 0
           dg.make_sampler(4, flags=dg.DG_SAMPLE_ANNEAL, temperature_first=float("inf"), temperature_last=0.4),
           dg.make_sampler(4, inv_temperature=0.0),
           dg.make_sampler(4, max_steps=70000, flags=dg.DG_SAMPLE_GUMBEL)]                 # pass beyond 16 bits
    for sp in bad:
        with pytest.raises(dg.DGError) as e:
            dg.dg_sampler_inv_temperature(sp, 1)
        assert e.value.status == dg.DG_ERR_INVALID
        with pytest.raises(dg.DGError) as e:
            dg.dg_generate_block(cfg, w, kv, sp, 0, buf, buf, ws_bytes, stream=0)
        assert e.value.status == dg.DG_ERR_INVALID
    ok = dg.make_sampler(4, flags=dg.DG_SAMPLE_ANNEAL | dg.DG_SAMPLE_GUMBEL, inv_temperature=0.0,
                         temperature_first=0.8, temperature_last=0.4)
    assert abs(dg.dg_sampler_inv_temperature(ok, 1) - 1.25) < 1e-6   # inv_temperature is ignored under anneal
    lock = dg.make_sampler(4, flags=dg.DG_KEEP_LOCK)
    cases = [
        lambda: dg.dg_stop_check(cfg, lock, 1, buf, buf, buf, buf, None, buf, 0),            # lock without canvas
        lambda: dg.dg_stop_check(cfg, lock, 1, buf, buf, buf, buf, buf, None, 0),            # lock without mask
        lambda: dg.dg_canvas_update_sampler(cfg, lock, 0, 2, buf, buf, buf, buf, None, 0),   # lock without mask
        lambda: dg.dg_canvas_update_sampler(cfg, dg.make_sampler(4), 0, -1, buf, buf, buf, buf, None, 0),
        lambda: dg.dg_canvas_update_sampler(cfg, dg.make_sampler(4, flags=dg.DG_KEEP_ENTROPY), 0, 2, buf, buf, None,
                                            buf, None, 0),                                 # entropy ranking, no entropy
        lambda: dg.dg_canvas_update_sampler(cfg, dg.make_sampler(4), 0, 1, buf, buf, buf, None, None, 0),
        lambda: dg.dg_denoise_step_sampler(cfg, w, kv, dg.make_sampler(4), 0, 0, buf, buf, buf, buf, buf, ws_bytes,
                                           stream=0),                                             # passes count from 1
        lambda: dg.dg_vocab_head_sampler(cfg, w, dg.make_sampler(4), 0, 70000, buf, 4, buf, buf, buf, buf, ws_bytes,
                                         0),
    ]
    for i, c in enumerate(cases):
        with pytest.raises(dg.DGError) as e:
            c()
        assert e.value.status == dg.DG_ERR_INVALID, i


def test_generate_blocks_validate():
    cfg = _cfg()
    w = _fake_weights(cfg.n_layers)
    buf = _Fake(0x20000)
    ws1 = dg.dg_workspace_size(cfg, cfg.canvas)
    ws3 = dg.dg_workspace_size(cfg, 3 * cfg.canvas)
    sp = dg.make_sampler(4)
    kvs = [dg.KV(_Fake(0x100000 * (i + 1)), _Fake(0x100000 * (i + 1) + 0x80000), capacity=128, length=0)
           for i in range(9)]
    cases = [
        (lambda: dg.dg_generate_blocks(cfg, w, [], sp, [], buf, buf, ws1, stream=0), dg.DG_ERR_INVALID),        # no sequence
        (lambda: dg.dg_generate_blocks(cfg, w, kvs, sp, list(range(9)), buf, buf, ws3, stream=0), dg.DG_ERR_INVALID),  # > 8
        (lambda: dg.dg_generate_blocks(cfg, w, [kvs[0], kvs[0]], sp, [0, 1], buf, buf, ws3, stream=0), dg.DG_ERR_INVALID),
        (lambda: dg.dg_generate_blocks(cfg, w, kvs[:3], sp, [0, 1, 2], buf, buf, ws1, stream=0), dg.DG_ERR_WORKSPACE),
        (lambda: dg.dg_generate_blocks(cfg, w, kvs[:2] + [dg.KV(buf, buf, capacity=96, length=80)], sp, [0, 1, 2],
                                       buf, buf, ws3, stream=0), dg.DG_ERR_KV_FULL),
    ]
    for i, (c, status) in enumerate(cases):
        with pytest.raises(dg.DGError) as e:
            c()
        assert e.value.status == status, i
    assert [kv.len for kv in kvs] == [0] * 9
    with pytest.raises(dg.DGError) as e:
        dg.dg_generate_blocks_overlapped(cfg, w, kvs[:2], sp, [0, 1], None, 2, buf, buf, ws3, stream=0)
    assert e.value.status == dg.DG_ERR_INVALID
    with pytest.raises(dg.DGError) as e:  # a pending block doubles the rows of the first pass
        dg.dg_generate_blocks_overlapped(cfg, w, kvs[:3], sp, [0, 1, 2], buf, 1, buf, buf, ws3, stream=0)
    assert e.value.status == dg.DG_ERR_WORKSPACE


def test_overlapped_pending_rows_within_routing_limit():
    """A pending block doubles the first pass's rows; with 256 experts and a 1024-slot canvas that is 2048 rows,
    beyond the 1024 one routing step orders for 256 experts: rejected before any device work, however large the
    workspace."""
    cfg = _cfg(n_experts=256, top_k=8, canvas=1024)
    w = _fake_weights(cfg.n_layers)
    buf = _Fake(0x20000)
    kv = dg.KV(buf, buf, capacity=4096, length=0)
    with pytest.raises(dg.DGError) as e:
        dg.dg_generate_block_overlapped(cfg, w, kv, dg.make_sampler(4), 0, buf, 1, buf, buf, 1 << 40, stream=0)
    assert e.value.status == dg.DG_ERR_INVALID
    assert kv.len == 0


def test_side_validates():
    """A dg_side with a stream needs two distinct events; an all-NULL side (or none) is accepted and means the
    shared expert runs on the caller's stream."""
    cfg = _cfg()
    w = _fake_weights(cfg.n_layers)
    buf = _Fake(0x20000)
    ws_bytes = dg.dg_workspace_size(cfg, cfg.canvas)
    kv = dg.KV(buf, buf, capacity=96, length=80)  # 80 + 32 > 96: a valid side gets as far as the cache check
    for bad in (dg.dg_side(0x1000, None, 0x3000), dg.dg_side(0x1000, 0x2000, None), dg.dg_side(0x1000, 0x2000, 0x2000)):
        with pytest.raises(dg.DGError) as e:
            dg.dg_denoise_step(cfg, w, kv, buf, 1.0, buf, buf, buf, None, buf, ws_bytes, bad, stream=0)
        assert e.value.status == dg.DG_ERR_INVALID
    for ok in (None, dg.dg_side(None, None, None), dg.dg_side(0x1000, 0x2000, 0x3000)):
        with pytest.raises(dg.DGError) as e:
            dg.dg_denoise_step(cfg, w, kv, buf, 1.0, buf, buf, buf, None, buf, ws_bytes, ok, stream=0)
        assert e.value.status == dg.DG_ERR_KV_FULL


def test_side_create_and_destroy_validate():
    lib = ctypes.CDLL(dg.LIB_PATH)
    lib.dg_side_create.argtypes = [ctypes.c_void_p]
    lib.dg_side_destroy.argtypes = [ctypes.c_void_p]
    assert lib.dg_side_create(None) == dg.DG_ERR_INVALID
    assert lib.dg_side_destroy(None) == dg.DG_ERR_INVALID
    empty = dg.dg_side(None, None, None)   # nothing to destroy: a no-op
    assert lib.dg_side_destroy(ctypes.byref(empty)) == dg.DG_OK


def test_verify_block_validates():
    cfg = _cfg()
    w = _fake_weights(cfg.n_layers)
    buf = _Fake(0x20000)
    ws_bytes = dg.dg_workspace_size(cfg, cfg.canvas)
    kv = dg.KV(buf, buf, capacity=96, length=80)   # 80 + 32 > 96
    with pytest.raises(dg.DGError) as e:
        dg.dg_verify_block(cfg, w, kv, buf, buf, buf, ws_bytes, stream=0)
    assert e.value.status == dg.DG_ERR_KV_FULL
    kv = dg.KV(buf, buf, capacity=128, length=0)
    with pytest.raises(dg.DGError) as e:
        dg.dg_verify_block(cfg, w, kv, None, buf, buf, ws_bytes, stream=0)
    assert e.value.status == dg.DG_ERR_INVALID
    with pytest.raises(dg.DGError) as e:
        dg.dg_verify_block(cfg, w, kv, buf, buf, buf, ws_bytes - 256, stream=0)
    assert e.value.status == dg.DG_ERR_WORKSPACE
    assert kv.len == 0


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one MI355X" in r.stderr and r.stdout == ""


def test_noalloc_rejects_configs_beyond_its_scratch():
    """dg_denoise_step_noalloc runs in a fixed array of dg_noalloc_scratch_bytes() (64 MiB): a configuration whose
    pass needs more (a 1024-slot canvas at the full widths) is refused with DG_ERR_WORKSPACE before any device
    work; the full-width 256-slot pass fits."""
    assert dg.dg_noalloc_scratch_bytes() == 64 << 20
    assert dg.dg_workspace_size(dg.make_config(recipe.C3.dims), recipe.C3.dims.canvas) <= 64 << 20
    cfg = dg.make_config(replace(recipe.C3.dims, canvas=1024))
    assert dg.dg_workspace_size(cfg, 1024) > 64 << 20
    w = _fake_weights(cfg.n_layers)
    buf = _Fake(0x20000)
    kv = dg.KV(buf, buf, capacity=4096, length=0)
    with pytest.raises(dg.DGError) as e:
        dg.dg_denoise_step_noalloc(cfg, w, kv, buf, 1.0, buf, buf, buf, stream=0)
    assert e.value.status == dg.DG_ERR_WORKSPACE
    with pytest.raises(dg.DGError) as e:   # the usual argument checks come first
        dg.dg_denoise_step_noalloc(dg.make_config(recipe.C3.dims), w, kv, None, 1.0, buf, buf, buf, stream=0)
    assert e.value.status == dg.DG_ERR_INVALID


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("dg_bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_bench_accounting_host_side():
    """bench.py's algorithmic byte counts and its lookup of the committed traffic summaries, for both expert
    precisions: FP8 experts count one byte per weight plus the per-channel float scales; a traffic summary is
    used only for the gate/up kernel it names and only while the kernel sources it was taken on are unchanged."""
    b = _bench_module()
    d16, d8 = recipe.C3.dims, recipe.C3_FP8.dims
    assert b.expert_weight_bytes(d16) == 2.0 and b.expert_weight_bytes(d8) == 1.0
    hit, pairs = 120.0, d16.canvas * d16.top_k
    w16 = hit * 2 * d16.ffn_expert * d16.d_model * 2
    w8 = hit * 2 * d8.ffn_expert * d8.d_model * 1 + hit * 2 * d8.ffn_expert * 4
    acts = b.gate_up_bytes(d16, hit, pairs) - w16
    assert acts > 0
    assert b.gate_up_bytes(d8, hit, pairs) == pytest.approx(w8 + acts)
    for d, kname in ((d16, "k_moe_gate_up"), (d8, "k_moe_gate_up_f8")):
        t = b.read_traffic(d, kname)   # None or a plausible byte count, never an exception
        assert t is None or 0.5 * b.gate_up_bytes(d, hit, pairs) < t < 4 * b.gate_up_bytes(d, hit, pairs)
        assert b.read_traffic(d, "k_other") is None


@pytest.mark.parametrize("kw,status", [
    (dict(head_dtype="e4m3"), dg.DG_ERR_UNSUPPORTED),                          # an fp32 model
    (dict(dtype="bf16", head_dtype="e4m3", d_model=96), dg.DG_ERR_UNSUPPORTED),  # rows not whole 64-column blocks
])
def test_fp8_head_config_limits(kw, status):
    with pytest.raises(dg.DGError) as e:
        dg.dg_workspace_size(_cfg(**kw), 32)
    assert e.value.status == status
    c = _cfg(dtype="bf16")
    c.head_dtype = 5   # neither 0, the model's dtype nor DG_E4M3
    with pytest.raises(dg.DGError) as e:
        dg.dg_workspace_size(c, 32)
    assert e.value.status == dg.DG_ERR_INVALID


def test_fp8_head_needs_row_scales():
    """With head_dtype DG_E4M3 the tied embedding's row scales are part of the weights: a call without them is
    refused before any device work; with them (and otherwise the same arguments) the weights pass validation."""
    cfg = _cfg(dtype="bf16", head_dtype="e4m3")
    assert dg.dg_workspace_size(cfg, cfg.canvas) > 0
    w = _fake_weights(cfg.n_layers)
    buf = _Fake(0x20000)
    kv = dg.KV(buf, buf, capacity=cfg.canvas + 64, length=0)
    ws_bytes = dg.dg_workspace_size(cfg, cfg.canvas)
    with pytest.raises(dg.DGError) as e:
        dg.dg_denoise_step(cfg, w, kv, buf, 1.0, buf, buf, buf, None, buf, ws_bytes, stream=0)
    assert e.value.status == dg.DG_ERR_INVALID
    a = _Fake(0x10000)
    w = dg.Weights(a, a, [{f: a for f in dg.Weights.LAYER_FIELDS} for _ in range(cfg.n_layers)], embed_scale=a)
    with pytest.raises(dg.DGError) as e:   # still refused, now for the workspace only
        dg.dg_denoise_step(cfg, w, kv, buf, 1.0, buf, buf, buf, None, buf, ws_bytes - 256, stream=0)
    assert e.value.status == dg.DG_ERR_WORKSPACE
