"""dg_denoise_step_noalloc (the pass for callers that cannot allocate) against dg_denoise_step through the C ABI.

Two calls in a row, the second with a smaller canvas, each compared with the workspace form of the same pass:
predictions, confidences and entropies equal bit for bit (the same kernels run in the same order; only the
scratch memory differs).  The fixed scratch keeps the first call's contents when the second runs.
"""
from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import block_diffusion_decoding_step_amd as dg  # noqa: E402
import dg_inputs  # noqa: E402
from dg_inputs import device as gdev  # noqa: E402
from dg_inputs import recipe  # noqa: E402
from tests._gpu import Session  # noqa: E402


def _outs(S):
    return (torch.full((S,), -1, dtype=torch.int32, device="cuda"),
            torch.full((S,), float("nan"), dtype=torch.float32, device="cuda"),
            torch.full((S,), float("nan"), dtype=torch.float32, device="cuda"))


def test_noalloc_pass_equals_workspace_pass_twice():
    d = replace(recipe.C3.dims, n_layers=2)
    P = 384
    print("no-alloc: weights and prompt", flush=True)
    sess = Session(d, capacity=P + d.canvas, max_tokens=d.canvas)
    sess.prefill(dg_inputs.prompt_tokens(P, d.vocab))
    assert dg.dg_noalloc_scratch_bytes() >= dg.dg_workspace_size(sess.cfg, d.canvas)
    for S in (d.canvas, 128):   # the second call has the smaller input
        print(f"no-alloc: canvas {S}", flush=True)
        cfg = dg.make_config(replace(d, canvas=S))
        canvas = gdev.uniform_tensor(S, 5, S, d.vocab)
        ref = _outs(S)
        dg.dg_denoise_step(cfg, sess.weights, sess.kv, canvas, 1.0, *ref, None, sess.ws, sess.ws_bytes,
                           side=sess.side)
        got = _outs(S)
        dg.dg_denoise_step_noalloc(cfg, sess.weights, sess.kv, canvas, 1.0, *got, side=sess.side)
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert torch.equal(a, b), S
        p = got[0].cpu().numpy()
        assert np.all((p >= 0) & (p < d.vocab)) and bool(torch.isfinite(got[2]).all())
    assert sess.kv.len == P
