"""The allocation-free AdamW entry point (gpt_adamw_step_noalloc) against the
existing gpt_adamw_step on the same inputs: two calls in a row, the second
with a smaller tensor set, so the built-in scratch carries the first call's
contents into the second.  Both entry points run the same kernels in the
same order, so every output must match bit for bit; the existing entry point
itself is checked against the oracle in test_gpu_optim.py."""
import numpy as np
import pytest
import torch

from decoder_only_gpt_bf16_amd import binding as B
from decoder_only_gpt_bf16_amd import synth
from tests._parity import print_case

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _tensors(shapes, seed, want16):
    host = synth.make_adamw_inputs(shapes, seed)
    out = []
    for j, ((p, g, m, v), w16) in enumerate(zip(host, want16)):
        t = {k: torch.tensor(np.asarray(a, dtype=np.float32), device="cuda") for k, a in
             (("param", p), ("grad", g), ("m", m), ("v", v))}
        t["param_bf16"] = torch.zeros(p.shape, dtype=torch.bfloat16, device="cuda") if w16 else None
        t["decay"] = len(p.shape) == 2
        out.append(t)
    return out


def _clone(ts):
    return [{k: (v.clone() if torch.is_tensor(v) else v) for k, v in t.items()} for t in ts]


def _same(a, b):
    for i, (x, y) in enumerate(zip(a, b)):
        for k in ("param", "m", "v", "param_bf16"):
            if x[k] is not None:
                assert torch.equal(x[k], y[k]), (i, k)


CALLS = [
    # (shapes, bf16 copies, max_norm, step): the first call fills more of the
    # scratch (11.9 M elements, 1,457 chunks) than the second reads
    ([(3840, 1280), (1280, 1280), (5120, 1280), (1280,), (777, 33), (1, 5)], [True, False, True, False, True, False],
     0.05, 1),
    ([(1280, 1280), (3001,), (64, 64)], [False, True, True], 0.01, 7),
]


def test_adamw_noalloc_matches_workspace_entry_point():
    for call, (shapes, w16, max_norm, step) in enumerate(CALLS):
        print_case("adamw-noalloc", call, shapes)
        ref = _tensors(shapes, call, w16)
        got = _clone(ref)
        ws = torch.empty(B.gpt_adamw_workspace_bytes(ref), dtype=torch.uint8, device="cuda")
        n_ref = torch.zeros(4, device="cuda")
        n_got = torch.full((4,), 7.0, device="cuda")
        B.gpt_adamw_step(ref, step=step, max_norm=max_norm, grad_norm=n_ref, ws=ws, **HP)
        B.gpt_adamw_step_noalloc(got, step=step, max_norm=max_norm, grad_norm=n_got, **HP)
        torch.cuda.synchronize()
        assert float(n_ref[0]) > max_norm          # the clip is active, so the norm partials are used
        assert torch.equal(n_ref[:1], n_got[:1])
        _same(got, ref)


def test_adamw_noalloc_refuses_more_than_its_scratch():
    """One chunk beyond the built-in scratch is refused before any launch."""
    n = B.ADAMW_NOALLOC_MAX_CHUNKS * 8192 + 1
    t = (B.AdamwTensorC * 1)()
    t[0] = B.AdamwTensorC(16, 32, 48, 64, None, n, 1)
    c = B.AdamwConfigC(1e-3, 0.9, 0.95, 1e-8, 0.1, 1, 1.0)
    import ctypes
    assert B.lib().gpt_adamw_step_noalloc(ctypes.byref(c), t, 1, None, None) == B.GPT_ERR_UNSUPPORTED
    assert b"scratch" in B.lib().gpt_last_error()
