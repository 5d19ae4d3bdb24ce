"""GPU parity of the optimizer step (gpt_adamw_step) against the oracle.

Tolerance REL_OPT, derived from the arithmetic: every updated quantity takes
a handful of fp32 roundings (2^-24 relative each) on the way, so m and v
carry relative errors of about 1e-7; the update of a parameter carries the
same relative error plus the rounding of the stored fp32 parameter, at most
2^-24 |p| / |update|, about 1e-6 for |p| ~ 0.02 and lr = 1e-3.  Errors are
measured on the change of each parameter, on m and on v, as
||gpu - oracle|| / ||oracle|| per tensor.
"""
import numpy as np
import pytest
import torch

import oracle as O
from decoder_only_gpt_bf16_amd import binding as B
from decoder_only_gpt_bf16_amd import synth
from tests._parity import assert_rel, print_case

pytestmark = pytest.mark.gpu

REL_OPT = 1e-5
HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _upload(a):
    return torch.tensor(np.asarray(a, dtype=np.float32), device="cuda")


def _run(shapes, decay, want16, max_norm, steps, seed=0):
    host = synth.make_adamw_inputs(shapes, seed)
    dev = []
    for (p, g, m, v), w16 in zip(host, want16):
        d = {"param": _upload(p), "grad": _upload(g), "m": _upload(m), "v": _upload(v)}
        d["param_bf16"] = torch.empty(p.shape, dtype=torch.bfloat16, device="cuda") if w16 else None
        dev.append(d)
    for d, dec in zip(dev, decay):
        d["decay"] = dec
    ws = torch.empty(B.gpt_adamw_workspace_bytes(dev), dtype=torch.uint8, device="cuda")
    norm = torch.zeros(4, dtype=torch.float32, device="cuda")
    norms = []
    for step in range(1, steps + 1):
        B.gpt_adamw_step(dev, step=step, max_norm=max_norm, grad_norm=norm, ws=ws, **HP)
        torch.cuda.synchronize()
        norms.append(float(norm[0]))
    return host, dev, norms


def _oracle(host, decay, max_norm, steps):
    st = [(p.copy(), m.copy(), v.copy()) for p, g, m, v in host]
    grads = [g for _, g, _, _ in host]
    norms = []
    for step in range(1, steps + 1):
        total, scale = O.clip_scale(grads, max_norm)
        norms.append(total)
        st = [O.adamw_step(p, g, m, v, step, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"],
                           dec, scale) for (p, m, v), g, dec in zip(st, grads, decay)]
    return st, norms


def _compare(host, dev, ref, norms, ref_norms):
    for i, ((p0, _, _, _), d, (p, m, v)) in enumerate(zip(host, dev, ref)):
        pg = d["param"].double().cpu().numpy()
        assert_rel(f"dp[{i}]", pg - p0, p - p0, REL_OPT)
        assert_rel(f"m[{i}]", d["m"].double().cpu().numpy(), m, REL_OPT)
        assert_rel(f"v[{i}]", d["v"].double().cpu().numpy(), v, REL_OPT)
        if d["param_bf16"] is not None:
            assert torch.equal(d["param_bf16"], d["param"].to(torch.bfloat16)), f"bf16 copy of tensor {i}"
    for a, b in zip(norms, ref_norms):
        assert a == pytest.approx(b, rel=1e-6)


MIXED = ([(8192 * 3 + 5,), (13,), (1024, 12), (3, 4096)], [1, 0, 1, 0], [True, False, True, False])


@pytest.mark.parametrize("max_norm", [0.0, 1e9, 0.05])
def test_adamw_mixed(max_norm):
    shapes, decay, want16 = MIXED
    print_case("adamw mixed", max_norm)
    host, dev, norms = _run(shapes, decay, want16, max_norm, steps=3)
    ref, ref_norms = _oracle(host, decay, max_norm, steps=3)
    _compare(host, dev, ref, norms, ref_norms)


def test_adamw_many_tensors():
    # more tensors than one launch takes, odd sizes (scalar tails)
    shapes = [(7 + 3 * i,) if i % 3 else (64, 5 + i) for i in range(45)]
    decay = [i % 2 for i in range(45)]
    print_case("adamw 45 tensors")
    host, dev, norms = _run(shapes, decay, [i % 4 == 0 for i in range(45)], 0.02, steps=2, seed=1)
    ref, ref_norms = _oracle(host, decay, 0.02, steps=2)
    _compare(host, dev, ref, norms, ref_norms)


@pytest.mark.parametrize("name", ["d20_block", "gpt2_block"])
def test_adamw_block_parameter_set(name):
    cfg = synth.BY_NAME[name].cfg
    shp = synth.block_param_shapes(cfg)
    shapes = [s for _, s in shp]
    decay = [len(s) == 2 for s in shapes]
    print_case("adamw block set", name)
    host, dev, norms = _run(shapes, decay, [True] * len(shapes), 1.0, steps=1, seed=2)
    ref, ref_norms = _oracle(host, decay, 1.0, steps=1)
    assert ref_norms[0] > 1.0  # the clip is active at this size
    _compare(host, dev, ref, norms, ref_norms)


def test_adamw_norm_many_partials():
    # 70 M elements: 8545 partials of the squared norm, enough for the norm
    # kernel's batched loads (32 x 256 of them at a time) to run
    shapes = [(70_000_000,)]
    print_case("adamw 70M")
    host, dev, norms = _run(shapes, [1], [False], 1.0, steps=1, seed=3)
    ref, ref_norms = _oracle(host, [1], 1.0, steps=1)
    _compare(host, dev, ref, norms, ref_norms)


def test_adamw_reproducible():
    shapes, decay, want16 = MIXED
    print_case("adamw twice")
    _, dev1, n1 = _run(shapes, decay, want16, 0.05, steps=2)
    _, dev2, n2 = _run(shapes, decay, want16, 0.05, steps=2)
    assert n1 == n2
    for a, b in zip(dev1, dev2):
        for k in ("param", "m", "v"):
            assert torch.equal(a[k], b[k])
