"""Pins of the oracle's optimizer step (CPU only).

The oracle's AdamW and global-norm clipping are checked against what fixes
them independently of the oracle's own code: PyTorch's torch.optim.AdamW and
torch.nn.utils.clip_grad_norm_ run in float64 on the CPU, and closed forms
(the first step with eps = 0 moves every element by exactly lr against the
sign of its gradient; with zero gradients only the decay acts; a (3, 4)
gradient clipped to norm 1 becomes (0.6, 0.8)).
"""
import numpy as np
import pytest
import torch

import oracle as O


def _tensors(seed):
    rng = np.random.default_rng([7, seed])
    shapes = [(5, 7), (13,), (3, 4, 2)]
    decay = [True, False, True]
    ps = [rng.normal(0, 0.02, s) for s in shapes]
    gs = [[rng.normal(0, 1e-2, s) for s in shapes] for _ in range(3)]
    return shapes, decay, ps, gs


@pytest.mark.parametrize("max_norm", [0.0, 0.05, 100.0])
def test_adamw_matches_torch(max_norm):
    lr, b1, b2, eps, wd = 3e-4, 0.9, 0.95, 1e-8, 0.1
    shapes, decay, ps, gs = _tensors(1)
    tp = [torch.nn.Parameter(torch.tensor(p, dtype=torch.float64)) for p in ps]
    groups = [{"params": [t for t, d in zip(tp, decay) if d], "weight_decay": wd},
              {"params": [t for t, d in zip(tp, decay) if not d], "weight_decay": 0.0}]
    opt = torch.optim.AdamW(groups, lr=lr, betas=(b1, b2), eps=eps, foreach=False)
    p = [x.copy() for x in ps]
    m = [np.zeros(s) for s in shapes]
    v = [np.zeros(s) for s in shapes]
    for step in range(1, 4):
        g = gs[step - 1]
        for t, gi in zip(tp, g):
            t.grad = torch.tensor(gi, dtype=torch.float64)
        if max_norm > 0:
            tn = float(torch.nn.utils.clip_grad_norm_(tp, max_norm))
        opt.step()
        total, scale = O.clip_scale(g, max_norm)
        if max_norm > 0:
            assert total == pytest.approx(tn, rel=1e-12)
        for i in range(len(p)):
            p[i], m[i], v[i] = O.adamw_step(p[i], g[i], m[i], v[i], step, lr, b1, b2, eps, wd, decay[i], scale)
        for i in range(len(p)):
            # torch clips with max_norm / (norm + 1e-6): a relative difference
            # of about 1e-6 / norm in the clipped gradient, hence the tolerance
            np.testing.assert_allclose(p[i], tp[i].detach().numpy(), rtol=0, atol=1e-9)


def test_first_step_is_sign_step():
    rng = np.random.default_rng(3)
    p = rng.normal(size=50)
    g = rng.normal(size=50)
    p1, m1, v1 = O.adamw_step(p, g, np.zeros(50), np.zeros(50), 1, 0.01, 0.9, 0.99, 0.0, 0.0, True)
    np.testing.assert_allclose(p1, p - 0.01 * np.sign(g), rtol=0, atol=1e-15)
    np.testing.assert_allclose(m1, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v1, 0.01 * g * g, rtol=1e-13)


def test_zero_gradient_only_decays():
    p = np.linspace(-1, 1, 9)
    z = np.zeros(9)
    p1, m1, v1 = O.adamw_step(p, z, z, z, 4, 0.5, 0.9, 0.95, 1e-8, 0.2, True)
    np.testing.assert_array_equal(p1, p * (1 - 0.5 * 0.2))
    p2, _, _ = O.adamw_step(p, z, z, z, 4, 0.5, 0.9, 0.95, 1e-8, 0.2, False)
    np.testing.assert_array_equal(p2, p)
    assert not m1.any() and not v1.any()


def test_clip_closed_form():
    total, scale = O.clip_scale([np.array([3.0]), np.array([4.0])], 1.0)
    assert total == 5.0 and scale == 0.2
    total, scale = O.clip_scale([np.array([0.3, 0.4])], 1.0)
    assert total == pytest.approx(0.5) and scale == 1.0
    total, scale = O.clip_scale([np.zeros(4)], 1.0)
    assert total == 0.0 and scale == 1.0
