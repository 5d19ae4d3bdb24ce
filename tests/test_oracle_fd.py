"""Pin every backward formula of the oracle with central finite differences.

For a scalar L = <f(theta), R> with a fixed random cotangent R, the
directional derivative along a random direction v is estimated as
(L(theta + eps v) - L(theta - eps v)) / (2 eps) and compared with <grad, v>
from the oracle's hand-written backward.  float64, eps = 1e-6, rel <= 1e-6.
A dropped term, wrong sign or transposed operand in any backward formula
moves the directional derivative far outside this bound.
"""
import numpy as np
import pytest

import oracle as O

EPS = 1e-6
TOL = 1e-6


def _dirderiv(f, x, v):
    return (f(x + EPS * v) - f(x - EPS * v)) / (2 * EPS)


def _check(f, x, grad, rng, n_dirs=3):
    for _ in range(n_dirs):
        v = rng.standard_normal(x.shape)
        fd = _dirderiv(f, x, v)
        an = float((grad * v).sum())
        assert abs(fd - an) <= TOL * max(1.0, abs(fd)), (fd, an)


def test_layernorm_bwd_fd():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 5, 16))
    w = 1 + 0.3 * rng.standard_normal(16)
    b = 0.3 * rng.standard_normal(16)
    R = rng.standard_normal(x.shape)
    dx, dw, db = O.layernorm_bwd(R, x, w, 1e-5)
    _check(lambda t: (O.layernorm_fwd(t, w, b, 1e-5)[0] * R).sum(), x, dx, rng)
    _check(lambda t: (O.layernorm_fwd(x, t, b, 1e-5)[0] * R).sum(), w, dw, rng)
    _check(lambda t: (O.layernorm_fwd(x, w, t, 1e-5)[0] * R).sum(), b, db, rng)


def test_rmsnorm_bwd_fd():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 7, 24))
    R = rng.standard_normal(x.shape)
    dx = O.rmsnorm_bwd(R, x, 1e-5)
    _check(lambda t: (O.rmsnorm_fwd(t, 1e-5)[0] * R).sum(), x, dx, rng)


def test_gelu_grad_fd():
    u = np.linspace(-6, 6, 121)
    fd = (O.gelu(u + EPS) - O.gelu(u - EPS)) / (2 * EPS)
    np.testing.assert_allclose(O.gelu_grad(u), fd, rtol=1e-7, atol=1e-9)


def test_rope_bwd_fd():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 9, 3, 8))
    R = rng.standard_normal(x.shape)
    _check(lambda t: (O.rope_fwd(t, 10000.0) * R).sum(), x, O.rope_bwd(R, 10000.0), rng)


def test_attention_bwd_fd():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((2, 7, 2, 8)) for _ in range(3))
    R = rng.standard_normal(q.shape)
    dq, dk, dv = O.causal_attention_bwd(R, q, k, v)
    _check(lambda t: (O.causal_attention_fwd(t, k, v)[0] * R).sum(), q, dq, rng)
    _check(lambda t: (O.causal_attention_fwd(q, t, v)[0] * R).sum(), k, dk, rng)
    _check(lambda t: (O.causal_attention_fwd(q, k, t)[0] * R).sum(), v, dv, rng)


def _cfg(form):
    if form == "gpt2":
        return dict(n_head=2, norm="layernorm", bias=True, rope=False, qk_norm=False,
                    rope_base=10000.0, eps=1e-5)
    return dict(n_head=2, norm="rmsnorm", bias=False, rope=True, qk_norm=True,
                rope_base=10000.0, eps=1e-5)


def _block_params(rng, C, cfg):
    p = {"w_qkv": 0.3 * rng.standard_normal((3 * C, C)), "w_o": 0.3 * rng.standard_normal((C, C)),
         "w_fc": 0.3 * rng.standard_normal((4 * C, C)), "w_proj": 0.3 * rng.standard_normal((C, 4 * C))}
    ln = cfg["norm"] == "layernorm"
    b = cfg["bias"]
    p["ln1_w"] = 1 + 0.2 * rng.standard_normal(C) if ln else None
    p["ln1_b"] = 0.2 * rng.standard_normal(C) if ln and b else None
    p["ln2_w"] = 1 + 0.2 * rng.standard_normal(C) if ln else None
    p["ln2_b"] = 0.2 * rng.standard_normal(C) if ln and b else None
    for k, n in (("b_qkv", 3 * C), ("b_o", C), ("b_fc", 4 * C), ("b_proj", C)):
        p[k] = 0.2 * rng.standard_normal(n) if b else None
    return p


@pytest.mark.parametrize("form", ["gpt2", "d20"])
def test_block_bwd_fd(form):
    rng = np.random.default_rng(5)
    cfg = _cfg(form)
    B, T, C = 2, 6, 16
    x = rng.standard_normal((B, T, C))
    p = _block_params(rng, C, cfg)
    R = rng.standard_normal(x.shape)
    _, cache = O.block_fwd(cfg, x, p)
    dx, grads = O.block_bwd(cfg, R, cache, p)

    _check(lambda t: (O.block_fwd(cfg, t, p)[0] * R).sum(), x, dx, rng)
    for name, val in p.items():
        if val is None:
            assert grads[name] is None
            continue

        def f(t, name=name):
            q = dict(p)
            q[name] = t
            return (O.block_fwd(cfg, x, q)[0] * R).sum()
        _check(f, val, grads[name], rng, n_dirs=2)


def test_xent_fd():
    rng = np.random.default_rng(6)
    N, C, V = 11, 8, 13
    h = rng.standard_normal((N, C))
    W = rng.standard_normal((V, C))
    y = rng.integers(0, V, N)
    _, _, dh, dW = O.xent_fwd_bwd(h, W, y, 1.0 / N, row_chunk=4)
    _check(lambda t: O.xent_fwd_bwd(t, W, y, 1.0 / N, want_grad=False)[0], h, dh, rng)
    _check(lambda t: O.xent_fwd_bwd(h, t, y, 1.0 / N, want_grad=False)[0], W, dW, rng)


def test_embed_bwd_fd():
    rng = np.random.default_rng(7)
    B, T, C, V = 3, 5, 4, 6
    ids = rng.integers(0, V, (B, T))
    wte = rng.standard_normal((V, C))
    wpe = rng.standard_normal((8, C))
    R = rng.standard_normal((B, T, C))
    dwte, dwpe = O.embed_bwd(R, ids, V, 8)
    _check(lambda t: (O.embed_fwd(ids, t, wpe) * R).sum(), wte, dwte, rng)
    _check(lambda t: (O.embed_fwd(ids, wte, t) * R).sum(), wpe, dwpe, rng)


@pytest.mark.parametrize("form", ["gpt2", "d20"])
def test_model_fwd_bwd_fd(form):
    """Whole step, two layers, tied (gpt2 form) and untied (d20 form) heads."""
    rng = np.random.default_rng(8)
    cfg = _cfg(form)
    B, T, C, V, L = 2, 5, 16, 11, 2
    ids = rng.integers(0, V, (B, T))
    y = rng.integers(0, V, (B, T))
    P = {"wte": 0.5 * rng.standard_normal((V, C)),
         "wpe": None if cfg["rope"] else 0.5 * rng.standard_normal((T + 2, C)),
         "blocks": [_block_params(rng, C, cfg) for _ in range(L)]}
    if cfg["norm"] == "layernorm":
        P["lnf_w"], P["lnf_b"] = 1 + 0.2 * rng.standard_normal(C), 0.2 * rng.standard_normal(C)
    else:
        P["lnf_w"], P["lnf_b"] = None, None
    P["lm_head"] = None if form == "gpt2" else 0.5 * rng.standard_normal((V, C))
    loss, nats, G = O.model_fwd_bwd(cfg, ids, y, P)

    def L_of(key, t, li=None, name=None):
        Q = dict(P)
        if li is None:
            Q[key] = t
        else:
            Q["blocks"] = [dict(bp) for bp in P["blocks"]]
            Q["blocks"][li][name] = t
        return O.model_fwd_bwd(cfg, ids, y, Q, want_grad=False)[0]

    for key in ("wte", "wpe", "lnf_w", "lnf_b", "lm_head"):
        if P.get(key) is None:
            continue
        _check(lambda t, key=key: L_of(key, t), P[key], G[key], rng, n_dirs=2)
    for li in range(L):
        for name, val in P["blocks"][li].items():
            if val is None:
                continue
            _check(lambda t, li=li, name=name: L_of(None, t, li, name), val, G["blocks"][li][name], rng, n_dirs=1)


def test_xent_weighted_fd():
    rng = np.random.default_rng(16)
    N, C, V = 9, 6, 11
    h = rng.standard_normal((N, C))
    W = rng.standard_normal((V, C))
    y = rng.integers(0, V, N)
    w = rng.uniform(0.0, 2.0, N)
    w[3] = 0.0
    _, _, dh, dW = O.xent_fwd_bwd(h, W, y, 0.37, row_chunk=4, weights=w)
    _check(lambda t: O.xent_fwd_bwd(t, W, y, 0.37, want_grad=False, weights=w)[0], h, dh, rng)
    _check(lambda t: O.xent_fwd_bwd(h, t, y, 0.37, want_grad=False, weights=w)[0], W, dW, rng)
    assert not dh[3].any()


@pytest.mark.parametrize("window", [1, 3])
def test_windowed_attention_bwd_fd(window):
    rng = np.random.default_rng(40 + window)
    q, k, v = (rng.standard_normal((2, 9, 2, 8)) for _ in range(3))
    R = rng.standard_normal(q.shape)
    dq, dk, dv = O.causal_attention_bwd(R, q, k, v, window)
    _check(lambda t: (O.causal_attention_fwd(t, k, v, window)[0] * R).sum(), q, dq, rng)
    _check(lambda t: (O.causal_attention_fwd(q, t, v, window)[0] * R).sum(), k, dk, rng)
    _check(lambda t: (O.causal_attention_fwd(q, k, t, window)[0] * R).sum(), v, dv, rng)
