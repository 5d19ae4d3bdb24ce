"""Pin the oracle against PyTorch CPU float64 autograd, an independent library.

The torch model is built from library routines (F.layer_norm, F.rms_norm,
F.scaled_dot_product_attention with is_causal, F.gelu(approximate='none'),
F.cross_entropy, F.embedding) and its gradients come from autograd, so a
mistake in the oracle's hand-derived backward or in its forward cannot be
reproduced on this side.  The one hand-written torch piece is the rotary
embedding, whose forward is pinned separately by closed forms.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O



@pytest.fixture(autouse=True)
def _float64_default():
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


def _rope_torch(x, base):
    B, T, H, D = x.shape
    i = torch.arange(D // 2, dtype=torch.float64)
    theta = base ** (-2.0 * i / D)
    phi = torch.outer(torch.arange(T, dtype=torch.float64), theta)
    c, s = torch.cos(phi)[None, :, None, :], torch.sin(phi)[None, :, None, :]
    a, b = x[..., : D // 2], x[..., D // 2:]
    return torch.cat([a * c - b * s, a * s + b * c], dim=-1)


def _torch_block(cfg, x, p):
    C = x.shape[-1]
    H = cfg["n_head"]
    D = C // H
    B, T, _ = x.shape

    def norm(t, w, b):
        if cfg["norm"] == "layernorm":
            return F.layer_norm(t, (C,), w, b, cfg["eps"])
        return F.rms_norm(t, (C,), None, cfg["eps"])

    a1 = norm(x, p["ln1_w"], p["ln1_b"])
    qkv = F.linear(a1, p["w_qkv"], p["b_qkv"])
    q, k, v = qkv.split(C, dim=2)
    q, k, v = (t.reshape(B, T, H, D) for t in (q, k, v))
    if cfg["rope"]:
        q, k = _rope_torch(q, cfg["rope_base"]), _rope_torch(k, cfg["rope_base"])
    if cfg["qk_norm"]:
        q, k = F.rms_norm(q, (D,), None, cfg["eps"]), F.rms_norm(k, (D,), None, cfg["eps"])
    o = F.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), is_causal=True)
    o = o.transpose(1, 2).reshape(B, T, C)
    x1 = x + F.linear(o, p["w_o"], p["b_o"])
    a2 = norm(x1, p["ln2_w"], p["ln2_b"])
    u = F.linear(a2, p["w_fc"], p["b_fc"])
    return x1 + F.linear(F.gelu(u, approximate="none"), p["w_proj"], p["b_proj"])


def _t(a):
    return None if a is None else torch.tensor(a, requires_grad=True)


def _rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


FORMS = {
    "gpt2": dict(n_head=4, norm="layernorm", bias=True, rope=False, qk_norm=False, rope_base=10000.0, eps=1e-5),
    "d20": dict(n_head=4, norm="rmsnorm", bias=False, rope=True, qk_norm=True, rope_base=10000.0, eps=1e-5),
}


def _params(rng, C, cfg):
    ln, b = cfg["norm"] == "layernorm", cfg["bias"]
    p = {"w_qkv": 0.1 * rng.standard_normal((3 * C, C)), "w_o": 0.1 * rng.standard_normal((C, C)),
         "w_fc": 0.1 * rng.standard_normal((4 * C, C)), "w_proj": 0.1 * rng.standard_normal((C, 4 * C)),
         "ln1_w": 1 + 0.1 * rng.standard_normal(C) if ln else None,
         "ln1_b": 0.1 * rng.standard_normal(C) if ln and b else None,
         "ln2_w": 1 + 0.1 * rng.standard_normal(C) if ln else None,
         "ln2_b": 0.1 * rng.standard_normal(C) if ln and b else None}
    for k, n in (("b_qkv", 3 * C), ("b_o", C), ("b_fc", 4 * C), ("b_proj", C)):
        p[k] = 0.1 * rng.standard_normal(n) if b else None
    return p


@pytest.mark.parametrize("form", ["gpt2", "d20"])
def test_block_matches_torch_autograd(form):
    cfg = FORMS[form]
    rng = np.random.default_rng(11)
    B, T, C = 2, 24, 64
    x = rng.standard_normal((B, T, C))
    p = _params(rng, C, cfg)
    dy = rng.standard_normal(x.shape)
    y, cache = O.block_fwd(cfg, x, p)
    dx, grads = O.block_bwd(cfg, dy, cache, p)

    xt = _t(x)
    pt = {k: _t(v) for k, v in p.items()}
    yt = _torch_block(cfg, xt, pt)
    yt.backward(torch.tensor(dy))
    assert _rel(y, yt.detach().numpy()) < 1e-12
    assert _rel(dx, xt.grad.numpy()) < 1e-10
    for k, v in pt.items():
        if v is None:
            assert grads[k] is None
        else:
            assert _rel(grads[k], v.grad.numpy()) < 1e-10, k


@pytest.mark.parametrize("form", ["gpt2", "d20"])
def test_model_step_matches_torch_autograd(form):
    cfg = FORMS[form]
    rng = np.random.default_rng(12)
    B, T, C, V, L = 2, 16, 32, 29, 2
    ids = rng.integers(0, V, (B, T))
    y = rng.integers(0, V, (B, T))
    P = {"wte": 0.3 * rng.standard_normal((V, C)),
         "wpe": None if cfg["rope"] else 0.3 * rng.standard_normal((T, C)),
         "blocks": [_params(rng, C, cfg) for _ in range(L)]}
    ln = cfg["norm"] == "layernorm"
    P["lnf_w"] = 1 + 0.1 * rng.standard_normal(C) if ln else None
    P["lnf_b"] = 0.1 * rng.standard_normal(C) if ln else None
    P["lm_head"] = None if form == "gpt2" else 0.3 * rng.standard_normal((V, C))
    loss, nats, G = O.model_fwd_bwd(cfg, ids, y, P)

    wte = _t(P["wte"])
    wpe = _t(P["wpe"])
    blocks = [{k: _t(v) for k, v in bp.items()} for bp in P["blocks"]]
    lnf_w, lnf_b, head = _t(P["lnf_w"]), _t(P["lnf_b"]), _t(P["lm_head"])
    x = F.embedding(torch.tensor(ids), wte)
    if wpe is not None:
        x = x + wpe[None]
    for bp in blocks:
        x = _torch_block(cfg, x, bp)
    h = F.layer_norm(x, (C,), lnf_w, lnf_b, cfg["eps"]) if ln else F.rms_norm(x, (C,), None, cfg["eps"])
    logits = F.linear(h, head if head is not None else wte)
    lt = F.cross_entropy(logits.reshape(-1, V), torch.tensor(y).reshape(-1))
    lt.backward()
    nt = F.cross_entropy(logits.detach().reshape(-1, V), torch.tensor(y).reshape(-1), reduction="none")
    assert abs(loss - lt.item()) <= 1e-12 * abs(lt.item())
    assert _rel(nats, nt.numpy()) < 1e-12
    assert _rel(G["wte"], wte.grad.numpy()) < 1e-10
    if wpe is not None:
        assert _rel(G["wpe"], wpe.grad.numpy()) < 1e-10
    if head is not None:
        assert _rel(G["lm_head"], head.grad.numpy()) < 1e-10
    if ln:
        assert _rel(G["lnf_w"], lnf_w.grad.numpy()) < 1e-10
        assert _rel(G["lnf_b"], lnf_b.grad.numpy()) < 1e-10
    for li in range(L):
        for k, v in blocks[li].items():
            if v is not None:
                assert _rel(G["blocks"][li][k], v.grad.numpy()) < 1e-10, (li, k)


def test_masked_xent_matches_torch():
    """The masked mean of the chat fine-tuning stage: per-token losses times
    the mask, summed, divided by the mask's sum (float64 autograd)."""
    rng = np.random.default_rng(21)
    N, C, V = 40, 16, 37
    h = rng.standard_normal((N, C))
    W = 0.3 * rng.standard_normal((V, C))
    y = rng.integers(0, V, N)
    mask = (rng.uniform(size=N) < 0.6).astype(np.float64)
    th = torch.tensor(h, requires_grad=True)
    tW = torch.tensor(W, requires_grad=True)
    losses = F.cross_entropy(th @ tW.T, torch.tensor(y), reduction="none")
    tm = torch.tensor(mask)
    loss_t = (losses * tm).sum() / tm.sum()
    loss_t.backward()
    loss, nats, dh, dW = O.xent_fwd_bwd(h, W, y, 1.0 / mask.sum(), weights=mask)
    assert loss == pytest.approx(loss_t.item(), rel=1e-12)
    np.testing.assert_allclose(nats, losses.detach().numpy(), rtol=1e-12)
    np.testing.assert_allclose(dh, th.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(dW, tW.grad.numpy(), rtol=1e-10, atol=1e-14)
    # all-ones weights give the unweighted loss exactly
    l1, _, dh1, _ = O.xent_fwd_bwd(h, W, y, 1.0 / N, weights=np.ones(N))
    l0, _, dh0, _ = O.xent_fwd_bwd(h, W, y, 1.0 / N)
    assert l1 == pytest.approx(l0, rel=1e-15)
    np.testing.assert_array_equal(dh1, dh0)


@pytest.mark.parametrize("form", ["gpt2", "d20"])
def test_model_eval_nats_matches_torch(form):
    """model_eval_nats, the forward-only pass of the bits-per-byte
    evaluation, is its own code path (no caches, its own head choice and
    final norm).  It must equal the training step's nats bit for bit, and
    torch's per-token cross-entropy of a model built from library ops, for
    the tied head (GPT-2 form) and the untied one (d20 form)."""
    cfg = FORMS[form]
    rng = np.random.default_rng(13)
    B, T, C, V, L = 2, 12, 32, 31, 2
    ids = rng.integers(0, V, (B, T))
    y = rng.integers(0, V, (B, T))
    ln = cfg["norm"] == "layernorm"
    P = {"wte": 0.3 * rng.standard_normal((V, C)),
         "wpe": None if cfg["rope"] else 0.3 * rng.standard_normal((T, C)),
         "blocks": [_params(rng, C, cfg) for _ in range(L)],
         "lnf_w": 1 + 0.1 * rng.standard_normal(C) if ln else None,
         "lnf_b": 0.1 * rng.standard_normal(C) if ln else None,
         "lm_head": None if form == "gpt2" else 0.3 * rng.standard_normal((V, C))}
    nats = O.model_eval_nats(cfg, ids, y, P)
    _, nats_step, _ = O.model_fwd_bwd(cfg, ids, y, P, want_grad=False)
    np.testing.assert_array_equal(nats, nats_step)
    with torch.no_grad():
        x = F.embedding(torch.tensor(ids), torch.tensor(P["wte"]))
        if P["wpe"] is not None:
            x = x + torch.tensor(P["wpe"])[None]
        for bp in P["blocks"]:
            x = _torch_block(cfg, x, {k: None if v is None else torch.tensor(v) for k, v in bp.items()})
        if ln:
            h = F.layer_norm(x, (C,), torch.tensor(P["lnf_w"]), torch.tensor(P["lnf_b"]), cfg["eps"])
        else:
            h = F.rms_norm(x, (C,), None, cfg["eps"])
        head = torch.tensor(P["lm_head"] if P["lm_head"] is not None else P["wte"])
        nt = F.cross_entropy(F.linear(h, head).reshape(-1, V), torch.tensor(y).reshape(-1), reduction="none")
    assert _rel(nats, nt.numpy()) < 1e-12
    # the head choice matters: the other weight gives different nats
    if P["lm_head"] is not None:
        P2 = dict(P, lm_head=None)
        assert _rel(O.model_eval_nats(cfg, ids, y, P2), nt.numpy()) > 1e-3
