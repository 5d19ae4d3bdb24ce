"""Pin the oracle's forward with closed forms, invariants, brute force and the
numbers the pages print (tests/golden/pages_values.json)."""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import ndtr

import oracle as O
from decoder_only_gpt_bf16_amd import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))

D20 = dict(n_head=2, norm="rmsnorm", bias=False, rope=True, qk_norm=True, rope_base=10000.0, eps=1e-5)
GPT2 = dict(n_head=2, norm="layernorm", bias=True, rope=False, qk_norm=False, rope_base=10000.0, eps=1e-5)


# ---- cross-entropy and bits per byte ---------------------------------------

@pytest.mark.parametrize("V", [27, 32768, 50304])
def test_uniform_logits_give_ln_V(V):
    """A zero head weight makes every logit 0: nats = ln V exactly."""
    rng = np.random.default_rng(0)
    h = rng.standard_normal((5, 8))
    y = rng.integers(0, V, 5)
    loss, nats, _, _ = O.xent_fwd_bwd(h, np.zeros((V, 8)), y, 1.0 / 5, want_grad=False)
    np.testing.assert_allclose(nats, math.log(V), rtol=0, atol=1e-12)
    assert abs(loss - math.log(V)) < 1e-12


def test_bpb_uniform_32768_is_15_bits():
    """Uniform logits over 32768 tokens with every token one byte long: 15 bits/byte."""
    V = 32768
    y = np.arange(0, 64) * 7
    _, nats, _, _ = O.xent_fwd_bwd(np.ones((64, 4)), np.zeros((V, 4)), y, 1.0, want_grad=False)
    s_n, s_b, bpb = O.val_bpb(nats, y, np.ones(V, dtype=np.int64))
    assert s_b == 64
    assert abs(bpb - 15.0) < 1e-12


def test_bpb_bytes_one_equals_loss_over_ln2():
    rng = np.random.default_rng(1)
    nats = rng.random(100) * 5
    y = rng.integers(0, 27, 100)
    _, _, bpb = O.val_bpb(nats, y, np.ones(27, dtype=np.int64))
    assert abs(bpb - nats.mean() / math.log(2)) < 1e-12


def test_bpb_zero_byte_tokens_drop_from_both_sums():
    """Brute force over a Python loop; special tokens (0 bytes) contribute nothing."""
    rng = np.random.default_rng(2)
    V = 50
    tb = rng.integers(1, 13, V)
    tb[[0, 3, 7]] = 0
    y = rng.integers(0, V, 300)
    y[:20] = 3
    nats = rng.random(300) * 4
    sn, sb = 0.0, 0
    for n in range(300):
        if tb[y[n]] > 0:
            sn += nats[n]
            sb += int(tb[y[n]])
    s_n, s_b, bpb = O.val_bpb(nats, y, tb)
    assert s_b == sb
    assert abs(s_n - sn) < 1e-9
    assert abs(bpb - sn / (math.log(2) * sb)) < 1e-12


def test_xent_brute_force():
    """Per-row nats from a pure-Python loop with math.exp/math.log."""
    rng = np.random.default_rng(3)
    N, C, V = 6, 5, 9
    h, W = rng.standard_normal((N, C)), rng.standard_normal((V, C))
    y = rng.integers(0, V, N)
    _, nats, _, _ = O.xent_fwd_bwd(h, W, y, 1.0, want_grad=False)
    for n in range(N):
        z = [sum(h[n, c] * W[v, c] for c in range(C)) for v in range(V)]
        ref = math.log(sum(math.exp(zz) for zz in z)) - z[y[n]]
        assert abs(nats[n] - ref) < 1e-12


def test_dlogit_rows_sum_to_zero():
    """softmax - onehot sums to 0 per row: a constant column of W gets dh = 0."""
    rng = np.random.default_rng(4)
    N, C, V = 7, 6, 31
    h, W = rng.standard_normal((N, C)), rng.standard_normal((V, C))
    W[:, 2] = 0.7
    y = rng.integers(0, V, N)
    _, _, dh, _ = O.xent_fwd_bwd(h, W, y, 1.0)
    np.testing.assert_allclose(dh[:, 2], 0.0, atol=1e-14)


def test_initial_loss_just_above_ln_V():
    """At init the loss sits slightly above ln V: mean nats ~ ln V + sigma^2/2
    for small Gaussian logits.  The pages print 9.21 at step 0 for V = 8192
    (ln 8192 = 9.011)."""
    g = GOLD["step0_loss_vocab8192"]
    V = g["vocab"]
    assert math.log(V) < g["value"] < math.log(V) + 0.25
    rng = np.random.default_rng(5)
    N, C = 512, 256
    h = rng.standard_normal((N, C))
    W = 0.02 * rng.standard_normal((V, C))
    y = rng.integers(0, V, N)
    loss, _, _, _ = O.xent_fwd_bwd(h, W, y, 1.0 / N, want_grad=False)
    sig2 = (h @ W.T).var()
    assert abs(loss - (math.log(V) + sig2 / 2)) < 0.02
    assert math.log(V) < loss < g["value"]


# ---- attention --------------------------------------------------------------

def test_attention_brute_force():
    rng = np.random.default_rng(6)
    B, T, H, D = 1, 5, 2, 3
    q, k, v = (rng.standard_normal((B, T, H, D)) for _ in range(3))
    o, lse = O.causal_attention_fwd(q, k, v)
    for h in range(H):
        for i in range(T):
            s = [sum(q[0, i, h, d] * k[0, j, h, d] for d in range(D)) / math.sqrt(D) for j in range(i + 1)]
            den = sum(math.exp(x) for x in s)
            assert abs(lse[0, h, i] - math.log(den)) < 1e-12
            for d in range(D):
                ref = sum(math.exp(s[j]) / den * v[0, j, h, d] for j in range(i + 1))
                assert abs(o[0, i, h, d] - ref) < 1e-12


def test_attention_T1_is_v():
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((3, 1, 2, 8)) for _ in range(3))
    o, _ = O.causal_attention_fwd(q, k, v)
    np.testing.assert_array_equal(o, v)


def test_attention_zero_q_is_prefix_mean():
    rng = np.random.default_rng(8)
    k, v = rng.standard_normal((2, 9, 2, 4)), rng.standard_normal((2, 9, 2, 4))
    o, _ = O.causal_attention_fwd(np.zeros_like(k), k, v)
    ref = np.cumsum(v, axis=1) / np.arange(1, 10)[None, :, None, None]
    np.testing.assert_allclose(o, ref, atol=1e-14)


def test_attention_rows_sum_to_one():
    """With v = 1 everywhere, O = sum_j P_ij = 1."""
    rng = np.random.default_rng(9)
    q, k = rng.standard_normal((2, 11, 3, 4)), rng.standard_normal((2, 11, 3, 4))
    o, _ = O.causal_attention_fwd(3 * q, k, np.ones_like(q))
    np.testing.assert_allclose(o, 1.0, atol=1e-14)


@pytest.mark.parametrize("form", ["gpt2", "d20"])
def test_block_causal_invariance(form):
    """Changing rows after t leaves the block output at rows <= t unchanged."""
    cfg = GPT2 if form == "gpt2" else D20
    rng = np.random.default_rng(10)
    from tests.test_oracle_fd import _block_params
    x = rng.standard_normal((2, 12, 16))
    p = _block_params(rng, 16, cfg)
    y, _ = O.block_fwd(cfg, x, p)
    t = 6
    x2 = x.copy()
    x2[:, t + 1:] = rng.standard_normal(x2[:, t + 1:].shape) * 5
    y2, _ = O.block_fwd(cfg, x2, p)
    np.testing.assert_allclose(y2[:, : t + 1], y[:, : t + 1], atol=1e-14, rtol=0)
    assert np.abs(y2[:, t + 1:] - y[:, t + 1:]).max() > 1e-3


# ---- RoPE / QK-norm -----------------------------------------------------------

def test_rope_unit_vectors():
    """Pair i rotates by t * base^(-2i/D): e_i -> cos e_i + sin e_{i+D/2},
    e_{i+D/2} -> -sin e_i + cos e_{i+D/2}; position 0 is the identity."""
    D, T, base = 8, 6, 10000.0
    for i in range(D // 2):
        for which in (i, i + D // 2):
            x = np.zeros((1, T, 1, D))
            x[..., which] = 1.0
            y = O.rope_fwd(x, base)
            for t in range(T):
                ang = t * base ** (-2.0 * i / D)
                c, s = math.cos(ang), math.sin(ang)
                exp = np.zeros(D)
                if which == i:
                    exp[i], exp[i + D // 2] = c, s
                else:
                    exp[i], exp[i + D // 2] = -s, c
                np.testing.assert_allclose(y[0, t, 0], exp, atol=1e-15)


def test_rope_norm_and_relative_position():
    rng = np.random.default_rng(11)
    T, D = 16, 8
    q, k = rng.standard_normal((1, T, 1, D)), rng.standard_normal((1, T, 1, D))
    qr, kr = O.rope_fwd(q, 10000.0), O.rope_fwd(k, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(qr, axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-14)
    # same vectors placed at every position: the score depends only on i - j
    qc = np.broadcast_to(q[:, :1], q.shape).copy()
    kc = np.broadcast_to(k[:, :1], k.shape).copy()
    S = O.rope_fwd(qc, 10000.0)[0, :, 0] @ O.rope_fwd(kc, 10000.0)[0, :, 0].T
    for d in range(-T + 1, T):
        np.testing.assert_allclose(np.diagonal(S, d), np.diagonal(S, d)[0], atol=1e-12)


def test_rope_and_qknorm_commute():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((2, 10, 3, 16))
    a = O.rmsnorm_fwd(O.rope_fwd(x, 10000.0), 1e-5)[0]
    b = O.rope_fwd(O.rmsnorm_fwd(x, 1e-5)[0], 10000.0)
    np.testing.assert_allclose(a, b, atol=1e-14)


# ---- norms, GELU ----------------------------------------------------------------

def test_norm_invariants():
    rng = np.random.default_rng(13)
    x = 3 + 2 * rng.standard_normal((5, 64))
    y, _, _ = O.layernorm_fwd(x, None, None, 0.0)
    np.testing.assert_allclose(y.mean(-1), 0, atol=1e-13)
    np.testing.assert_allclose(y.var(-1), 1, atol=1e-12)
    r, _ = O.rmsnorm_fwd(x, 0.0)
    np.testing.assert_allclose(np.sqrt((r * r).mean(-1)), 1, atol=1e-13)
    dy = rng.standard_normal(x.shape)
    # the orthogonality relations are exact at eps = 0
    dx, _, _ = O.layernorm_bwd(dy, x, np.ones(64), 0.0)
    xhat = O.layernorm_fwd(x, None, None, 0.0)[0]
    np.testing.assert_allclose(dx.sum(-1), 0, atol=1e-12)
    np.testing.assert_allclose((dx * xhat).sum(-1), 0, atol=1e-11)
    dr = O.rmsnorm_bwd(dy, x, 0.0)
    np.testing.assert_allclose((dr * x).sum(-1), 0, atol=1e-11)


def test_layernorm_against_torch():
    rng = np.random.default_rng(14)
    x, w, b = rng.standard_normal((4, 32)), rng.standard_normal(32), rng.standard_normal(32)
    ref = torch.nn.functional.layer_norm(torch.tensor(x), (32,), torch.tensor(w), torch.tensor(b), 1e-5)
    np.testing.assert_allclose(O.layernorm_fwd(x, w, b, 1e-5)[0], ref.numpy(), atol=1e-13)


def test_gelu_values():
    assert O.gelu(np.array(0.0)) == 0.0
    assert abs(O.gelu_grad(np.array(0.0)) - 0.5) < 1e-15
    u = np.linspace(-8, 8, 161)
    np.testing.assert_allclose(O.gelu(u), u * ndtr(u), atol=1e-15)   # u * Phi(u), scipy's ndtr
    assert abs(O.gelu(np.array(1.0)) - 0.8413447460685429) < 1e-15  # Phi(1)
    assert abs(O.gelu(np.array(30.0)) - 30.0) < 1e-12
    assert abs(O.gelu(np.array(-30.0))) < 1e-12


# ---- embeddings -------------------------------------------------------------------

def test_embed_bwd_sum_and_untouched_rows():
    rng = np.random.default_rng(15)
    ids = rng.integers(0, 10, (3, 7))
    ids[ids == 4] = 5
    dx0 = rng.standard_normal((3, 7, 6))
    dwte, dwpe = O.embed_bwd(dx0, ids, 12, 9)
    np.testing.assert_allclose(dwte.sum(0), dx0.reshape(-1, 6).sum(0), atol=1e-13)
    for v in (4, 10, 11):
        assert not dwte[v].any()
    np.testing.assert_allclose(dwpe[:7], dx0.sum(0), atol=1e-14)
    assert not dwpe[7:].any()
    for v in range(10):
        ref = np.zeros(6)
        for b in range(3):
            for t in range(7):
                if ids[b, t] == v:
                    ref += dx0[b, t]
        np.testing.assert_allclose(dwte[v], ref, atol=1e-14)


# ---- shapes the pages print (pins the synthetic parameter layout) --------------------

def _count(P):
    n = 0
    for k, v in P.items():
        if k == "blocks":
            for bp in v:
                n += sum(a.size for a in bp.values() if a is not None)
        elif v is not None:
            n += v.size
    return n


def test_d20_transformer_weights_393M():
    w = synth.D20_BLOCK
    _, _, p = synth.make_block_inputs(synth.scaled(w, B=1, T=1))
    per_block = sum(a.size for a in p.values() if a is not None)
    assert per_block == 12 * 1280 * 1280
    assert round(20 * per_block / 1e6) == GOLD["d20_transformer_weights_millions"]["value"]


def test_gpt2_124M_and_tying():
    g = GOLD["padded_vocab"]
    assert g["value"] % g["multiple"] == 0 and g["value"] - g["multiple"] < g["real"] <= g["value"]
    cfg = synth.GPT2_STEP.cfg
    C, L, V, Tm = cfg.n_embd, cfg.n_layer, cfg.vocab_size, cfg.block_size
    per_block = 12 * C * C + 13 * C
    total = V * C + Tm * C + L * per_block + 2 * C
    assert round(total / 1e6) == GOLD["gpt2_small_params_millions"]["value"]
    assert int(V * C / 1e6) == GOLD["tying_saves_params_millions"]["value"]
    r = GOLD["residual_init_std_rule"]
    assert abs(r["base_std"] / math.sqrt(2 * r["n_layer"]) - r["derived_value"]) < 1e-15


def test_synth_model_param_count_tiny():
    ids, y, P, tb = synth.make_model_inputs(synth.TINY)
    assert _count(P) == 27 * 64 + 32 * 64 + (12 * 64 * 64 + 13 * 64) + 2 * 64 == 53888
    assert ids.shape == (2, 32) and (ids[:, 1:] == y[:, :-1]).all()


# ---- the input generator --------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    vals = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 3.14159, 1e-30, -7.7e5, 0.0])
    ours = synth.round_to(vals, "bf16")
    ref = torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)
    assert ours[0] == 1.0 and ours[1] == 1 + 2 ** -6
    rng = np.random.default_rng(0)
    r = rng.standard_normal(10000) * 10
    ref = torch.tensor(r, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(synth.round_to(r, "bf16"), ref)


def test_zipf_head_frequency():
    rng = np.random.default_rng(0)
    ids = synth.zipf_ids(rng, (200000,), 50257, 1.1)
    k = np.arange(1, 50258, dtype=np.float64)
    p0 = 1.0 / (k ** -1.1).sum()
    assert abs((ids == 0).mean() - p0) < 0.005
    assert ids.min() >= 0 and ids.max() < 50257


# ---- sliding-window attention --------------------------------------------------

@pytest.mark.parametrize("window", [1, 2, 4])
def test_windowed_attention_brute_force(window):
    """Query i attends to keys max(0, i - W + 1) .. i only."""
    rng = np.random.default_rng(60 + window)
    B, T, H, D = 1, 7, 2, 3
    q, k, v = (rng.standard_normal((B, T, H, D)) for _ in range(3))
    o, lse = O.causal_attention_fwd(q, k, v, window)
    for h in range(H):
        for i in range(T):
            js = range(max(0, i - window + 1), i + 1)
            s = {j: sum(q[0, i, h, d] * k[0, j, h, d] for d in range(D)) / math.sqrt(D) for j in js}
            den = sum(math.exp(x) for x in s.values())
            assert abs(lse[0, h, i] - math.log(den)) < 1e-12
            for d in range(D):
                ref = sum(math.exp(s[j]) / den * v[0, j, h, d] for j in js)
                assert abs(o[0, i, h, d] - ref) < 1e-12


def test_window_one_is_v_and_wide_window_is_causal():
    rng = np.random.default_rng(70)
    q, k, v = (rng.standard_normal((2, 10, 2, 4)) for _ in range(3))
    o1, _ = O.causal_attention_fwd(q, k, v, 1)
    np.testing.assert_allclose(o1, v, atol=1e-15)
    ofull, lfull = O.causal_attention_fwd(q, k, v)
    for w in (10, 11, 100):
        ow, lw = O.causal_attention_fwd(q, k, v, w)
        np.testing.assert_array_equal(ow, ofull)
        np.testing.assert_array_equal(lw, lfull)


def test_window_zero_q_is_trailing_mean():
    rng = np.random.default_rng(71)
    T, W = 9, 3
    k, v = rng.standard_normal((1, T, 1, 4)), rng.standard_normal((1, T, 1, 4))
    o, _ = O.causal_attention_fwd(np.zeros_like(k), k, v, W)
    for i in range(T):
        ref = v[0, max(0, i - W + 1):i + 1, 0].mean(axis=0)
        np.testing.assert_allclose(o[0, i, 0], ref, atol=1e-14)
