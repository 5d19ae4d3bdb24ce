"""GPU parity of the helper entry points: LM head + cross-entropy (chunked
vocabulary, ragged tails, fp32 and bf16), bits-per-byte reduction (integer
sums bit-exact), embedding forward/backward (Zipf-skewed ids, out-of-range
ids), and the row norms."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from decoder_only_gpt_bf16_amd import binding as B
from decoder_only_gpt_bf16_amd import synth
from decoder_only_gpt_bf16_amd.model import to_f64, upload, upload_i32, workspace
from tests._parity import REL_ACT, REL_LOSS, assert_rel, print_case

pytestmark = pytest.mark.gpu


def _cfg(dtype="bf16", V=1000, C=64, H=4, norm="layernorm", bias=True, rope=False):
    return synth.GPTConfig(n_layer=1, n_head=H, n_embd=C, block_size=16384, vocab_size=V, bias=bias, norm=norm,
                           rope=rope, qk_norm=rope, dtype=dtype)


XENT = [
    ("bf16", 300, 64, 1000),      # one ragged chunk
    ("bf16", 1, 64, 27),           # single token, tiny vocab
    ("bf16", 517, 768, 50304),     # 7 chunks, last one ragged
    ("bf16", 1000, 1280, 32768),   # 4 full chunks
    ("fp32", 64, 64, 27),
    ("fp32", 200, 64, 9000),       # two chunks, ragged
    # the full-size heads: the GPT-2 124M step (tied, V 50304) and the d20
    # evaluation (V 32768), N = 16384 tokens (dW and dh sum over all of them)
    pytest.param("bf16", 16384, 768, 50304, marks=pytest.mark.timeout(900)),
    pytest.param("bf16", 16384, 1280, 32768, marks=pytest.mark.timeout(900)),
]


@pytest.mark.parametrize("dtype,N,C,V", XENT)
def test_lm_head_xent(dtype, N, C, V):
    print_case("xent", dtype, N, C, V)
    rng = np.random.default_rng(N + V)
    h = synth.round_to(rng.standard_normal((N, C)), dtype)
    W = synth.round_to(0.05 * rng.standard_normal((V, C)), dtype)
    y = rng.integers(0, V, N)
    cfg = _cfg(dtype, V, C, H=C // 64 if C >= 64 else 1)
    c = B.make_config(cfg)
    ws = workspace(c, 1, N)
    dh = torch.empty((N, C), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
    dW = torch.full((V, C), 7.0, dtype=torch.float32, device="cuda")
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    nats = torch.zeros(N, dtype=torch.float32, device="cuda")
    B.lm_head_xent_fwd_bwd(c, N, upload(h, dtype), upload(W, dtype), upload_i32(y), 1.0 / N, loss, nats, dh, dW, 0,
                           ws)
    torch.cuda.synchronize()
    l_ref, n_ref, dh_ref, dW_ref = O.xent_fwd_bwd(h, W, y, 1.0 / N)
    rep = {}
    assert_rel("loss", loss.item(), l_ref, REL_LOSS, rep)
    assert_rel("nats", to_f64(nats), n_ref, REL_ACT, rep)
    assert_rel("dh", to_f64(dh), dh_ref, REL_ACT, rep)
    assert_rel("dW", to_f64(dW), dW_ref, REL_ACT, rep)
    # forward only leaves dW alone and gives the same loss
    loss2 = torch.zeros(1, dtype=torch.float32, device="cuda")
    B.lm_head_xent_fwd_bwd(c, N, upload(h, dtype), upload(W, dtype), upload_i32(y), 1.0 / N, loss2, None, None, None,
                           0, ws)
    torch.cuda.synchronize()
    assert loss2.item() == loss.item()
    print(dtype, N, C, V, {k: f"{v:.2e}" for k, v in rep.items()})


XENT_W = [
    ("bf16", 517, 768, 50304, "mask"),      # the chat fine-tuning masked mean, ragged chunks
    ("bf16", 1000, 1280, 32768, "weights"),  # general non-negative weights
    ("fp32", 200, 64, 9000, "mask"),
]


@pytest.mark.parametrize("dtype,N,C,V,kind", XENT_W)
def test_lm_head_xent_weighted(dtype, N, C, V, kind):
    print_case("xent weighted", dtype, N, C, V, kind)
    rng = np.random.default_rng(3 * N + V)
    h = synth.round_to(rng.standard_normal((N, C)), dtype)
    W = synth.round_to(0.05 * rng.standard_normal((V, C)), dtype)
    y = rng.integers(0, V, N)
    if kind == "mask":
        w = (rng.uniform(size=N) < 0.5).astype(np.float64)
        y[w == 0] = -1          # masked positions may carry an ignore id
        scale = 1.0 / w.sum()
    else:
        w = synth.round_to(rng.uniform(0.0, 2.0, N), "fp32")
        w[::7] = 0.0
        scale = 1.0 / N
    cfg = _cfg(dtype, V, C, H=C // 64 if C >= 64 else 1)
    c = B.make_config(cfg)
    ws = workspace(c, 1, N)
    dh = torch.empty((N, C), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
    dW = torch.zeros((V, C), dtype=torch.float32, device="cuda")
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    nats = torch.zeros(N, dtype=torch.float32, device="cuda")
    tw = torch.tensor(w, dtype=torch.float32, device="cuda")
    B.lm_head_xent_weighted_fwd_bwd(c, N, upload(h, dtype), upload(W, dtype), upload_i32(y), tw, scale, loss, nats,
                                    dh, dW, 0, ws)
    torch.cuda.synchronize()
    keep = w != 0
    y_ref = np.where(keep, y, 0)    # any valid id: a zero-weight row contributes nothing
    l_ref, n_ref, dh_ref, dW_ref = O.xent_fwd_bwd(h, W, y_ref, scale, weights=w)
    rep = {}
    assert_rel("loss", loss.item(), l_ref, REL_LOSS, rep)
    assert_rel("nats(kept)", to_f64(nats)[keep], n_ref[keep], REL_ACT, rep)
    assert_rel("dh", to_f64(dh), dh_ref, REL_ACT, rep)
    assert_rel("dW", to_f64(dW), dW_ref, REL_ACT, rep)
    assert not to_f64(dh)[~keep].any(), "zero-weight rows must have zero input gradients"
    print(dtype, N, C, V, kind, {k: f"{v:.2e}" for k, v in rep.items()})


def test_xent_uniform_logits_give_ln_V():
    """A zero head weight: every token's nats is ln V."""
    N, C, V = 64, 128, 32768
    cfg = _cfg("bf16", V, C)
    c = B.make_config(cfg)
    ws = workspace(c, 1, N)
    h = upload(synth.round_to(np.random.default_rng(0).standard_normal((N, C)), "bf16"), "bf16")
    W = torch.zeros((V, C), dtype=torch.bfloat16, device="cuda")
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    nats = torch.zeros(N, dtype=torch.float32, device="cuda")
    y = upload_i32(np.arange(N) * 500)
    B.lm_head_xent_fwd_bwd(c, N, h, W, y, 1.0 / N, loss, nats, None, None, 0, ws)
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_f64(nats), math.log(V), rtol=1e-6)
    tb = upload_i32(np.ones(V, dtype=np.int32))
    sn = torch.zeros(1, dtype=torch.float64, device="cuda")
    sb = torch.zeros(1, dtype=torch.int64, device="cuda")
    B.val_bpb_reduce(N, nats, y, tb, V, sn, sb)
    torch.cuda.synchronize()
    assert sb.item() == N
    assert abs(sn.item() / (math.log(2) * sb.item()) - 15.0) < 1e-5


def test_val_bpb_reduce_exact():
    rng = np.random.default_rng(5)
    N, V = 16384, 32768
    tb = rng.integers(1, 13, V)
    tb[[0, 1, 99]] = 0
    y = rng.integers(0, V, N)
    y[:50] = 99
    y[50] = V + 5      # out of range: counts as a zero-byte token
    y[51] = -3
    nats = synth.round_to(rng.random(N) * 8, "fp32")
    print_case("bpb", N, V)
    sn = torch.zeros(1, dtype=torch.float64, device="cuda")
    sb = torch.zeros(1, dtype=torch.int64, device="cuda")
    nt = torch.from_numpy(nats.astype(np.float32)).cuda()
    yt = upload_i32(y)
    tbt = upload_i32(tb)
    B.val_bpb_reduce(N, nt, yt, tbt, V, sn, sb)
    B.val_bpb_reduce(N, nt, yt, tbt, V, sn, sb)   # accumulates
    torch.cuda.synchronize()
    valid = (y >= 0) & (y < V)
    keep = valid.copy()
    keep[valid] = tb[y[valid]] > 0
    exp_b = 2 * int(tb[y[keep]].sum())
    assert sb.item() == exp_b
    s_n, s_b, _ = O.val_bpb(nats[valid], y[valid], tb)
    assert 2 * s_b == exp_b
    assert abs(sn.item() - 2 * s_n) <= 1e-9 * abs(2 * s_n)


@pytest.mark.parametrize("dtype,rope,zipf", [("bf16", False, True), ("bf16", True, True), ("fp32", False, False)])
def test_embed_fwd_bwd(dtype, rope, zipf):
    print_case("embed", dtype, rope, zipf)
    rng = np.random.default_rng(9)
    Bsz, T, C, V = 4, 300, 768, 50304
    cfg = synth.GPTConfig(n_layer=1, n_head=12, n_embd=C, block_size=512, vocab_size=V, rope=rope, dtype=dtype)
    c = B.make_config(cfg)
    ids = synth.zipf_ids(rng, (Bsz, T), 50257, 1.1) if zipf else rng.integers(0, V, (Bsz, T))
    wte = synth.round_to(0.02 * rng.standard_normal((V, C)), dtype)
    wpe = None if rope else synth.round_to(0.02 * rng.standard_normal((512, C)), dtype)
    dx0 = synth.round_to(rng.standard_normal((Bsz, T, C)), dtype)
    x0 = torch.empty((Bsz * T, C), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
    B.gpt_embed_fwd(c, Bsz, T, upload_i32(ids), upload(wte, dtype), upload(wpe, dtype), x0)
    ws = workspace(c, Bsz, T)
    dwte = torch.full((V, C), 3.0, dtype=torch.float32, device="cuda")
    dwpe = None if rope else torch.full((512, C), 3.0, dtype=torch.float32, device="cuda")
    B.gpt_embed_bwd(c, Bsz, T, upload_i32(ids), upload(dx0.reshape(-1, C), dtype), dwte, dwpe, 0, ws)
    torch.cuda.synchronize()
    x_ref = O.embed_fwd(ids, wte, wpe)
    if rope:   # a pure gather: bit-exact
        assert np.array_equal(to_f64(x0).reshape(x_ref.shape), x_ref)
    else:
        assert_rel("x0", to_f64(x0).reshape(x_ref.shape), x_ref, 1e-2)
    dwte_ref, dwpe_ref = O.embed_bwd(dx0, ids, V, 0 if rope else 512)
    assert_rel("dwte", to_f64(dwte), dwte_ref, 1e-5)
    untouched = np.setdiff1d(np.arange(V), ids.reshape(-1))
    assert not to_f64(dwte)[untouched].any()
    if not rope:
        assert_rel("dwpe", to_f64(dwpe), dwpe_ref, 1e-5)
    # deterministic; accumulate adds
    d1 = dwte.clone()
    B.gpt_embed_bwd(c, Bsz, T, upload_i32(ids), upload(dx0.reshape(-1, C), dtype), dwte, dwpe, 1, ws)
    torch.cuda.synchronize()
    torch.testing.assert_close(dwte, 2 * d1, rtol=0, atol=0)


@pytest.mark.parametrize("T", [5000, 20000])
def test_embed_bwd_multi_tile_sort(T):
    """The (id, position) sort across several 8192-key tiles: 10000 tokens
    sort as 16384 keys (one merge over global memory), 40000 as 65536 keys
    (three merges, six global stages); Zipf ids, so long runs of one id cross
    tile and chunk boundaries.  The sums must equal the oracle's, untouched
    rows stay zero, and a second call with accumulate adds the identical
    result."""
    print_case("embed-multi-tile", T)
    rng = np.random.default_rng(11)
    Bsz, C, V = 2, 64, 50304
    cfg = synth.GPTConfig(n_layer=1, n_head=2, n_embd=C, block_size=T, vocab_size=V, rope=True, dtype="bf16")
    c = B.make_config(cfg)
    ids = synth.zipf_ids(rng, (Bsz, T), 50257, 1.1)
    dx0 = synth.round_to(rng.standard_normal((Bsz, T, C)), "bf16")
    ws = workspace(c, Bsz, T)
    dwte = torch.full((V, C), 3.0, dtype=torch.float32, device="cuda")
    B.gpt_embed_bwd(c, Bsz, T, upload_i32(ids), upload(dx0.reshape(-1, C), "bf16"), dwte, None, 0, ws)
    torch.cuda.synchronize()
    ref, _ = O.embed_bwd(dx0, ids, V, 0)
    assert_rel("dwte", to_f64(dwte), ref, 1e-5)
    untouched = np.setdiff1d(np.arange(V), ids.reshape(-1))
    assert not to_f64(dwte)[untouched].any()
    d1 = dwte.clone()
    B.gpt_embed_bwd(c, Bsz, T, upload_i32(ids), upload(dx0.reshape(-1, C), "bf16"), dwte, None, 1, ws)
    torch.cuda.synchronize()
    torch.testing.assert_close(dwte, 2 * d1, rtol=0, atol=0)


def test_embed_out_of_range_ids():
    """ids outside [0, V) embed to zero and contribute no gradient."""
    Bsz, T, C, V = 1, 40, 64, 100
    cfg = synth.GPTConfig(n_layer=1, n_head=4, n_embd=C, block_size=64, vocab_size=V, rope=True)
    c = B.make_config(cfg)
    rng = np.random.default_rng(1)
    ids = rng.integers(0, V, (Bsz, T))
    ids[0, 3] = V
    ids[0, 7] = -1
    ids[0, 8] = 1 << 20
    wte = synth.round_to(rng.standard_normal((V, C)), "bf16")
    x0 = torch.empty((T, C), dtype=torch.bfloat16, device="cuda")
    B.gpt_embed_fwd(c, Bsz, T, upload_i32(ids), upload(wte, "bf16"), None, x0)
    dx0 = synth.round_to(rng.standard_normal((T, C)), "bf16")
    ws = workspace(c, Bsz, T)
    dwte = torch.zeros((V, C), dtype=torch.float32, device="cuda")
    B.gpt_embed_bwd(c, Bsz, T, upload_i32(ids), upload(dx0, "bf16"), dwte, None, 0, ws)
    torch.cuda.synchronize()
    x = to_f64(x0)
    assert not x[[3, 7, 8]].any()
    ok = (ids[0] >= 0) & (ids[0] < V)
    ref, _ = O.embed_bwd(dx0[None][:, ok], ids[:, ok], V, 0)
    assert_rel("dwte", to_f64(dwte), ref, 1e-5)


# N = 8192 gives the column-sum finish 1024 block partials per column (its
# batched loads); N = 777 only its tail loop
@pytest.mark.parametrize("norm,dtype,N", [("layernorm", "bf16", 777), ("rmsnorm", "bf16", 777),
                                          ("layernorm", "fp32", 777), ("layernorm", "bf16", 8192)])
def test_norm_fwd_bwd(norm, dtype, N):
    print_case("norm", norm, dtype, N)
    rng = np.random.default_rng(2)
    C = 1280
    cfg = _cfg(dtype, 100, C, 10, norm=norm)
    c = B.make_config(cfg)
    x = synth.round_to(2 + 3 * rng.standard_normal((N, C)), dtype)
    w = synth.round_to(1 + 0.1 * rng.standard_normal(C), dtype) if norm == "layernorm" else None
    b = synth.round_to(0.1 * rng.standard_normal(C), dtype) if norm == "layernorm" else None
    dy = synth.round_to(rng.standard_normal((N, C)), dtype)
    res = synth.round_to(rng.standard_normal((N, C)), dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    y = torch.empty((N, C), dtype=tdt, device="cuda")
    stats = torch.empty(2 * N, dtype=torch.float32, device="cuda")
    B.gpt_norm_fwd(c, N, upload(x, dtype), upload(w, dtype), upload(b, dtype), y, stats)
    dx = torch.empty_like(y)
    dw = torch.zeros(C, dtype=torch.float32, device="cuda") if w is not None else None
    db = torch.zeros(C, dtype=torch.float32, device="cuda") if b is not None else None
    Tw = min(N, cfg.block_size)  # the workspace is sized for B * T = N rows
    ws = workspace(c, N // Tw, Tw)
    B.gpt_norm_bwd(c, N, upload(x, dtype), upload(w, dtype), upload(dy, dtype), upload(res, dtype), dx, dw, db, 0, ws)
    torch.cuda.synchronize()
    if norm == "layernorm":
        y_ref, mu, rstd = O.layernorm_fwd(x, w, b, 1e-5)
        dx_ref, dw_ref, db_ref = O.layernorm_bwd(dy, x, w, 1e-5)
        assert_rel("dw", to_f64(dw), dw_ref, 1e-4)
        assert_rel("db", to_f64(db), db_ref, 1e-4)
        assert_rel("mean", to_f64(stats)[:N], mu, 1e-5)
    else:
        y_ref, rstd = O.rmsnorm_fwd(x, 1e-5)
        dx_ref = O.rmsnorm_bwd(dy, x, 1e-5)
    assert_rel("y", to_f64(y), y_ref, REL_ACT)
    assert_rel("rstd", to_f64(stats)[N:], rstd, 1e-5)
    assert_rel("dx", to_f64(dx), dx_ref + res, REL_ACT)
