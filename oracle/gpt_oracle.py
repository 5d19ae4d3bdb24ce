"""Plain float64 NumPy definition of one GPT training step (test oracle).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

Conventions (readings of the pages where they are silent are listed in the
design notes of the repository and repeated here next to each step):
  * activations are [B, T, C] float64; a row is one token;
  * Linear weights use the [out, in] layout of nn.Linear, y = x W^T + b
    ("nanoGPT — Karpathy's minimal GPT pretraining repo", model.py section,
    MLP and CausalSelfAttention paragraphs);
  * the fused QKV weight is [3C, C] with row blocks q | k | v; head h owns
    rows [h*D, (h+1)*D) of each block (same page, CausalSelfAttention: one
    Linear, split by n_embd, each reshaped to (B, n_head, T, head_dim)).

Nothing here is blocked, fused or reordered: attention forms the full T x T
score matrix per (batch, head), the LM head forms full logit rows.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "layernorm_fwd", "layernorm_bwd", "rmsnorm_fwd", "rmsnorm_bwd",
    "gelu", "gelu_grad", "rope_angles", "rope_fwd", "rope_bwd",
    "linear_fwd", "linear_bwd", "causal_attention_fwd", "causal_attention_bwd",
    "block_fwd", "block_bwd", "embed_fwd", "embed_bwd",
    "xent_fwd_bwd", "val_bpb", "model_fwd_bwd", "model_eval_nats",
    "norm_fwd", "norm_bwd", "clip_scale", "adamw_step",
    "FP8_FORMATS", "fp8_round", "fp8_encode", "fp8_quantize", "fp8_gemm",
    "bf16_round", "fp8_linear_fwd", "fp8_linear_bwd",
]


# ----------------------------------------------------------------------------
# Normalisation.
# nanoGPT page, model.py section: pre-LayerNorm blocks; LayerNorm has a gain
# and an optional bias.  The parameter-free RMSNorm of the nanochat form is
# the plain definition x / sqrt(mean(x^2) + eps).  Readings: eps = 1e-5 and
# the biased (divide-by-C) variance.
# ----------------------------------------------------------------------------

def layernorm_fwd(x, w, b, eps):
    """LayerNorm over the last axis.  Returns (y, mean, rstd)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mu) * rstd
    y = xhat * w if w is not None else xhat.copy()
    if b is not None:
        y = y + b
    return y, mu[..., 0], rstd[..., 0]


def layernorm_bwd(dy, x, w, eps):
    """Gradient of LayerNorm: returns (dx, dw, db).

    With xhat = (x - mu) * rstd and g = dy * w:
      dx = rstd * (g - mean(g) - xhat * mean(g * xhat)),
      dw = sum over rows of dy * xhat, db = sum over rows of dy.
    """
    C = x.shape[-1]
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mu) * rstd
    g = dy * w if w is not None else dy
    mg = g.sum(axis=-1, keepdims=True) / C
    mgx = (g * xhat).sum(axis=-1, keepdims=True) / C
    dx = rstd * (g - mg - xhat * mgx)
    rows = dy.reshape(-1, C)
    dw = (rows * xhat.reshape(-1, C)).sum(axis=0)
    db = rows.sum(axis=0)
    return dx, dw, db


def rmsnorm_fwd(x, eps):
    """Parameter-free RMSNorm over the last axis.  Returns (y, rstd)."""
    ms = (x * x).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(ms + eps)
    return x * rstd, rstd[..., 0]


def rmsnorm_bwd(dy, x, eps):
    """Gradient of parameter-free RMSNorm.

    y = x * r with r = (mean(x^2) + eps)^(-1/2) gives
    dx = r * (dy - y * mean(dy * y)).
    """
    C = x.shape[-1]
    ms = (x * x).mean(axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(ms + eps)
    y = x * r
    return r * (dy - y * ((dy * y).sum(axis=-1, keepdims=True) / C))


def norm_fwd(cfg, x, w, b):
    """The configuration's norm: LayerNorm (gain, optional bias) or RMSNorm."""
    if cfg["norm"] == "layernorm":
        y, _, _ = layernorm_fwd(x, w, b, cfg["eps"])
        return y
    y, _ = rmsnorm_fwd(x, cfg["eps"])
    return y


def norm_bwd(cfg, dy, x, w):
    """Returns (dx, dw, db); dw and db are None for the parameter-free RMSNorm."""
    if cfg["norm"] == "layernorm":
        dx, dw, db = layernorm_bwd(dy, x, w, cfg["eps"])
        return dx, dw, (db if cfg["bias"] else None)
    return rmsnorm_bwd(dy, x, cfg["eps"]), None, None


# ----------------------------------------------------------------------------
# GELU, exact erf form (reading: nanoGPT's MLP uses GELU; the tanh
# approximation is not used).
# ----------------------------------------------------------------------------

def gelu(u):
    return 0.5 * u * (1.0 + _erf(u / math.sqrt(2.0)))


def gelu_grad(u):
    """d/du of u * Phi(u) = Phi(u) + u * phi(u)."""
    cdf = 0.5 * (1.0 + _erf(u / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)
    return cdf + u * pdf


# ----------------------------------------------------------------------------
# Rotary position embedding (nanochat-d20 model card, Architecture row:
# "RoPE").  Reading: half-split pairs (i, i + D/2) for i < D/2, rotated by the
# angle t * theta_i with theta_i = base^(-2i/D), positions t = 0..T-1.
# ----------------------------------------------------------------------------

def rope_angles(T, D, base):
    i = np.arange(D // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / D)
    t = np.arange(T, dtype=np.float64)
    return np.outer(t, theta)  # [T, D/2]


def _rotate(x, phi):
    """x: [B, T, H, D]; phi: [T, D/2]; rotate each pair by +phi."""
    h = x.shape[-1] // 2
    c = np.cos(phi)[None, :, None, :]
    s = np.sin(phi)[None, :, None, :]
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def rope_fwd(x, base):
    T, D = x.shape[1], x.shape[-1]
    return _rotate(x, rope_angles(T, D, base))


def rope_bwd(dy, base):
    """A rotation is orthogonal: its adjoint is the rotation by -phi."""
    T, D = dy.shape[1], dy.shape[-1]
    return _rotate(dy, -rope_angles(T, D, base))


# ----------------------------------------------------------------------------
# Linear layers.
# ----------------------------------------------------------------------------

def linear_fwd(x, w, b):
    y = x @ w.T
    if b is not None:
        y = y + b
    return y


def linear_bwd(dy, x, w, has_bias):
    """dx = dy W, dW = dy^T x, db = column sums of dy."""
    K = x.shape[-1]
    O = dy.shape[-1]
    dy2 = dy.reshape(-1, O)
    x2 = x.reshape(-1, K)
    dx = (dy2 @ w).reshape(x.shape)
    dw = dy2.T @ x2
    db = dy2.sum(axis=0) if has_bias else None
    return dx, dw, db


_linear_fwd, _linear_bwd = linear_fwd, linear_bwd


def bf16_round(x):
    """Nearest bfloat16 value (8 significant bits, ties to even) of each
    element, through float32 (itself rounded to nearest even)."""
    bits = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    keep = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return keep.astype(np.uint32).view(np.float32).astype(np.float64)


# FP8 Linear layers ("Train your own ChatGPT", 6.2, FP8 paragraph: per-tensor
# dynamic scales, E4M3 for activations and weights, E5M2 for gradients, and
# both backward matmuls in FP8 as well).  Reading: the quantized operand of
# an activation or gradient is the bf16 value its storage holds (activations
# and activation gradients are bf16 tensors), then quantized by
# fp8_quantize; the bias and its gradient stay in full precision.

def _q(x, fmt):
    return fp8_quantize(bf16_round(x), fmt)


def fp8_linear_fwd(x, w, b):
    """y = x W^T + b with x and W quantized to E4M3, each with its own scale."""
    K = x.shape[-1]
    qx, sx, _ = _q(x.reshape(-1, K), "e4m3")
    qw, sw, _ = _q(w, "e4m3")
    y = fp8_gemm(qx, sx, qw, sw).reshape(x.shape[:-1] + (w.shape[0],))
    if b is not None:
        y = y + b
    return y


def fp8_linear_bwd(dy, x, w, has_bias):
    """dx = q(dy) q(W) and dW = q(dy)^T q(x), dy in E5M2, W and x in E4M3
    (the same codes as the forward's); db = column sums of dy."""
    K = x.shape[-1]
    O = dy.shape[-1]
    dy2 = dy.reshape(-1, O)
    qg, sg, _ = _q(dy2, "e5m2")
    qw, sw, _ = _q(w, "e4m3")
    qx, sx, _ = _q(x.reshape(-1, K), "e4m3")
    dx = fp8_gemm(qg, sg, qw.T, sw).reshape(x.shape)
    dw = fp8_gemm(qg.T, sg, qx.T, sx)
    db = dy2.sum(axis=0) if has_bias else None
    return dx, dw, db


# ----------------------------------------------------------------------------
# Causal self-attention (nanoGPT page, CausalSelfAttention paragraph: the
# explicit lower-triangular mask blocks attention to future positions).
# Reading: scores scaled by 1/sqrt(D) in every configuration.
# ----------------------------------------------------------------------------

def _hidden(T, window):
    """Mask of the key positions j a query i does not see: the future j > i,
    and with a sliding window of W > 0 positions also j <= i - W ("Train your
    own ChatGPT", 6.2: per-layer (left, right) windows of the "SSSL" pattern;
    the window lengths are a parameter here, since the pages give none)."""
    hidden = np.triu(np.ones((T, T), dtype=bool), k=1)
    if window and window > 0:
        hidden |= np.tril(np.ones((T, T), dtype=bool), k=-window)
    return hidden


def causal_attention_fwd(q, k, v, window=0):
    """q, k, v: [B, T, H, D].  Returns (O [B,T,H,D], lse [B,H,T]).

    For each (b, h): S = q k^T / sqrt(D), S_ij = -inf for j > i (and for
    j <= i - window when window > 0), P = row softmax of S, O = P v.  lse is
    the row log-sum-exp of S.
    """
    B, T, H, D = q.shape
    scale = 1.0 / math.sqrt(D)
    out = np.empty_like(q)
    lse = np.empty((B, H, T))
    future = _hidden(T, window)
    for b in range(B):
        for h in range(H):
            S = (q[b, :, h, :] @ k[b, :, h, :].T) * scale
            S[future] = -np.inf
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            s = E.sum(axis=1, keepdims=True)
            P = E / s
            out[b, :, h, :] = P @ v[b, :, h, :]
            lse[b, h, :] = (m + np.log(s))[:, 0]
    return out, lse


def causal_attention_bwd(dO, q, k, v, window=0):
    """Gradients of causal_attention_fwd's O with respect to q, k, v.

    With P the masked softmax: dV = P^T dO, dP = dO v^T,
    dS_i = P_i * (dP_i - <P_i, dP_i>) (softmax Jacobian, row by row),
    dq = dS k / sqrt(D), dk = dS^T q / sqrt(D).
    """
    B, T, H, D = q.shape
    scale = 1.0 / math.sqrt(D)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    future = _hidden(T, window)
    for b in range(B):
        for h in range(H):
            qb, kb, vb, dob = q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], dO[b, :, h, :]
            S = (qb @ kb.T) * scale
            S[future] = -np.inf
            E = np.exp(S - S.max(axis=1, keepdims=True))
            P = E / E.sum(axis=1, keepdims=True)
            dv[b, :, h, :] = P.T @ dob
            dP = dob @ vb.T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dq[b, :, h, :] = (dS @ kb) * scale
            dk[b, :, h, :] = (dS.T @ qb) * scale
    return dq, dk, dv


# ----------------------------------------------------------------------------
# One transformer block (nanoGPT page, Block paragraph: pre-norm residual,
# x = x + attn(ln_1(x)); x = x + mlp(ln_2(x))).  The nanochat form swaps the
# norm for parameter-free RMSNorm, drops the biases and applies RoPE then
# QK-norm (a per-head parameter-free RMSNorm over head_dim) to q and k.
# ----------------------------------------------------------------------------

def _heads(x, H):
    B, T, C = x.shape
    return x.reshape(B, T, H, C // H)


def block_fwd(cfg, x, p):
    """x: [B, T, C]; p: dict of block parameters (None where absent).
    cfg["fp8"] true: the four Linear layers run in FP8 (fp8_linear_fwd).

    Returns (y, cache) where cache holds what block_bwd needs.
    """
    H = cfg["n_head"]
    C = x.shape[-1]
    bias = cfg["bias"]
    linear_fwd = fp8_linear_fwd if cfg.get("fp8") else _linear_fwd
    a1 = norm_fwd(cfg, x, p.get("ln1_w"), p.get("ln1_b"))
    qkv = linear_fwd(a1, p["w_qkv"], p.get("b_qkv") if bias else None)
    q, k, v = _heads(qkv[..., :C], H), _heads(qkv[..., C:2 * C], H), _heads(qkv[..., 2 * C:], H)
    q_r, k_r = q, k
    if cfg["rope"]:
        q_r, k_r = rope_fwd(q, cfg["rope_base"]), rope_fwd(k, cfg["rope_base"])
    q_n, k_n = q_r, k_r
    if cfg["qk_norm"]:
        q_n, _ = rmsnorm_fwd(q_r, cfg["eps"])
        k_n, _ = rmsnorm_fwd(k_r, cfg["eps"])
    o, lse = causal_attention_fwd(q_n, k_n, v, cfg.get("window", 0))
    o = o.reshape(x.shape)
    x1 = x + linear_fwd(o, p["w_o"], p.get("b_o") if bias else None)
    a2 = norm_fwd(cfg, x1, p.get("ln2_w"), p.get("ln2_b"))
    u = linear_fwd(a2, p["w_fc"], p.get("b_fc") if bias else None)
    g = gelu(u)
    y = x1 + linear_fwd(g, p["w_proj"], p.get("b_proj") if bias else None)
    cache = dict(x=x, a1=a1, q_r=q_r, k_r=k_r, q_n=q_n, k_n=k_n, v=v, o=o,
                 lse=lse, x1=x1, a2=a2, u=u, g=g)
    return y, cache


def block_bwd(cfg, dy, cache, p):
    """Backward of block_fwd (FP8 Linear backward with cfg["fp8"]).
    Returns (dx, grads dict with the same keys as p)."""
    H = cfg["n_head"]
    bias = cfg["bias"]
    linear_bwd = fp8_linear_bwd if cfg.get("fp8") else _linear_bwd
    x, x1 = cache["x"], cache["x1"]
    grads = {}
    # MLP: y = x1 + gelu(a2 W_fc^T + b_fc) W_proj^T + b_proj
    dg, grads["w_proj"], grads["b_proj"] = linear_bwd(dy, cache["g"], p["w_proj"], bias)
    du = dg * gelu_grad(cache["u"])
    da2, grads["w_fc"], grads["b_fc"] = linear_bwd(du, cache["a2"], p["w_fc"], bias)
    dn2, grads["ln2_w"], grads["ln2_b"] = norm_bwd(cfg, da2, x1, p.get("ln2_w"))
    dx1 = dy + dn2
    # attention: x1 = x + attn(a1) W_o^T + b_o
    do, grads["w_o"], grads["b_o"] = linear_bwd(dx1, cache["o"], p["w_o"], bias)
    dq_n, dk_n, dv = causal_attention_bwd(_heads(do, H), cache["q_n"], cache["k_n"], cache["v"],
                                          cfg.get("window", 0))
    dq_r, dk_r = dq_n, dk_n
    if cfg["qk_norm"]:
        dq_r = rmsnorm_bwd(dq_n, cache["q_r"], cfg["eps"])
        dk_r = rmsnorm_bwd(dk_n, cache["k_r"], cfg["eps"])
    dq, dk = dq_r, dk_r
    if cfg["rope"]:
        dq, dk = rope_bwd(dq_r, cfg["rope_base"]), rope_bwd(dk_r, cfg["rope_base"])
    B, T, C = x.shape
    dqkv = np.concatenate([dq.reshape(B, T, C), dk.reshape(B, T, C), dv.reshape(B, T, C)], axis=-1)
    da1, grads["w_qkv"], grads["b_qkv"] = linear_bwd(dqkv, cache["a1"], p["w_qkv"], bias)
    dn1, grads["ln1_w"], grads["ln1_b"] = norm_bwd(cfg, da1, x, p.get("ln1_w"))
    dx = dx1 + dn1
    return dx, grads


# ----------------------------------------------------------------------------
# Embeddings (nanoGPT page, model.py: token embedding wte plus learned
# absolute positions wpe; the nanochat form uses RoPE and no wpe).
# ----------------------------------------------------------------------------

def embed_fwd(ids, wte, wpe):
    x = wte[ids]
    if wpe is not None:
        x = x + wpe[None, : ids.shape[1], :]
    return x


def embed_bwd(dx0, ids, V, wpe_rows):
    """dwte[v] = sum of dx0 rows whose id is v; dwpe[t] = sum over the batch."""
    C = dx0.shape[-1]
    dwte = np.zeros((V, C))
    np.add.at(dwte, ids.reshape(-1), dx0.reshape(-1, C))
    dwpe = None
    if wpe_rows:
        dwpe = np.zeros((wpe_rows, C))
        dwpe[: dx0.shape[1]] = dx0.sum(axis=0)
    return dwte, dwpe


# ----------------------------------------------------------------------------
# LM head + softmax cross-entropy (nanoGPT page, train.py: targets are the
# inputs shifted by one and the loss is the mean over tokens; weight tying
# makes the head weight the token embedding).
# ----------------------------------------------------------------------------

def xent_fwd_bwd(h, W, targets, scale, want_grad=True, row_chunk=2048, weights=None):
    """h: [N, C]; W: [V, C]; targets: int [N].

    nats_n = logsumexp(z_n) - z_n[y_n] with z = h W^T; loss = scale * sum nats.
    With want_grad: dz = (softmax(z) - onehot(y)) * scale, dh = dz W,
    dW = dz^T h.  Rows are processed in chunks only to bound memory; each row
    is complete (all V logits) inside its chunk.

    weights (float [N], optional) weight each token: loss = scale * sum
    w_n nats_n and row n of dz carries scale * w_n.  With w the 0/1 mask of
    the tokens to learn and scale = 1 / sum(mask) this is the masked mean of
    the chat fine-tuning stage ("Train your own ChatGPT", section 6.3: the
    per-token losses times the mask, summed, over the mask's sum).
    """
    N, C = h.shape
    nats = np.empty(N)
    dh = np.empty_like(h) if want_grad else None
    dW = np.zeros_like(W) if want_grad else None
    for r0 in range(0, N, row_chunk):
        r1 = min(N, r0 + row_chunk)
        z = h[r0:r1] @ W.T
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        s = e.sum(axis=1, keepdims=True)
        lse = (m + np.log(s))[:, 0]
        rows = np.arange(r1 - r0)
        nats[r0:r1] = lse - z[rows, targets[r0:r1]]
        if want_grad:
            dz = e / s
            dz[rows, targets[r0:r1]] -= 1.0
            dz *= scale
            if weights is not None:
                dz *= np.asarray(weights[r0:r1], dtype=np.float64)[:, None]
            dh[r0:r1] = dz @ W
            dW += dz.T @ h[r0:r1]
    if weights is None:
        loss = scale * nats.sum()
    else:
        loss = scale * float(np.dot(np.asarray(weights, dtype=np.float64), nats))
    return loss, nats, dh, dW


def val_bpb(nats, targets, token_bytes):
    """Bits per byte ("Train your own ChatGPT", 6.2, loss_eval.py paragraph).

    Sum the nats of the evaluated targets, sum the byte lengths of those
    targets, divide with a ln 2 factor; tokens of zero byte length (special
    tokens) are left out of both sums.  Returns (sum_nats, sum_bytes, bpb).
    """
    nb = token_bytes[targets.reshape(-1)]
    keep = nb > 0
    sum_nats = float(nats.reshape(-1)[keep].sum())
    sum_bytes = int(nb[keep].sum())
    bpb = sum_nats / (math.log(2.0) * sum_bytes) if sum_bytes > 0 else float("nan")
    return sum_nats, sum_bytes, bpb


# ----------------------------------------------------------------------------
# Whole model.
# ----------------------------------------------------------------------------

def _final_norm_params(P):
    return P.get("lnf_w"), P.get("lnf_b")


def model_fwd_bwd(cfg, ids, targets, P, want_grad=True):
    """One training step: forward, mean cross-entropy, backward.

    P holds wte [V,C], wpe [T_max,C] or None, blocks (list of block dicts),
    lnf_w, lnf_b, lm_head [V,C] or None (None = tied to wte).
    Returns (loss, nats, grads) with grads keyed like P (blocks as a list).
    """
    B, T = ids.shape
    N = B * T
    x = embed_fwd(ids, P["wte"], P.get("wpe"))
    caches = []
    for bp in P["blocks"]:
        x, c = block_fwd(cfg, x, bp)
        caches.append(c)
    lw, lb = _final_norm_params(P)
    hf = norm_fwd(cfg, x, lw, lb)
    W = P["lm_head"] if P.get("lm_head") is not None else P["wte"]
    loss, nats, dh, dW = xent_fwd_bwd(hf.reshape(N, -1), W, targets.reshape(-1), 1.0 / N, want_grad)
    if not want_grad:
        return loss, nats, None
    grads = {}
    dx, grads["lnf_w"], grads["lnf_b"] = norm_bwd(cfg, dh.reshape(x.shape), x, lw)
    gb = [None] * len(P["blocks"])
    for i in range(len(P["blocks"]) - 1, -1, -1):
        dx, gb[i] = block_bwd(cfg, dx, caches[i], P["blocks"][i])
    grads["blocks"] = gb
    wpe = P.get("wpe")
    dwte, dwpe = embed_bwd(dx, ids, P["wte"].shape[0], 0 if wpe is None else wpe.shape[0])
    if P.get("lm_head") is not None:
        grads["lm_head"] = dW
        grads["wte"] = dwte
    else:
        grads["wte"] = dwte + dW
    grads["wpe"] = dwpe
    return loss, nats, grads


def model_eval_nats(cfg, ids, targets, P):
    """Forward only: per-target nats [B*T] (the val_bpb evaluation pass)."""
    x = embed_fwd(ids, P["wte"], P.get("wpe"))
    for bp in P["blocks"]:
        x, _ = block_fwd(cfg, x, bp)
    lw, lb = _final_norm_params(P)
    hf = norm_fwd(cfg, x, lw, lb)
    W = P["lm_head"] if P.get("lm_head") is not None else P["wte"]
    N = ids.size
    _, nats, _, _ = xent_fwd_bwd(hf.reshape(N, -1), W, targets.reshape(-1), 1.0, want_grad=False)
    return nats


# ----------------------------------------------------------------------------
# Optimizer step.
# nanoGPT page, model.py section (configure_optimizers): AdamW with weight
# decay on every 2-D tensor and none on 1-D tensors; train.py section:
# gradients clipped to a global norm of 1.0 before the step.  The pages name
# AdamW without restating it; the steps below are the decoupled-weight-decay
# Adam of Loshchilov & Hutter ("Decoupled Weight Decay Regularization",
# Algorithm 2, with the bias-corrected moments of Adam), in the order
# PyTorch's AdamW applies them: decay of the old parameter, then the Adam
# step.  Readings: clipping multiplies every gradient by max_norm / ||g||
# when the global L2 norm ||g|| exceeds max_norm (no further epsilon);
# beta1, beta2, eps, the decay rate and the learning rate are caller inputs
# (the pages fix none of them).
# ----------------------------------------------------------------------------

def clip_scale(grads, max_norm):
    """Global L2 norm over all gradient arrays and the factor that clips it."""
    total = math.sqrt(sum(float(np.sum(np.asarray(g, dtype=np.float64) ** 2)) for g in grads))
    if max_norm > 0 and total > max_norm:
        return total, max_norm / total
    return total, 1.0


def adamw_step(p, g, m, v, step, lr, beta1, beta2, eps, weight_decay, decay, scale=1.0):
    """One AdamW update of one tensor (float64).  step counts from 1.

    Returns (p_new, m_new, v_new).  g is multiplied by the clip factor
    `scale` first; `decay` selects weight decay for this tensor.
    """
    g = np.asarray(g, dtype=np.float64) * scale
    m_new = beta1 * m + (1.0 - beta1) * g
    v_new = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m_new / (1.0 - beta1 ** step)
    v_hat = v_new / (1.0 - beta2 ** step)
    p_new = p * (1.0 - lr * weight_decay) if decay else np.array(p, dtype=np.float64, copy=True)
    p_new = p_new - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p_new, m_new, v_new


# ----------------------------------------------------------------------------
# FP8 GEMMs.  "Train your own ChatGPT", 6.2 (the FP8 paragraph) and the
# nanochat-d20 card (Pretraining row: the published run trained in FP8): the
# matmuls run on 8-bit floats with a dynamic per-tensor scale.  The formats
# are the OCP 8-bit floats: E4M3 (bias 7, no infinities, largest 448) for
# activations and weights, E5M2 (bias 15, largest 57344) for gradients.
# Readings: the scale of a tensor is fmt_max / amax (1 when amax = 0), both in
# float32, and a value's code is x * scale rounded in float32, clamped to
# +-fmt_max, then rounded to nearest even on the format's grid; the GEMM
# result is (sum_k qa qb) / (scale_a scale_b).
# ----------------------------------------------------------------------------

FP8_FORMATS = {"e4m3": dict(mbits=3, bias=7, max=448.0), "e5m2": dict(mbits=2, bias=15, max=57344.0)}


def fp8_round(x, fmt):
    """Nearest value of the format's grid (ties to even), saturating at the
    largest finite value.  x: float64 array of values to round."""
    f = FP8_FORMATS[fmt]
    x = np.clip(np.asarray(x, dtype=np.float64), -f["max"], f["max"])
    a = np.abs(x)
    emin = 1 - f["bias"]                       # exponent of the smallest normal
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)                    # subnormals share the quantum of emin
    q = np.exp2(e - f["mbits"])                # spacing of the grid at a
    r = np.round(a / q) * q                    # numpy rounds half to even
    return np.copysign(np.minimum(r, f["max"]), x)


def fp8_encode(v, fmt):
    """Byte codes (uint8) of values already on the format's grid."""
    f = FP8_FORMATS[fmt]
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    emin = 1 - f["bias"]
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    normal = (a >= 2.0 ** emin) & (a > 0)
    exp_field = np.where(normal, e + f["bias"], 0)
    mant = np.where(normal, a / np.exp2(e) - 1.0, a / 2.0 ** emin) * 2 ** f["mbits"]
    code = (exp_field.astype(np.int64) << f["mbits"]) | np.rint(mant).astype(np.int64)
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def fp8_quantize(x, fmt):
    """(values on the fp8 grid, scale, amax) of a tensor, the scale and the
    product x * scale formed in float32 as the kernels do."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0.0)
    scale = np.float32(FP8_FORMATS[fmt]["max"]) / amax if amax > 0 else np.float32(1.0)
    y = (x32 * scale).astype(np.float64)
    return fp8_round(y, fmt), float(scale), float(amax)


def fp8_gemm(qa, scale_a, qb, scale_b):
    """C[m, n] = sum_k qa[m, k] qb[n, k] / (scale_a scale_b) in float64."""
    return (np.asarray(qa, dtype=np.float64) @ np.asarray(qb, dtype=np.float64).T) / (scale_a * scale_b)
