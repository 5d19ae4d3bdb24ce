"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and the oracle.

This module holds no arithmetic of the method: it draws token ids, weights,
activations and upstream gradients from fixed seeds, rounds them once to the
storage type, and returns float64 arrays whose values are exactly
representable in that storage type (bf16 or fp32).  Both sides of a parity
test receive these same values.

Recipe (all draws float64 from numpy's PCG64):
  * tensor number j of workload c is drawn from default_rng([c, seed, j]) in
    the fixed order listed by each generator;
  * Linear and embedding weights ~ N(0, 0.02^2); residual output projections
    of a full model ~ N(0, (0.02/sqrt(2*n_layer))^2) ("nanoGPT — Karpathy's
    minimal GPT pretraining repo", model.py section, scaled residual init);
  * norm gains 1, biases 0, unless random_affine=True (then gains 1+N(0,0.1^2),
    biases N(0,0.1^2), so those code paths carry non-trivial values);
  * block inputs x ~ N(0,1), upstream gradient dy ~ N(0, 1e-2^2);
  * token ids: uniform, or Zipf(s) on a finite support 1..V_real with
    p(k) proportional to k^-s, id = k-1, by inverse-CDF sampling;
    targets are the ids shifted by one (draw [B, T+1], x = [:, :T],
    y = [:, 1:]; nanoGPT page, train.py section);
  * token byte lengths: one value per vocabulary entry, uniform in 1..12;
  * optimizer state (make_adamw_inputs): per tensor, param ~ N(0, 0.02^2),
    grad ~ N(0, g_std^2), first moment ~ N(0, (0.1 g_std)^2), second moment
    = (N(0, g_std^2))^2, all fp32; tensor j drawn from
    default_rng([100, seed, j]).
Rounding: float64 -> float32 (round to nearest even) -> bf16 (round to
nearest even on the float32 bits).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


# ----------------------------------------------------------------------------
# Model configuration (mirrors nanoGPT's GPTConfig plus the fields the two
# model forms need).
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class GPTConfig:
    n_layer: int
    n_head: int
    n_embd: int
    block_size: int
    vocab_size: int
    bias: bool = True
    norm: str = "layernorm"      # or "rmsnorm" (parameter-free)
    rope: bool = False           # False: learned absolute positions (wpe)
    qk_norm: bool = False
    rope_base: float = 10000.0
    eps: float = 1e-5
    dtype: str = "bf16"          # storage type: "bf16" or "fp32"
    window: int = 0              # sliding attention window (keys i-W+1..i); 0: full causal
    fp8: bool = False            # the block's Linear layers as FP8 GEMMs
    tied: bool = True            # lm_head weight is wte
    vocab_real: Optional[int] = None  # ids are drawn below this (padded vocab)

    @property
    def head_dim(self) -> int:
        return self.n_embd // self.n_head

    def as_dict(self) -> dict:
        return dataclasses.asdict(self)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One named workload: a model form plus batch shape and input recipe."""
    index: int
    name: str
    cfg: GPTConfig
    B: int
    T: int
    kind: str                    # "step" (full model fwd+bwd), "block", "eval"
    ids: str = "uniform"         # "uniform" or "zipf"
    zipf_s: float = 1.1
    bytes_mode: str = "ones"     # "ones" or "uniform_1_12"


TINY = Workload(0, "tiny_gpt_fp32", GPTConfig(
    n_layer=1, n_head=4, n_embd=64, block_size=32, vocab_size=27,
    bias=True, norm="layernorm", rope=False, qk_norm=False, dtype="fp32"),
    B=2, T=32, kind="step", ids="uniform", bytes_mode="ones")

GPT2_BLOCK = Workload(1, "gpt2_block", GPTConfig(
    n_layer=1, n_head=12, n_embd=768, block_size=1024, vocab_size=50304,
    bias=True, norm="layernorm", rope=False, qk_norm=False),
    B=8, T=1024, kind="block")

D20_BLOCK = Workload(2, "d20_block", GPTConfig(
    n_layer=1, n_head=10, n_embd=1280, block_size=2048, vocab_size=32768,
    bias=False, norm="rmsnorm", rope=True, qk_norm=True),
    B=4, T=2048, kind="block")

GPT2_STEP = Workload(3, "gpt2_124m_step", GPTConfig(
    n_layer=12, n_head=12, n_embd=768, block_size=1024, vocab_size=50304,
    bias=True, norm="layernorm", rope=False, qk_norm=False, vocab_real=50257),
    B=16, T=1024, kind="step", ids="zipf")

D20_EVAL = Workload(4, "d20_val_bpb", GPTConfig(
    n_layer=20, n_head=10, n_embd=1280, block_size=2048, vocab_size=32768,
    bias=False, norm="rmsnorm", rope=True, qk_norm=True, tied=False),
    B=8, T=2048, kind="eval", ids="zipf", bytes_mode="uniform_1_12")

WORKLOADS = [TINY, GPT2_BLOCK, D20_BLOCK, GPT2_STEP, D20_EVAL]
BY_NAME = {w.name: w for w in WORKLOADS}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with other sizes (B, T, or config fields)."""
    top = {k: changes.pop(k) for k in list(changes) if k in ("B", "T", "kind", "ids", "bytes_mode", "name")}
    cfg = dataclasses.replace(w.cfg, **changes) if changes else w.cfg
    return dataclasses.replace(w, cfg=cfg, **top)


# ----------------------------------------------------------------------------
# Storage rounding.
# ----------------------------------------------------------------------------

def bf16_bits(a) -> np.ndarray:
    """float64/float32 array -> uint16 bf16 bit patterns (round to nearest even)."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(f)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_to(a, dtype: str) -> np.ndarray:
    """Round float64 values once to the storage type and return them as float64."""
    if dtype == "fp32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    return bits_to_f64(bf16_bits(a))


# ----------------------------------------------------------------------------
# Draws.
# ----------------------------------------------------------------------------

class _Stream:
    """Hands out one independent generator per tensor, in draw order."""

    def __init__(self, index: int, seed: int):
        self.index, self.seed, self.j = index, seed, 0

    def next(self) -> np.random.Generator:
        g = np.random.default_rng([self.index, self.seed, self.j])
        self.j += 1
        return g


def zipf_ids(rng: np.random.Generator, shape, v_real: int, s: float) -> np.ndarray:
    k = np.arange(1, v_real + 1, dtype=np.float64)
    p = k ** (-s)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    u = rng.random(size=shape)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, v_real - 1).astype(np.int64)


def _normal(st: _Stream, shape, std, dtype):
    return round_to(st.next().standard_normal(size=shape) * std, dtype)


def block_params(st: _Stream, cfg: GPTConfig, resid_std: float, random_affine: bool):
    """Draw order: w_qkv, w_o, w_fc, w_proj, then (if present) ln1_w, ln1_b,
    b_qkv, b_o, ln2_w, ln2_b, b_fc, b_proj."""
    C = cfg.n_embd
    dt = cfg.dtype
    p = {
        "w_qkv": _normal(st, (3 * C, C), 0.02, dt),
        "w_o": _normal(st, (C, C), resid_std, dt),
        "w_fc": _normal(st, (4 * C, C), 0.02, dt),
        "w_proj": _normal(st, (C, 4 * C), resid_std, dt),
    }
    ln = cfg.norm == "layernorm"

    def gain():
        if random_affine:
            return round_to(1.0 + 0.1 * st.next().standard_normal(C), dt)
        return np.ones(C)

    def vec(n):
        if random_affine:
            return round_to(0.1 * st.next().standard_normal(n), dt)
        return np.zeros(n)

    p["ln1_w"] = gain() if ln else None
    p["ln1_b"] = vec(C) if (ln and cfg.bias) else None
    p["b_qkv"] = vec(3 * C) if cfg.bias else None
    p["b_o"] = vec(C) if cfg.bias else None
    p["ln2_w"] = gain() if ln else None
    p["ln2_b"] = vec(C) if (ln and cfg.bias) else None
    p["b_fc"] = vec(4 * C) if cfg.bias else None
    p["b_proj"] = vec(C) if cfg.bias else None
    return p


def make_block_inputs(w: Workload, seed: int = 0, random_affine: bool = False):
    """Inputs of one block fwd+bwd.  Draw order: x, dy, block params.
    Weights all N(0, 0.02^2) (no residual scaling for a lone block)."""
    cfg = w.cfg
    st = _Stream(w.index, seed)
    x = _normal(st, (w.B, w.T, cfg.n_embd), 1.0, cfg.dtype)
    dy = _normal(st, (w.B, w.T, cfg.n_embd), 1e-2, cfg.dtype)
    p = block_params(st, cfg, 0.02, random_affine)
    return x, dy, p


def make_model_inputs(w: Workload, seed: int = 0, random_affine: bool = False,
                      n_layer: Optional[int] = None):
    """Inputs of a full model step or eval.

    Draw order: ids [B, T+1], wte, wpe (learned positions only), then each
    block's params, then final-norm gain/bias (LayerNorm only), lm_head
    (untied only), token_bytes.  Returns (ids, targets, P, token_bytes).
    """
    cfg = w.cfg
    L = cfg.n_layer if n_layer is None else n_layer
    st = _Stream(w.index, seed)
    V, C = cfg.vocab_size, cfg.n_embd
    v_real = cfg.vocab_real or V
    g = st.next()
    if w.ids == "zipf":
        seq = zipf_ids(g, (w.B, w.T + 1), v_real, w.zipf_s)
    else:
        seq = g.integers(0, v_real, size=(w.B, w.T + 1)).astype(np.int64)
    ids, targets = seq[:, :-1].copy(), seq[:, 1:].copy()
    P = {"wte": _normal(st, (V, C), 0.02, cfg.dtype)}
    P["wpe"] = None if cfg.rope else _normal(st, (cfg.block_size, C), 0.02, cfg.dtype)
    resid = 0.02 / math.sqrt(2 * cfg.n_layer)
    P["blocks"] = [block_params(st, cfg, resid, random_affine) for _ in range(L)]
    if cfg.norm == "layernorm":
        if random_affine:
            P["lnf_w"] = round_to(1.0 + 0.1 * st.next().standard_normal(C), cfg.dtype)
            P["lnf_b"] = round_to(0.1 * st.next().standard_normal(C), cfg.dtype) if cfg.bias else None
        else:
            P["lnf_w"] = np.ones(C)
            P["lnf_b"] = np.zeros(C) if cfg.bias else None
    else:
        P["lnf_w"], P["lnf_b"] = None, None
    P["lm_head"] = None if cfg.tied else _normal(st, (V, C), 0.02, cfg.dtype)
    if w.bytes_mode == "uniform_1_12":
        token_bytes = st.next().integers(1, 13, size=V).astype(np.int64)
    else:
        token_bytes = np.ones(V, dtype=np.int64)
    return ids, targets, P, token_bytes


def oracle_cfg(cfg: GPTConfig) -> dict:
    """The plain-dict form of a configuration that the oracle takes."""
    return dict(n_layer=cfg.n_layer, n_head=cfg.n_head, n_embd=cfg.n_embd,
                vocab_size=cfg.vocab_size, norm=cfg.norm, bias=cfg.bias,
                rope=cfg.rope, qk_norm=cfg.qk_norm, rope_base=cfg.rope_base,
                eps=cfg.eps, window=cfg.window, fp8=cfg.fp8)


def make_adamw_inputs(shapes, seed: int = 0, g_std: float = 1e-2):
    """fp32-representable float64 arrays (param, grad, m, v) per shape."""
    out = []
    for j, shp in enumerate(shapes):
        rng = np.random.default_rng([100, seed, j])
        p = round_to(rng.normal(0.0, 0.02, shp), "fp32")
        g = round_to(rng.normal(0.0, g_std, shp), "fp32")
        m = round_to(rng.normal(0.0, 0.1 * g_std, shp), "fp32")
        v = round_to(rng.normal(0.0, g_std, shp) ** 2, "fp32")
        out.append((p, g, m, v))
    return out


def block_param_shapes(cfg: "GPTConfig"):
    """(shape, is 2-D) of one block's parameters in BLOCK_FIELDS order, biases
    and norm gains included only where the configuration has them."""
    C = cfg.n_embd
    ln = cfg.norm == "layernorm"
    out = []
    for name, shp in (("ln1_w", (C,)), ("ln1_b", (C,)), ("w_qkv", (3 * C, C)), ("b_qkv", (3 * C,)),
                      ("w_o", (C, C)), ("b_o", (C,)), ("ln2_w", (C,)), ("ln2_b", (C,)),
                      ("w_fc", (4 * C, C)), ("b_fc", (4 * C,)), ("w_proj", (C, 4 * C)), ("b_proj", (C,))):
        if name.startswith("ln") and not ln:
            continue
        if name.endswith("_b") and not (ln and cfg.bias):
            continue
        if name.startswith("b_") and not cfg.bias:
            continue
        out.append((name, shp))
    return out
