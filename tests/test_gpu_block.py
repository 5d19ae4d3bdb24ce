"""GPU parity of gpt_block_fwd / gpt_block_bwd against the float64 oracle.

Both forms of the block (GPT-2: LayerNorm with bias, learned positions; d20:
parameter-free RMSNorm, RoPE, QK-norm), at a ragged size that spans several
tiles and at the full single-block workload sizes, plus edge cases and
bitwise invariants (causality, run-to-run determinism).
"""
import numpy as np
import pytest
import torch

import oracle as O
from decoder_only_gpt_bf16_amd import synth
from decoder_only_gpt_bf16_amd.model import BlockRunner, to_f64
from tests._parity import REL_ACT, assert_rel, print_case

pytestmark = pytest.mark.gpu

CASES = [
    ("gpt2_block", dict(B=2, T=200), False),
    ("gpt2_block", dict(B=2, T=200), True),
    ("d20_block", dict(B=2, T=200), False),
    ("d20_block", dict(B=3, T=1), False),
    ("d20_block", dict(B=1, T=64), False),
    ("gpt2_block", dict(), False),   # full: B=8, T=1024
    ("d20_block", dict(), False),    # full: B=4, T=2048 (the benchmarked workload)
    # sliding-window attention: windows that cut tiles, a window of one key,
    # the 64-wide heads, the fp32 (SIMT) path, and the full d20 size
    ("d20_block", dict(B=2, T=320, window=96), False),
    ("d20_block", dict(B=2, T=320, window=200), False),
    ("d20_block", dict(B=1, T=300, window=1), False),
    ("gpt2_block", dict(B=2, T=200, window=64), True),
    ("tiny_gpt_fp32", dict(B=2, T=32, window=5), False),
    ("d20_block", dict(window=512), False),
    # bf16 with head_dim 32: the vector-ALU attention, with the transposed
    # weights of the backward written by a launch of their own
    ("gpt2_block", dict(B=2, T=130, n_head=24), True),
    # the d20 form at C = 640 over 16384 tokens: the 256 x 160 GEMM tiles with
    # k-tile counts 10, 30 and 40 (all three remainders of the loop's
    # unrolling by three)
    ("d20_block", dict(B=8, T=2048, n_embd=640, n_head=5), False),
    # the d20 form at C = 1216 (19 heads of 64): the four weight gradients
    # take the single round of 256 x 320 tiles (236 of them), ragged in both
    # dimensions (1216 = 4 x 256 + 192 rows, 3648 = 11 x 320 + 128 columns)
    ("d20_block", dict(B=2, T=300, n_embd=1216, n_head=19), False),
]


def _ids(c):
    name, sz, aff = c
    win = f"-W{sz['window']}" if "window" in sz else ""
    heads = f"-H{sz['n_head']}" if "n_head" in sz else ""
    width = f"-C{sz['n_embd']}" if "n_embd" in sz else ""
    return f"{name}-B{sz.get('B', 'full')}-T{sz.get('T', 'full')}{win}{heads}{width}{'-affine' if aff else ''}"


def _run(w, random_affine, seed=0):
    x, dy, p = synth.make_block_inputs(w, seed=seed, random_affine=random_affine)
    r = BlockRunner(w.cfg, w.B, w.T, x, dy, p)
    r.step()
    torch.cuda.synchronize()
    return x, dy, p, r


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_block_parity(case):
    name, sz, aff = case
    w = synth.scaled(synth.BY_NAME[name], **sz)
    print_case("block", name, w.B, w.T, f"window={w.cfg.window}", "affine" if aff else "")
    x, dy, p, r = _run(w, aff)
    cfg = synth.oracle_cfg(w.cfg)
    y_ref, cache = O.block_fwd(cfg, x, p)
    dx_ref, g_ref = O.block_bwd(cfg, dy, cache, p)
    N = w.B * w.T
    y = to_f64(r.y).reshape(x.shape)
    rep = {}
    assert_rel("y", y, y_ref, REL_ACT, rep)
    assert_rel("y-x", y - x, y_ref - x, REL_ACT, rep)
    assert_rel("dx", to_f64(r.dx).reshape(x.shape), dx_ref, REL_ACT, rep)
    for k, v in g_ref.items():
        if v is None:
            assert r.g[k] is None
            continue
        assert_rel("d" + k, to_f64(r.g[k]), v, REL_ACT, rep)
    print(name, N, {k: f"{v:.2e}" for k, v in rep.items()})


@pytest.mark.parametrize("name", ["gpt2_block", "d20_block"])
def test_block_deterministic_and_causal(name):
    """Bitwise: the same inputs give the same outputs twice; changing rows
    after position t leaves the forward output at positions <= t unchanged."""
    w = synth.scaled(synth.BY_NAME[name], B=2, T=256)
    print_case("block-invariants", name)
    x, dy, p, r = _run(w, False)
    y1, dx1 = r.y.clone(), r.dx.clone()
    g1 = {k: v.clone() for k, v in r.g.items() if v is not None}
    r.step()
    torch.cuda.synchronize()
    assert torch.equal(y1, r.y) and torch.equal(dx1, r.dx)
    for k, v in g1.items():
        assert torch.equal(v, r.g[k]), k
    t = 100
    x2 = x.copy()
    x2[:, t + 1:] = synth.round_to(np.random.default_rng(3).standard_normal(x2[:, t + 1:].shape), "bf16")
    r2 = BlockRunner(w.cfg, w.B, w.T, x2, dy, p)
    r2.forward()
    torch.cuda.synchronize()
    ya = r.y.view(w.B, w.T, -1)
    yb = r2.y.view(w.B, w.T, -1)
    assert torch.equal(ya[:, : t + 1], yb[:, : t + 1])
    assert not torch.equal(ya[:, t + 1:], yb[:, t + 1:])


@pytest.mark.parametrize("window", [0, 512])
def test_block_deterministic_full(window):
    """Bitwise run-to-run equality at the full d20 size (causal and
    windowed), over four steps of one runner."""
    w = synth.scaled(synth.D20_BLOCK, window=window)
    print_case("block-deterministic-full", window)
    x, dy, p, r = _run(w, False)
    y1, dx1 = r.y.clone(), r.dx.clone()
    g1 = {k: v.clone() for k, v in r.g.items() if v is not None}
    for _ in range(3):
        r.step()
        torch.cuda.synchronize()
        assert torch.equal(y1, r.y) and torch.equal(dx1, r.dx)
        for k, v in g1.items():
            assert torch.equal(v, r.g[k]), k


@pytest.mark.parametrize("name,window", [("d20_block", 70), ("gpt2_block", 130)])
def test_block_window_locality(name, window):
    """Bitwise: with a window of W keys, changing the inputs at positions
    <= t - W leaves the forward output at positions >= t unchanged."""
    w = synth.scaled(synth.BY_NAME[name], B=2, T=320, window=window)
    print_case("block-window-locality", name, window)
    x, dy, p = synth.make_block_inputs(w)
    r1 = BlockRunner(w.cfg, w.B, w.T, x, dy, p)
    r1.forward()
    t = 250
    x2 = x.copy()
    x2[:, : t - window + 1] = synth.round_to(np.random.default_rng(5).standard_normal(x2[:, : t - window + 1].shape),
                                             "bf16")
    r2 = BlockRunner(w.cfg, w.B, w.T, x2, dy, p)
    r2.forward()
    torch.cuda.synchronize()
    ya = r1.y.view(w.B, w.T, -1)
    yb = r2.y.view(w.B, w.T, -1)
    assert torch.equal(ya[:, t:], yb[:, t:])
    assert not torch.equal(ya[:, t - 1], yb[:, t - 1])


def test_block_accumulate():
    """accumulate=1 adds the new parameter gradients to the old ones."""
    w = synth.scaled(synth.GPT2_BLOCK, B=1, T=96)
    print_case("block-accumulate")
    x, dy, p, r = _run(w, True)
    g1 = {k: v.clone() for k, v in r.g.items() if v is not None}
    r.forward()
    r.backward(accumulate=1)
    torch.cuda.synchronize()
    for k, v in g1.items():
        torch.testing.assert_close(r.g[k], 2 * v, rtol=1e-5, atol=1e-7)


def test_block_inference_matches_training_forward():
    """saved = NULL (inference) gives the same y as the training forward."""
    w = synth.scaled(synth.D20_BLOCK, B=2, T=130)
    print_case("block-inference")
    x, dy, p, r = _run(w, False)
    y1 = r.y.clone()
    r.forward(saved=False)
    torch.cuda.synchronize()
    assert torch.equal(y1, r.y)


# Small token counts for the grouped weight-gradient launch: at the GPT-2
# width (108 tiles of 256 x 256, stream-K) 128 tokens leave some of the 256
# blocks without k-steps in the split phase; the d20 width takes one round of
# 240 tiles of 256 x 320 at any token count.
STREAMK_SPARSE = [("d20_block", 1, 128), ("d20_block", 1, 192), ("d20_block", 1, 320), ("gpt2_block", 1, 128)]


@pytest.mark.parametrize("name,Bsz,T", STREAMK_SPARSE, ids=[f"{n}-B{b}-T{t}" for n, b, t in STREAMK_SPARSE])
def test_block_parity_stale_workspace(name, Bsz, T):
    """Block parity with every workspace byte set to 0xFF (NaN as fp32)
    before the call: no result may depend on workspace contents the call did
    not write itself."""
    w = synth.scaled(synth.BY_NAME[name], B=Bsz, T=T)
    print_case("block-stale-ws", name, Bsz, T)
    x, dy, p = synth.make_block_inputs(w, random_affine=name == "gpt2_block")
    r = BlockRunner(w.cfg, w.B, w.T, x, dy, p)
    r.ws.fill_(255)
    r.step()
    torch.cuda.synchronize()
    cfg = synth.oracle_cfg(w.cfg)
    y_ref, cache = O.block_fwd(cfg, x, p)
    dx_ref, g_ref = O.block_bwd(cfg, dy, cache, p)
    rep = {}
    assert_rel("y", to_f64(r.y).reshape(x.shape), y_ref, REL_ACT, rep)
    assert_rel("dx", to_f64(r.dx).reshape(x.shape), dx_ref, REL_ACT, rep)
    for k, v in g_ref.items():
        if v is not None:
            assert_rel("d" + k, to_f64(r.g[k]), v, REL_ACT, rep)
    print(name, Bsz, T, {k: f"{v:.2e}" for k, v in rep.items()})


@pytest.mark.parametrize("name,Bsz,T,fp8", [("d20_block", 1, 192, False), ("d20_block", 2, 2048, False),
                                             ("d20_block", 2, 2048, True), ("gpt2_block", 1, 128, False),
                                             ("gpt2_block", 8, 1024, False)])
def test_block_accumulate_streamk(name, Bsz, T, fp8):
    """accumulate=1 through the grouped weight gradients: the d20 width's
    single round of 256 x 320 tiles (bf16, or FP8 codes with fp8) and the
    GPT-2 width's stream-K launch (the whole tiles' epilogue and the fixup of
    the split tiles).  A second identical backward doubles every parameter
    gradient exactly (the reductions have a fixed order, so the two passes
    are bitwise equal)."""
    w = synth.scaled(synth.BY_NAME[name], B=Bsz, T=T, fp8=fp8)
    print_case("block-accumulate-streamk", name, Bsz, T, "fp8" if fp8 else "")
    x, dy, p, r = _run(w, False)
    g1 = {k: v.clone() for k, v in r.g.items() if v is not None}
    r.ws.fill_(255)
    r.forward()
    r.backward(accumulate=1)
    torch.cuda.synchronize()
    for k, v in g1.items():
        assert torch.equal(r.g[k], 2 * v), k
