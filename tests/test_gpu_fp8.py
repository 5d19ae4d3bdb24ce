"""GPU parity of the FP8 path: dynamic per-tensor quantization (codes,
scale and amax bit-exact against the oracle) and the FP8 GEMM on the 8-bit
MFMA (against the oracle's float64 product of the same codes).

GEMM tolerance, from the arithmetic: products of two 8-bit floats are exact
in fp32; the fp32 sums carry about K 2^-24 relative error and the bf16
output rounds each element by at most 2^-9, so ||gpu - oracle|| / ||oracle||
stays below 1e-2.
"""
import numpy as np
import pytest
import torch

import oracle as O
from decoder_only_gpt_bf16_amd import binding as B
from decoder_only_gpt_bf16_amd import synth
from decoder_only_gpt_bf16_amd.model import BlockRunner, to_f64
from tests._parity import assert_rel, print_case

pytestmark = pytest.mark.gpu

FMT = {"e4m3": B.FP8_E4M3, "e5m2": B.FP8_E5M2}
REL_FP8_GEMM = 1e-2
# The block with FP8 Linear layers against the oracle's FP8 block.  Both
# quantize nearly equal bf16 inputs, with nearly equal per-tensor scales;
# where the two inputs fall on either side of a rounding boundary of the
# format the codes differ by one step of it, so the two results differ at
# the scale of FP8 rounding itself rather than of bf16's.  The gradient
# operand is E5M2 (2 mantissa bits, relative half-step 2^-3), which bounds
# the per-tensor difference: REL_FP8 = 2^-3 (worst measured 8.4%, dW_qkv).
# Rows and single elements average fewer such disagreements, as in the bf16
# bounds: 2^-1 per row (worst measured 0.22) and 2 per element of its row's
# scale (worst measured 1.25, a LayerNorm gain gradient).  A wrong scale,
# operand or layout misses these by an order of magnitude or more.
REL_FP8, REL_FP8_ROW, REL_FP8_ELEM = 2.0 ** -3, 2.0 ** -1, 2.0


def _bf16(a):
    return torch.tensor(synth.bf16_bits(a).view(np.int16), device="cuda").view(torch.bfloat16)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
# 4096 * 4096 + 999 elements give 4097 amax partials: the finish kernel's
# batched loads (16 x 256 at a time) run
@pytest.mark.parametrize("n,std", [(13, 1.0), (4096 * 3 + 17, 0.02), (1280 * 5120, 0.02), (8192 * 1280, 3.0),
                                   (4096 * 4096 + 999, 1.0)])
def test_quantize_bit_exact(fmt, n, std):
    print_case("fp8 quantize", fmt, n)
    rng = np.random.default_rng(n)
    x = synth.round_to(rng.standard_normal(n) * std, "bf16")
    q = torch.empty(n, dtype=torch.uint8, device="cuda")
    sc = torch.zeros(4, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(256, B.gpt_fp8_workspace_bytes(n)), dtype=torch.uint8, device="cuda")
    B.gpt_fp8_quantize(_bf16(x), FMT[fmt], q, sc, ws)
    torch.cuda.synchronize()
    v, scale, amax = O.fp8_quantize(x, fmt)
    assert sc[1].item() == amax
    assert sc[0].item() == scale
    assert sc[2].item() == np.float32(1.0) / np.float32(scale)
    codes = O.fp8_encode(v, fmt)
    got = q.cpu().numpy()
    np.testing.assert_array_equal(got, codes)


def _codes(shape, fmt, rng, spread):
    """Random values on the format's grid and their codes."""
    v = O.fp8_round(rng.standard_normal(shape) * spread, fmt)
    return v, O.fp8_encode(v, fmt)


GEMMS = [
    (300, 264, 208, "e4m3", "e4m3"),      # ragged M, N; K not a multiple of the 128-byte k tile
    (512, 512, 1280, "e4m3", "e4m3"),
    (256, 1280, 5120, "e5m2", "e4m3"),    # an input-gradient shape: E5M2 gradients times E4M3 weights
    (1000, 3840, 1280, "e4m3", "e5m2"),
]


@pytest.mark.parametrize("M,N,K,fa,fb", GEMMS)
def test_fp8_gemm(M, N, K, fa, fb):
    print_case("fp8 gemm", M, N, K, fa, fb)
    rng = np.random.default_rng(M + N + K)
    va, ca = _codes((M, K), fa, rng, 20.0)
    vb, cb = _codes((N, K), fb, rng, 20.0 if fb == "e4m3" else 200.0)
    sa, sb = np.float32(37.5), np.float32(0.125)
    sca = torch.tensor([sa, 1.0, np.float32(1.0) / sa, 0.0], dtype=torch.float32, device="cuda")
    scb = torch.tensor([sb, 1.0, np.float32(1.0) / sb, 0.0], dtype=torch.float32, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    B.gpt_fp8_gemm(torch.tensor(ca, device="cuda"), FMT[fa], sca, torch.tensor(cb, device="cuda"), FMT[fb], scb, out)
    torch.cuda.synchronize()
    ref = O.fp8_gemm(va, float(sa), vb, float(sb))
    rep = {}
    assert_rel("C", to_f64(out), ref, REL_FP8_GEMM, rep)
    print(M, N, K, fa, fb, rep)


def test_fp8_linear_end_to_end():
    """bf16 activations and weight quantized on the GPU, then the GEMM: the
    result matches the oracle's FP8 product and stays near the bf16 one."""
    M, N, K = 8192, 5120, 1280
    print_case("fp8 linear", M, N, K)
    rng = np.random.default_rng(5)
    x = synth.round_to(rng.standard_normal((M, K)), "bf16")
    w = synth.round_to(rng.normal(0, 0.02, (N, K)), "bf16")
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    qb = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sa = torch.zeros(4, dtype=torch.float32, device="cuda")
    sb = torch.zeros(4, dtype=torch.float32, device="cuda")
    ws = torch.empty(B.gpt_fp8_workspace_bytes(M * K), dtype=torch.uint8, device="cuda")
    B.gpt_fp8_quantize(_bf16(x), B.FP8_E4M3, qa, sa, ws)
    B.gpt_fp8_quantize(_bf16(w), B.FP8_E4M3, qb, sb, ws)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    B.gpt_fp8_gemm(qa, B.FP8_E4M3, sa, qb, B.FP8_E4M3, sb, out)
    torch.cuda.synchronize()
    va, s_a, _ = O.fp8_quantize(x, "e4m3")
    vb, s_b, _ = O.fp8_quantize(w, "e4m3")
    rows = np.random.default_rng(6).choice(M, 256, replace=False)
    got = to_f64(out)[rows]
    ref = O.fp8_gemm(va[rows], s_a, vb, s_b)
    assert_rel("C(sampled rows)", got, ref, REL_FP8_GEMM)
    full = x[rows] @ w.T
    assert np.linalg.norm(got - full) / np.linalg.norm(full) < 0.1


# ---- the block with FP8 Linear layers (gpt_config.fp8) against the oracle's
# FP8 block ----
# (C = 1216: the FP8 weight gradients' single round of 256 x 320 tiles,
# ragged in both dimensions)
FP8_BLOCK = [("d20_block", dict(B=2, T=200)), ("gpt2_block", dict(B=2, T=200)), ("d20_block", dict(B=1, T=77)),
             ("d20_block", dict()), ("gpt2_block", dict()), ("d20_block", dict(B=2, T=300, n_embd=1216, n_head=19))]


@pytest.mark.parametrize("name,sz", FP8_BLOCK, ids=[f"{n}-{s.get('B', 'full')}-{s.get('T', 'full')}-C{s.get('n_embd', 'std')}" for n, s in FP8_BLOCK])
def test_fp8_block_parity(name, sz):
    w = synth.scaled(synth.BY_NAME[name], fp8=True, **sz)
    print_case("fp8-block", name, w.B, w.T)
    x, dy, p = synth.make_block_inputs(w)
    r = BlockRunner(w.cfg, w.B, w.T, x, dy, p)
    r.step()
    torch.cuda.synchronize()
    cfg = synth.oracle_cfg(w.cfg)
    y_ref, cache = O.block_fwd(cfg, x, p)
    dx_ref, g_ref = O.block_bwd(cfg, dy, cache, p)
    rep = {}
    y = to_f64(r.y).reshape(x.shape)
    kw = dict(row_tol=REL_FP8_ROW, elem_tol=REL_FP8_ELEM)
    assert_rel("y-x", y - x, y_ref - x, REL_FP8, rep, **kw)
    assert_rel("dx", to_f64(r.dx).reshape(x.shape), dx_ref, REL_FP8, rep, **kw)
    for k, v in g_ref.items():
        if v is not None:
            assert_rel("d" + k, to_f64(r.g[k]), v, REL_FP8, rep, **kw)
    print(name, w.B, w.T, {k: f"{v:.2e}" for k, v in rep.items()})
