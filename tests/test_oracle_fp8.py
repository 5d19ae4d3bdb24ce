"""Pins of the oracle's FP8 quantization and GEMM (CPU only).

The rounding is checked against PyTorch's float8_e4m3fn / float8_e5m2
conversions (an independent implementation) over many values, ties and
subnormals included, and against closed forms: the largest finite values,
the smallest subnormals, and exact byte codes of chosen values.
"""
import numpy as np
import pytest
import torch

import oracle as O

TORCH = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_round_matches_torch(fmt):
    fmax = O.FP8_FORMATS[fmt]["max"]
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 4, 20000),
        rng.uniform(-fmax, fmax, 5000),
        np.array([0.0, -0.0, fmax, -fmax]),
    ])
    x = x[np.abs(x) <= fmax].astype(np.float32).astype(np.float64)
    ours = O.fp8_round(x, fmt)
    theirs = torch.tensor(x, dtype=torch.float32).to(TORCH[fmt]).double().numpy()
    np.testing.assert_array_equal(ours, theirs)
    codes = O.fp8_encode(ours, fmt)
    tcodes = torch.tensor(x, dtype=torch.float32).to(TORCH[fmt]).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes[ours != 0], tcodes[ours != 0])


def test_ties_to_even_and_saturation():
    # grid steps: e4m3 spacing 16 in [128, 256): 232 is halfway between 224 and 240
    assert O.fp8_round(np.array([232.0, 248.0]), "e4m3").tolist() == [224.0, 256.0]
    # 2^-10 is halfway between 0 and the smallest subnormal 2^-9: ties to 0
    assert O.fp8_round(np.array([2.0 ** -10, 3 * 2.0 ** -10]), "e4m3").tolist() == [0.0, 2.0 ** -8]
    assert O.fp8_round(np.array([1e9, -1e9]), "e4m3").tolist() == [448.0, -448.0]
    assert O.fp8_round(np.array([1e9]), "e5m2").tolist() == [57344.0]
    assert O.fp8_encode(np.array([448.0, 1.0, -2.0, 2.0 ** -9]), "e4m3").tolist() == [0x7E, 0x38, 0xC0, 0x01]
    assert O.fp8_encode(np.array([57344.0, 1.0, 2.0 ** -16]), "e5m2").tolist() == [0x7B, 0x3C, 0x01]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quantize_scale_and_amax(fmt):
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(1000) * 3.0).astype(np.float32).astype(np.float64)
    q, scale, amax = O.fp8_quantize(x, fmt)
    assert amax == np.max(np.abs(x))
    assert np.max(np.abs(q)) == O.FP8_FORMATS[fmt]["max"]          # the largest element lands on fmt_max
    rel = np.linalg.norm(q / scale - x) / np.linalg.norm(x)
    assert rel < (0.04 if fmt == "e4m3" else 0.08)                  # 3 or 2 mantissa bits
    q0, s0, a0 = O.fp8_quantize(np.zeros(5), fmt)
    assert s0 == 1.0 and a0 == 0.0 and not q0.any()


def test_fp8_gemm_is_dequantized_product():
    rng = np.random.default_rng(13)
    a = rng.standard_normal((7, 48))
    b = rng.standard_normal((5, 48))
    qa, sa, _ = O.fp8_quantize(a, "e4m3")
    qb, sb, _ = O.fp8_quantize(b, "e5m2")
    c = O.fp8_gemm(qa, sa, qb, sb)
    np.testing.assert_allclose(c, (qa / sa) @ (qb / sb).T, rtol=1e-12)
    # and close to the full-precision product
    assert np.linalg.norm(c - a @ b.T) / np.linalg.norm(a @ b.T) < 0.1


# ---- the FP8 block: pinned to a torch model built on torch's own bf16 and
# float8 casts, with autograd for everything outside the Linear layers ----

def _tq(t, fmt):
    """torch: quantize a tensor from its bf16 value with a per-tensor scale."""
    t32 = t.detach().to(torch.float32).to(torch.bfloat16).to(torch.float32)
    amax = t32.abs().max()
    fmax = torch.tensor(O.FP8_FORMATS[fmt]["max"], dtype=torch.float32)
    scale = fmax / amax if amax > 0 else torch.tensor(1.0, dtype=torch.float32)
    q = (t32 * scale).to(TORCH[fmt]).to(torch.float64)
    return q, scale.double()


class _Fp8Linear(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w, b):
        ctx.save_for_backward(x, w)
        ctx.has_b = b is not None
        x2 = x.reshape(-1, x.shape[-1])
        qx, sx = _tq(x2, "e4m3")
        qw, sw = _tq(w, "e4m3")
        y = (qx @ qw.T) / (sx * sw)
        y = y.reshape(x.shape[:-1] + (w.shape[0],))
        return y + b if b is not None else y

    @staticmethod
    def backward(ctx, dy):
        x, w = ctx.saved_tensors
        dy2 = dy.reshape(-1, dy.shape[-1])
        x2 = x.reshape(-1, x.shape[-1])
        qg, sg = _tq(dy2, "e5m2")
        qw, sw = _tq(w, "e4m3")
        qx, sx = _tq(x2, "e4m3")
        dx = ((qg @ qw) / (sg * sw)).reshape(x.shape)
        dw = (qg.T @ qx) / (sg * sx)
        db = dy2.sum(0) if ctx.has_b else None
        return dx, dw, db


@pytest.mark.parametrize("form", ["gpt2", "d20"])
def test_fp8_block_matches_torch_float8_autograd(form, monkeypatch):
    """The oracle's FP8 block (forward and backward) against a torch model
    whose Linear layers quantize with torch's float8 casts and whose
    backward outside the Linear layers is torch autograd."""
    from tests import test_oracle_torch as TT
    import torch.nn.functional as F
    cfg = dict(TT.FORMS[form], fp8=True)
    rng = np.random.default_rng(5)
    B, T, C = 2, 24, 64
    x = O.bf16_round(rng.standard_normal((B, T, C)))
    p = TT._params(rng, C, cfg)
    p = {k: (None if v is None else O.bf16_round(v)) for k, v in p.items()}
    dy = O.bf16_round(1e-2 * rng.standard_normal(x.shape))
    y, cache = O.block_fwd(cfg, x, p)
    dx, grads = O.block_bwd(cfg, dy, cache, p)
    monkeypatch.setattr(F, "linear", lambda a, w, b=None: _Fp8Linear.apply(a, w, b))
    torch.set_default_dtype(torch.float64)
    try:
        xt = torch.tensor(x, requires_grad=True)
        pt = {k: (None if v is None else torch.tensor(v, requires_grad=True)) for k, v in p.items()}
        yt = TT._torch_block(cfg, xt, pt)
        yt.backward(torch.tensor(dy))
    finally:
        torch.set_default_dtype(torch.float32)
    rel = lambda a, b: np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b))  # noqa: E731
    assert rel(y, yt.detach().numpy()) < 1e-12
    assert rel(dx, xt.grad.numpy()) < 1e-9
    for k, v in pt.items():
        if v is not None:
            assert rel(grads[k], v.grad.numpy()) < 1e-9, k
    # and the FP8 block is an FP8 approximation of the full-precision one
    y0, c0 = O.block_fwd(dict(cfg, fp8=False), x, p)
    dx0, g0 = O.block_bwd(dict(cfg, fp8=False), dy, c0, p)
    assert 1e-3 < rel(y - x, y0 - x) < 0.1
    assert 1e-3 < rel(grads["w_fc"], g0["w_fc"]) < 0.2


def test_fp8_linear_closed_forms():
    """Operands already on the E4M3 grid with amax = 448 (scale 1) pass
    through unchanged, so the FP8 product is exact; a gradient of one value
    in E5M2 and the input of the same kind make dW exact as well."""
    x = np.array([[448.0, 1.0, -2.0, 0.5], [3.0, -448.0, 0.25, 1.5]])
    w = np.array([[448.0, 0.5, 1.0, -1.0], [2.0, 4.0, -448.0, 0.125]])
    np.testing.assert_array_equal(O.fp8_linear_fwd(x, w, None), x @ w.T)
    dy = np.array([[57344.0, 1.0], [-2.0, 0.5]])
    dx, dw, db = O.fp8_linear_bwd(dy, x, w, True)
    np.testing.assert_array_equal(dx, dy @ w)
    np.testing.assert_array_equal(dw, dy.T @ x)
    np.testing.assert_array_equal(db, dy.sum(axis=0))
