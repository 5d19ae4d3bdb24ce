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
