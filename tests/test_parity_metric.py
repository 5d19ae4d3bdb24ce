"""The parity metrics themselves: the per-row and per-element bounds pass
bf16-sized noise and fail a single wrong row or element that the global
per-tensor norm cannot see."""
import numpy as np

from tests._parity import ELEM_TOL, REL_ACT, ROW_TOL, rel, row_errors


def test_row_and_element_bounds():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((8192, 1280))
    got = ref * (1 + 2 ** -8 * rng.uniform(-1, 1, ref.shape))   # one bf16 rounding per element
    row, elem = row_errors(got, ref)
    assert rel(got, ref) < 3e-3 and row < ROW_TOL / 8 and elem < ELEM_TOL / 8
    bad = got.copy()
    bad[4321] = rng.standard_normal(1280)                         # one wrong row of 8192
    assert rel(bad, ref) < REL_ACT                                # invisible to the global norm
    assert row_errors(bad, ref)[0] > 8 * ROW_TOL
    bad = got.copy()
    bad[77, 5] += ref[77].std() * 1.0                             # one element off by its row's scale
    assert row_errors(bad, ref)[0] < ROW_TOL
    assert row_errors(bad, ref)[1] > ELEM_TOL
    # rows of tiny norm are judged against a quarter of the typical row norm
    ref2 = ref.copy()
    ref2[10] *= 1e-6
    got2 = got.copy()
    got2[10] = ref2[10] + 1e-3 * rng.standard_normal(1280)
    assert row_errors(got2, ref2)[0] < ROW_TOL
    # 1-D arrays: every element is a row
    v = rng.standard_normal(1000) + 10
    assert row_errors(v * (1 + 1e-3), v)[1] < 2e-3
    w = v.copy()
    w[3] = -v[3]
    assert row_errors(w, v)[1] > 3 * ELEM_TOL
