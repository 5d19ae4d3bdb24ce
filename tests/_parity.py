"""Shared helpers of the GPU parity tests (not collected by pytest).

Three bounds apply to every array compared with the oracle:

  * global: ||gpu - ref||_2 / ||ref||_2 <= tol per tensor (REL_ACT 2e-2 for
    bf16 activations and gradients, REL_LOSS 1e-3 for loss, nats sums, bpb);
  * per row (arrays of two or more axes): ||gpu_i - ref_i||_2 <= ROW_TOL * s_i
    for every row i of the 2-D view [-1, last axis], with
    s_i = max(||ref_i||_2, ROW_FLOOR * R) and R the root-mean-square row norm;
  * per element: |gpu_ij - ref_ij| <= ELEM_TOL * s_i / sqrt(L), L the row
    length (s_i / sqrt(L) is the row's root-mean-square element, floored).
    A 1-D array is a column of one-element rows and takes this bound only.

Derivation from bf16 rounding (unit roundoff u = 2^-8): an element of a bf16
result carries a few roundings of u each along its path, so whole tensors
measure 0.7u-1.5u globally.  A row of L >= 64 elements averages L such
errors, so its relative error stays near the tensor's, except for weight
gradients summed over few tokens, whose rows measured up to 8u (sums over
77-128 tokens).  ROW_TOL = 32u = 2^-3 leaves a factor of 4 over that, while
a wrong row (error of the order of the row itself) scores about 1 and fails
by 8x.  Rows whose reference norm is small take absolute errors set by the
upstream activations, which scale with the typical row, hence the floor at a
quarter of R.  Single elements have no averaging: their tails measured up to
31u (the same few-token weight gradients; 22u for LayerNorm gain gradients);
ELEM_TOL = 128u = 2^-1 keeps a factor of 4 and still fails an element that
is wrong by half its row's typical magnitude.
"""
import json
import os

import numpy as np

REL_ACT = 2e-2     # bf16 activations and gradients vs the float64 oracle
REL_LOSS = 1e-3    # loss and bpb
ROW_TOL = 2.0 ** -3
ROW_FLOOR = 0.25
ELEM_TOL = 2.0 ** -1

_CASE = {"name": ""}


def rel(a, b) -> float:
    """||a - b||_2 / ||b||_2 in float64 (scalars: |a - b| / |b|)."""
    a = np.asarray(a, dtype=np.float64).reshape(-1)
    b = np.asarray(b, dtype=np.float64).reshape(-1)
    nb = np.linalg.norm(b)
    if nb == 0.0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def row_errors(a, b):
    """(max over rows of ||a_i - b_i|| / s_i, max over elements of
    |a_ij - b_ij| sqrt(L) / s_i), with rows and s_i as in the module notes."""
    b = np.asarray(b, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64).reshape(b.shape)
    L = b.shape[-1] if b.ndim >= 2 else 1
    b2 = b.reshape(-1, L)
    d2 = a.reshape(-1, L) - b2
    rn = np.sqrt(np.einsum("ij,ij->i", b2, b2))
    R = float(np.sqrt(np.mean(rn * rn)))
    s = np.maximum(rn, ROW_FLOOR * R)
    if R == 0.0:
        s = np.ones_like(rn)
    dn = np.sqrt(np.einsum("ij,ij->i", d2, d2))
    row = float(np.max(dn / s))
    elem = float(np.max(np.max(np.abs(d2), axis=1) * np.sqrt(L) / s))
    return row, elem


def assert_rel(name, got, ref, tol, report=None, row_tol=None, elem_tol=None):
    """Global, per-row and per-element bounds (row_tol, elem_tol default to
    the bf16-derived ROW_TOL, ELEM_TOL)."""
    row_tol = ROW_TOL if row_tol is None else row_tol
    elem_tol = ELEM_TOL if elem_tol is None else elem_tol
    g = np.asarray(got, dtype=np.float64)
    r = rel(g, ref)
    if report is not None:
        report[name] = r
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    row = elem = None
    if np.asarray(ref).size > 1:
        row, elem = row_errors(g, ref)
    _log(name, r, tol, row, elem)
    assert r <= tol, f"{name}: rel err {r:.3e} > {tol:.1e}"
    if row is not None:
        if np.asarray(ref).ndim >= 2:
            assert row <= row_tol, f"{name}: a row's rel err {row:.3e} > {row_tol:.2e}"
        assert elem <= elem_tol, f"{name}: an element's err {elem:.3e} of its row scale > {elem_tol:.2e}"
    return r


def _log(name, r, tol, row, elem):
    path = os.environ.get("GPTMI_PARITY_LOG")
    if not path:
        return
    rec = {"case": _CASE["name"], "name": name, "rel": r, "tol": tol, "row": row, "elem": elem}
    with open(path, "a") as f:
        f.write(json.dumps(rec) + "\n")


def print_case(*parts):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    _CASE["name"] = " ".join(str(p) for p in parts)
    print("CASE", *parts, flush=True)
