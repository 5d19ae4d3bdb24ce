"""Shared helpers of the GPU parity tests (not collected by pytest)."""
import numpy as np

REL_ACT = 2e-2     # bf16 activations and gradients vs the float64 oracle
REL_LOSS = 1e-3    # loss and bpb


def rel(a, b) -> float:
    """||a - b||_2 / ||b||_2 in float64 (scalars: |a - b| / |b|)."""
    a = np.asarray(a, dtype=np.float64).reshape(-1)
    b = np.asarray(b, dtype=np.float64).reshape(-1)
    nb = np.linalg.norm(b)
    if nb == 0.0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def assert_rel(name, got, ref, tol, report=None):
    r = rel(got, ref)
    if report is not None:
        report[name] = r
    assert np.all(np.isfinite(np.asarray(got, dtype=np.float64))), f"{name}: non-finite values"
    assert r <= tol, f"{name}: rel err {r:.3e} > {tol:.1e}"
    return r


def print_case(*parts):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print("CASE", *parts, flush=True)
