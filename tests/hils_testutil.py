"""Helpers shared by the GPU parity tests (tolerances, near-tie bookkeeping)."""
from __future__ import annotations

import sys

import numpy as np

# Output tolerances: float32 paths (and every float32 intermediate: summaries,
# scores, log-sum-exps) 1e-4; bf16 outputs 2e-2; bf16 gradients 5e-2.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2
TOL_GRAD_BF16 = 5e-2
NEAR_TIE = 1e-4   # rows whose K-th/(K+1)-th oracle score gap is below this are excluded


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_report(x, y):
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    rms = float(np.sqrt(np.mean(y * y))) if y.size else 0.0
    err = np.abs(x - y)
    elem = float(np.max(err / np.maximum(np.abs(y), 1e-30))) if y.size else 0.0
    norm = float(np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-30)) if y.size else 0.0
    return rms, elem, norm


def assert_close(x, y, tol, what=""):
    """Pass iff |x - y| <= tol*|y| + tol*rms(y) elementwise (allclose with atol = tol*rms(y))."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    assert x.shape == y.shape, (what, x.shape, y.shape)
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    rms, elem, norm = rel_report(x, y)
    bad = np.abs(x - y) > tol * np.abs(y) + tol * rms
    if bad.any():
        k = int(np.argmax(np.abs(x - y) - tol * np.abs(y)))
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{x.size} outside tol {tol} (rms {rms:.3g}, max elem rel "
            f"{elem:.3g}, normwise {norm:.3g}); worst flat index {k}: got {x.flat[k]!r} "
            f"want {y.flat[k]!r}")
    return elem, norm


def compare_selection(idx_gpu, idx_or, gap, K):
    """Bit-exact index sets on rows whose oracle gap is >= NEAR_TIE.

    Returns (excluded mask, equal mask). Rows with at most K candidates have gap = inf.
    """
    excl = gap < NEAR_TIE
    eq = np.all(idx_gpu == idx_or, axis=-1)
    bad = (~excl) & (~eq)
    if bad.any():
        w = np.argwhere(bad)[0]
        raise AssertionError(f"{int(bad.sum())} rows select different chunks; first {tuple(w)}: "
                             f"gpu {idx_gpu[tuple(w)]} oracle {idx_or[tuple(w)]} gap {gap[tuple(w)]}")
    return excl, eq
