"""Helpers shared by the GPU parity tests (tolerances, near-tie bookkeeping)."""
from __future__ import annotations

import re
import sys

import numpy as np

import oracle

# Output tolerances: float32 paths (and every float32 intermediate: summaries,
# scores, log-sum-exps) 1e-4; bf16 outputs 2e-2; bf16 gradients 5e-2.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2
TOL_GRAD_BF16 = 5e-2
NEAR_TIE = 1e-4   # rows whose K-th/(K+1)-th oracle score gap is below this are excluded
# elements at least this many rms(y) in magnitude must also meet the tolerance as a
# plain relative error |x - y| / |y| (below it, relative error is dominated by
# cancellation in y and the allclose form governs)
REL_FLOOR_RMS = 1.0


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


# Quantities that are vectors per row (the last axis is the head dimension): an
# output row O_i, a gradient row, a summary key. Rows attend to different numbers
# of keys and their magnitudes differ by an order of magnitude, so their absolute
# floor is the larger of the rms of the row's own vector and the array's rms (a row
# much larger than the rest is judged at its own scale; a row made small by
# cancellation, e.g. the gradient of a peaked softmax, at the array's); per-row
# scalars (scores, log-sum-exps) use the array's rms.
_VECTOR = re.compile(r"^(decode )?(O|dQ|dK|dV|dQl|dQs|ksum)\b")


def assert_close(x, y, tol, what="", rel_floor=REL_FLOOR_RMS):
    """Pass iff |x - y| <= tol*|y| + tol*rms elementwise (allclose with atol = tol*rms), and
    |x - y| <= tol*|y| on every element with |y| >= rel_floor * rms; rms is the larger of
    the element's row rms and the array's for vector quantities (see _VECTOR), else the
    array's."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    assert x.shape == y.shape, (what, x.shape, y.shape)
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    rms_all, elem, norm = rel_report(x, y)
    if y.ndim >= 2 and _VECTOR.match(what):
        rms = np.maximum(np.sqrt(np.mean(y * y, axis=-1, keepdims=True)), rms_all)
    else:
        rms = rms_all
    bad = np.abs(x - y) > tol * np.abs(y) + tol * rms
    if bad.any():
        k = int(np.argmax(np.abs(x - y) - tol * np.abs(y)))
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{x.size} outside tol {tol} (rms {rms_all:.3g}, max elem rel "
            f"{elem:.3g}, normwise {norm:.3g}); worst flat index {k}: got {x.flat[k]!r} "
            f"want {y.flat[k]!r}")
    big = (np.abs(y) >= rel_floor * np.broadcast_to(rms, y.shape)) & (y != 0)
    if big.any():
        rel = np.abs(x - y)[big] / np.abs(y)[big]
        if rel.max() > tol:
            k = int(np.argmax(rel))
            raise AssertionError(
                f"{what}: {int((rel > tol).sum())}/{int(big.sum())} elements with |y| >= "
                f"{rel_floor} rms exceed relative error {tol} (max {rel.max():.3g}); got "
                f"{x[big][k]!r} want {y[big][k]!r}")
    return elem, norm


def all_scores(Q, ksum, ent, S, rows, q_pos0=0, group_hkv=None, window=0):
    """Oracle chunk scores of every candidate of the listed rows (flattened (b*Tq+i)*H+h
    indices) -> [len(rows), NC], -inf for chunks that are not candidates. With group_hkv
    the score is the group maximum over the kv head's query heads (the group-max order key)."""
    B, Tq, H, d = Q.shape
    NC = ksum.shape[1]
    rows = np.asarray(rows, np.int64)
    if group_hkv is not None:
        G = H // group_hkv
        h = rows % H
        base = rows - h + (h // G) * G
        per = [all_scores(Q, ksum, ent, S, base + x, q_pos0, None, window) for x in range(G)]
        return np.max(np.stack(per), axis=0)
    idx, sc, _ = oracle.score_topk(Q, ksum, ent, S, NC, q_pos0=q_pos0, rows=rows, window=window)
    out = np.full((rows.size, NC), -np.inf)
    fi, fs = idx.reshape(-1, NC)[rows], sc.reshape(-1, NC)[rows]
    for n in range(rows.size):
        m = fi[n] >= 0
        out[n, fi[n][m]] = fs[n][m]
    return out


def check_band(gsel, scores, K, tol=NEAR_TIE):
    """A selection within the near-tie band: gsel [n, K] GPU ids (-1 padded), scores [n, NC]
    oracle scores (-inf: not a candidate). Every selected chunk scores at least the K-th
    best minus tol, every unselected candidate at most the (K+1)-th best plus tol, and the
    set holds min(K, candidates) distinct candidates."""
    for n in range(gsel.shape[0]):
        s = scores[n]
        cand = np.isfinite(s)
        nc = int(cand.sum())
        sel = gsel[n][gsel[n] >= 0]
        assert sel.size == min(K, nc) and np.unique(sel).size == sel.size, (n, sel)
        assert np.all(cand[sel]), (n, sel)
        order = np.sort(s[cand])[::-1]
        sk = order[min(K, nc) - 1]
        sk1 = order[K] if nc > K else -np.inf
        assert np.all(s[sel] >= sk - tol), (n, sel, s[sel], sk)
        rest = cand.copy()
        rest[sel] = False
        assert np.all(s[rest] <= sk1 + tol), (n, s[rest].max(), sk1)


def compare_selection(idx_gpu, idx_or, gap, K, scores_fn=None):
    """Bit-exact index sets on rows whose oracle gap is >= NEAR_TIE.

    Rows below the gap (excluded, counted) whose GPU set differs are checked to be a
    valid top-K within the band when scores_fn is given: scores_fn(flat row numbers of
    those rows within idx_gpu) -> oracle scores [n, NC] (see all_scores, check_band).
    Returns (excluded mask, equal mask). Rows with at most K candidates have gap = inf.
    """
    excl = gap < NEAR_TIE
    eq = np.all(idx_gpu == idx_or, axis=-1)
    bad = (~excl) & (~eq)
    if bad.any():
        w = np.argwhere(bad)[0]
        raise AssertionError(f"{int(bad.sum())} rows select different chunks; first {tuple(w)}: "
                             f"gpu {idx_gpu[tuple(w)]} oracle {idx_or[tuple(w)]} gap {gap[tuple(w)]}")
    differ = np.flatnonzero((excl & ~eq).reshape(-1))
    if differ.size:
        assert scores_fn is not None, "near-tie rows differ and no oracle scores were given"
        check_band(idx_gpu.reshape(-1, K)[differ], scores_fn(differ), K)
    return excl, eq
