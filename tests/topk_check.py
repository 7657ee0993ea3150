"""Checks of a selection against the fp64 definition of the score (CPU).

The scan's fp32 order is the library's own convention (the pages fix none),
so the bit-exact comparisons against the oracle's fp32 scores are backed by a
leg that does not depend on that order: every GPU score lies within the
tolerance band TOL * sum_j |q_hj khat_ij| of the fp64 definition (§3.2, §3.3),
and every returned index set is a top-k that scores inside those bands could
produce (§2: the k highest scores of the row).
"""
import numpy as np

TOL = 1e-4


def assert_scores_within_band(gpu, s64, l1, tol=TOL):
    """|S_gpu - S_fp64| <= tol * L1 for every score."""
    err = np.abs(np.asarray(gpu, dtype=np.float64) - s64)
    bad = err > tol * l1
    assert not bad.any(), "%d scores outside the band, worst ratio %.3g" % (
        int(bad.sum()), float(np.max(err / np.maximum(l1, 1e-300))))


def assert_topk_valid(idx, s64, l1, k, tol=TOL):
    """idx [rows][k]: ascending, distinct, in range, and a valid top-k of the
    fp64 scores up to the band: for every selected i and unselected u,
    s64_i + tol*l1_i >= s64_u - tol*l1_u (so no unselected key is certainly
    above a selected one)."""
    idx = np.asarray(idx)
    rows = idx.shape[0]
    s = np.asarray(s64, dtype=np.float64).reshape(rows, -1)
    b = tol * np.asarray(l1, dtype=np.float64).reshape(rows, -1)
    n = s.shape[1]
    assert idx.shape == (rows, k)
    for r in range(rows):
        sel = idx[r].astype(np.int64)
        assert np.all(sel >= 0) and np.all(sel < n), "row %d: index out of range" % r
        assert np.all(np.diff(sel) > 0), "row %d: indices not strictly ascending" % r
        if k == n:
            continue
        mask = np.ones(n, dtype=bool)
        mask[sel] = False
        low_sel = float(np.min(s[r, sel] + b[r, sel]))
        high_unsel = float(np.max(s[r, mask] - b[r, mask]))
        assert low_sel >= high_unsel, (
            "row %d: an unselected key scores above a selected one beyond the band "
            "(%.9g < %.9g)" % (r, low_sel, high_unsel))
