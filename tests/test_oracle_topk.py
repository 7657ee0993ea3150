"""Pins of the oracle's top-k (CPU only).

Source: "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV
Caches" §2 (top-k selected per query head by the method's score).  The tie
rule (lower index first) and the ascending output are this library's
definition.  Checks: the defining order property, numpy's lexsort as an
independent library route, and degenerate inputs.
"""
import numpy as np
import pytest

import fathom_inputs
import oracle


def _check_property(scores, k, idx):
    rows, n = scores.shape
    for r in range(rows):
        sel = idx[r]
        assert len(sel) == k
        assert np.all(np.diff(sel) > 0)                # ascending, unique
        mask = np.zeros(n, dtype=bool)
        mask[sel] = True
        s = scores[r].astype(np.float64)
        if k == n:
            continue
        # worst selected vs best unselected under (score desc, index asc)
        worst_s = s[mask].min()
        worst_i = sel[s[sel] == worst_s].max()
        best_s = s[~mask].max()
        best_i = np.flatnonzero((~mask) & (s == best_s)).min()
        assert worst_s > best_s or (worst_s == best_s and worst_i < best_i)


def _lexsort_topk(scores, k):
    out = []
    for row in scores:
        order = np.lexsort((np.arange(len(row)), -row.astype(np.float64)))
        out.append(np.sort(order[:k]))
    return np.array(out, dtype=np.int32)


@pytest.mark.parametrize("kind", ["normal", "ties", "const", "signed_zero"])
def test_topk_property_and_lexsort(kind):
    scores = fathom_inputs.random_scores(6, 3000, seed=31, kind=kind)
    for k in (1, 7, 64, 1000, 2999, 3000):
        idx = oracle.topk(scores, k)
        _check_property(scores, k, idx)
        assert np.array_equal(idx, _lexsort_topk(scores, k))


def test_all_equal_scores_take_lowest_indices():
    """A zero budget gives every key score 0: the top-k is {0..k-1}."""
    scores = np.zeros((3, 1000), dtype=np.float32)
    scores[1] = -0.0
    idx = oracle.topk(scores, 10)
    assert np.array_equal(idx, np.tile(np.arange(10, dtype=np.int32), (3, 1)))


def test_duplicate_scores_across_blocks():
    rng = np.random.default_rng(32)
    s = rng.standard_normal((2, 4096)).astype(np.float32)
    s[:, [5, 700, 1400, 3000, 4095]] = np.float32(10.0)
    s[:, [6, 701]] = np.float32(9.0)
    idx = oracle.topk(s, 6)
    assert list(idx[0]) == [5, 6, 700, 1400, 3000, 4095]
    idx = oracle.topk(s, 3)
    assert list(idx[0]) == [5, 700, 1400]


def test_validity_check_accepts_exact_and_rejects_swaps():
    """The fp64 validity check used by the GPU parity tests: the oracle's own
    top-k of fp64-close scores passes; swapping one selected index for a
    clearly lower-scoring key fails; a duplicate or unsorted set fails."""
    import pytest
    from topk_check import assert_topk_valid
    rng = np.random.default_rng(5)
    rows, n, k = 3, 5000, 100
    s64 = rng.standard_normal((rows, n))
    l1 = np.abs(s64) + 1.0
    s32 = s64.astype(np.float32)
    idx = oracle.topk(s32, k)
    assert_topk_valid(idx, s64, l1, k)
    bad = idx.copy()
    worst = int(np.argmin(s64[0]))
    bad[0, 0] = worst
    bad[0] = np.sort(bad[0])
    with pytest.raises(AssertionError):
        assert_topk_valid(bad, s64, l1, k)
    dup = idx.copy()
    dup[1, 1] = dup[1, 0]
    with pytest.raises(AssertionError):
        assert_topk_valid(dup, s64, l1, k)
    rev = idx[:, ::-1].copy()
    with pytest.raises(AssertionError):
        assert_topk_valid(rev, s64, l1, k)
