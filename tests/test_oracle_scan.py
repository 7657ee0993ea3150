"""Pins of the oracle's scan (CPU only).

Sources: "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV
Caches" §3.2 (prefix value; t = 4 is the full 4-bit value), §3.3 (channels
with t_j = 0 are skipped; cell-centre error at most half a cell), §2 (the
2-bit thumbnail is the uniform-depth special case).

Independent routes: the 4-bit dequantized keys rebuilt here from K with exact
rationals and a numpy fp64 dot product; the quantizer error bound; decode()
(pinned separately by the prefix invariant) times q.
"""
from fractions import Fraction

import numpy as np
import pytest

import fathom_inputs
import oracle


@pytest.fixture(scope="module")
def small():
    ins = fathom_inputs.make_inputs(2, 4, 64 * 6, seed=21)
    planes, scales, bad = oracle.encode(ins.k)
    assert bad == 0
    return ins, planes, scales


def _dequant4_direct(k):
    """4-bit values straight from K: (floor(k/s) clamped + 1/2) * s, s = a/8,
    with a the per-(block, channel) max |k|; exact rationals -> fp64."""
    groups, n, d = k.shape
    out = np.zeros((groups, n, d))
    for g in range(groups):
        for b in range(n // 64):
            blk = k[g, b * 64:(b + 1) * 64].astype(np.float64)
            a = np.abs(blk).max(axis=0)
            for j in range(d):
                if a[j] == 0:
                    continue
                s = Fraction(a[j]) / 8
                for i in range(64):
                    q = Fraction(blk[i, j]) / s
                    m = min(7, max(-8, q.numerator // q.denominator))
                    out[g, b * 64 + i, j] = float((m + Fraction(1, 2)) * s)
    return out


def test_full_depth_equals_full_4bit_dot(small):
    ins, planes, scales = small
    depths = np.full((2, 128), 4, dtype=np.uint8)
    s64, l1 = oracle.scan_f64(planes, scales, depths, ins.q, ins.k.shape[1])
    khat = _dequant4_direct(ins.k)
    ref = np.einsum("gnd,ghd->ghn", khat, ins.q.astype(np.float64))
    assert np.all(np.abs(s64 - ref) <= 1e-12 * l1)


def test_uniform_depth_matches_decoded_keys(small):
    """Thumbnail-style uniform depth t (t = 2 reads every channel at 2 bits)."""
    ins, planes, scales = small
    n = ins.k.shape[1]
    for t in (1, 2, 3):
        depths = np.full((2, 128), t, dtype=np.uint8)
        s64, l1 = oracle.scan_f64(planes, scales, depths, ins.q, n)
        dec = oracle.decode(planes, scales, n, t)
        ref = np.einsum("gnd,ghd->ghn", dec, ins.q.astype(np.float64))
        assert np.all(np.abs(s64 - ref) <= 1e-12 * l1)


def test_error_bound_and_skipped_channels(small):
    """|S_t - q.k| <= sum_{t_j>0} |q_j| a_j / 2^t_j + sum_{t_j=0} |q_j k_j|:
    a t-bit mid-rise cell has half-width a / 2^t; skipped channels contribute
    nothing."""
    ins, planes, scales = small
    n = ins.k.shape[1]
    rng = np.random.default_rng(22)
    k64 = ins.k.astype(np.float64)
    a = np.abs(k64.reshape(2, n // 64, 64, 128)).max(axis=2)          # [g][blk][d]
    for _ in range(5):
        depths = rng.integers(0, 5, size=(2, 128)).astype(np.uint8)
        s64, _ = oracle.scan_f64(planes, scales, depths, ins.q, n)
        exact = np.einsum("gnd,ghd->ghn", k64, ins.q.astype(np.float64))
        t = depths.astype(np.float64)[:, None, :]                      # [g][1][d]
        act = (depths > 0)[:, None, :]
        half = np.where(act, a / 2.0 ** t, 0.0)                        # [g][blk][d]
        half_tok = np.repeat(half, 64, axis=1)                         # [g][n][d]
        qa = np.abs(ins.q.astype(np.float64))
        bound = np.einsum("gnd,ghd->ghn", half_tok, qa)
        skipped = np.einsum("gnd,ghd->ghn", np.abs(k64) * (~act), qa)
        assert np.all(np.abs(s64 - exact) <= (bound + skipped) * (1 + 1e-9) + 1e-12)


def test_ref32_within_tolerance_of_fp64(small):
    """The fp32 evaluation order agrees with the fp64 definition within
    1e-4 relative to the L1 magnitude sum_j |q_j khat_j| (in practice far
    below)."""
    ins, planes, scales = small
    n = ins.k.shape[1]
    rng = np.random.default_rng(23)
    worst = 0.0
    for B in (0, 5, 48, 92, 136, 300, 512):
        depths, _, _ = oracle.plan(ins.q, ins.var, B)
        s32 = oracle.scan_ref32(planes, scales, depths, ins.q, n)
        s64, l1 = oracle.scan_f64(planes, scales, depths, ins.q, n)
        err = np.abs(s32.astype(np.float64) - s64)
        assert np.all(err <= 1e-4 * l1)
        worst = max(worst, float(np.max(err / np.maximum(l1, 1e-300))))
    depths = rng.integers(0, 5, size=(2, 128)).astype(np.uint8)
    s32 = oracle.scan_ref32(planes, scales, depths, ins.q, n)
    s64, l1 = oracle.scan_f64(planes, scales, depths, ins.q, n)
    assert np.all(np.abs(s32 - s64) <= 1e-4 * l1)
    assert worst < 1e-5


def test_zero_budget_scores_are_zero(small):
    ins, planes, scales = small
    n = ins.k.shape[1]
    depths = np.zeros((2, 128), dtype=np.uint8)
    s32 = oracle.scan_ref32(planes, scales, depths, ins.q, n)
    assert np.all(s32 == 0.0) and not np.any(np.signbit(s32))


def test_store_capacity_is_respected(small):
    """Scanning the first n tokens of a larger store equals scanning a store
    of exactly n tokens."""
    ins, planes, scales = small
    n = ins.k.shape[1]
    big_p = np.zeros((2, 128, 4, 10), dtype=np.uint64)
    big_s = np.zeros((2, 128, 10), dtype=np.uint16)
    big_p[..., :n // 64] = planes
    big_s[..., :n // 64] = scales
    depths, _, _ = oracle.plan(ins.q, ins.var, 92)
    a = oracle.scan_ref32(planes, scales, depths, ins.q, n)
    b = oracle.scan_ref32(big_p, big_s, depths, ins.q, n)
    assert np.array_equal(a, b)
