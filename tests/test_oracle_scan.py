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


# ---------------------------------------------------------------------------
# The fp32 evaluation order of scan_ref32, pinned by exact rational arithmetic
# ---------------------------------------------------------------------------
# The pages fix the score (§3.2 prefix value, §3.3 active channels) but no
# fp32 order; the library states one (fathom.h: U over fma(w, m) and o over
# fma(e, a), each folded from +0 over the active channels deepest first and
# by ascending index within a depth, then S = fl32(U + o)).  Here that order
# is re-derived with Python Fractions, every fp32 step rounded to nearest-even
# by hand below, so the oracle's bits are checked by a route that shares no
# floating-point arithmetic with it.  Cases are chosen where other orders (one
# ascending-index fold, or U and o in one accumulator) round differently, so
# a change of order fails here.

def _r32(x: Fraction) -> Fraction:
    """x rounded to the nearest binary32 value, ties to even (normal and
    subnormal range; the cases here stay far from overflow)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    m = a / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    assert r < Fraction(2) ** 128
    return sign * r


def _fma32(a: Fraction, b: Fraction, c: Fraction) -> Fraction:
    return _r32(a * b + c)


def _f16(bits: int) -> Fraction:
    """binary16 bit pattern -> exact rational (finite values only)."""
    e, m = (bits >> 10) & 0x1F, bits & 0x3FF
    assert e != 0x1F
    v = Fraction(m, 1 << 24) if e == 0 else Fraction(m | 0x400, 1 << 10) * Fraction(2) ** (e - 15)
    return -v if bits & 0x8000 else v


def _prefix(planes, g, j, b, i, t):
    c = 0
    for p in range(t):
        c = 2 * c + int((int(planes[g, j, p, b]) >> i) & 1)
    return c


def _scores_by_order(planes, scales, depths, q, n, order_kind):
    """Scores of token range [0, n) with the U/o split, folds in the given
    channel order: 'stated' (depth 4, 3, 2, 1; ascending within a depth),
    'ascending' (one ascending-index fold), or 'one_acc' (the stated order
    with U and o in one accumulator started at o)."""
    groups, G, d = q.shape
    out = np.zeros((groups, G, n), dtype=np.float64)
    for g in range(groups):
        t = [min(int(x), 4) for x in depths[g]]
        if order_kind == "ascending":
            order = [j for j in range(d) if t[j] > 0]
        else:
            order = [j for dep in (4, 3, 2, 1) for j in range(d) if t[j] == dep]
        for b in range(n // 64):
            for h in range(G):
                qh = [Fraction(float(x)) for x in q[g, h]]
                o = Fraction(0)
                for j in order:
                    e = _r32(qh[j] * (Fraction(1, 2 ** t[j]) - 1))
                    o = _fma32(e, _f16(int(scales[g, j, b])), o)
                for i in range(64):
                    u = o if order_kind == "one_acc" else Fraction(0)
                    for j in order:
                        w = qh[j] * Fraction(2) ** (11 - t[j])
                        m = _f16(int(scales[g, j, b])) * _prefix(planes, g, j, b, i, t[j]) \
                            * Fraction(1, 1024)
                        u = _fma32(w, m, u)
                    s = u if order_kind == "one_acc" else _r32(u + o)
                    out[g, h, b * 64 + i] = float(s)
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_ref32_order_pinned_by_exact_arithmetic(seed):
    rng = np.random.default_rng(400 + seed)
    G, n = 2, 128
    ins = fathom_inputs.make_inputs(1, G, n, seed=410 + seed)
    planes, scales, _ = oracle.encode(ins.k)
    depths = np.zeros((1, 128), dtype=np.uint8)
    chans = rng.choice(128, 12, replace=False)
    depths[0, chans] = rng.permutation([4, 4, 3, 3, 3, 2, 2, 2, 1, 1, 1, 1])
    depths[0, rng.choice(np.setdiff1d(np.arange(128), chans), 1)] = 7   # reads as 4
    got = oracle.scan_ref32(planes, scales, depths, ins.q, n).astype(np.float64)
    want = _scores_by_order(planes, scales, depths, ins.q, n, "stated")
    assert np.array_equal(got, want)
    # the test can tell the stated order from the others
    for other in ("ascending", "one_acc"):
        alt = _scores_by_order(planes, scales, depths, ins.q, n, other)
        assert np.count_nonzero(alt != want) > 0, other
