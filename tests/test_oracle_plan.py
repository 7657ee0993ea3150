"""Pins of the oracle's planner (CPU only).

Sources: "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV
Caches" §3.3 (importance g_j, error g_j 4^-t_j, Eq. 4, 30-step bisection for
the smallest theta that fits) and the Appendix A walkthrough on the jaehun.me
review page (printed g, depths at theta = 0.1 / 0.01, B = 8 and B = 6 plans).

Independent routes used here: the literal Eq. 4 with a logarithm, brute force
over all 5^d integer plans for small d, and the breakpoint characterisation
of the step function sum_j t_j(theta).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import fathom_inputs
import oracle


@pytest.fixture(scope="module")
def gold(golden_dir):
    return json.load(open(os.path.join(golden_dir, "appendix_a.json")))


def _toy_g(gold):
    q = np.array([gold["q_A"], gold["q_B"]], dtype=np.float32)
    var = np.array(gold["var"], dtype=np.float32)
    return oracle.importance(q, var)


def test_appendix_a_importance(gold):
    g = _toy_g(gold)
    for j in range(4):
        assert abs(g[j] - gold["g_printed"][j]) <= gold["g_printed_tolerance"][j]
    # exact values behind the printed roundings: (9+1)*1.222, (1+4)*0.755, ...
    assert g[0] == pytest.approx(12.22, rel=1e-6)
    assert g[1] == pytest.approx(3.775, rel=1e-6)
    assert g[2] == pytest.approx(0.635, rel=1e-6)
    assert g[3] == pytest.approx(5e-5, rel=1e-5)


def test_appendix_a_depths_at_theta(gold):
    g = _toy_g(gold)
    for row in gold["depths_at_theta"]:
        t, s = oracle.depths_at(g, row["theta"])
        assert list(t) == row["depths"] and s == row["bits"]


def test_appendix_a_plans_toy_bracket(gold):
    g = _toy_g(gold)
    lo, hi = gold["bracket"]
    for row in gold["plans"]:
        t, theta, bits = oracle.bisect(g, row["budget"], lo, hi, 30)
        assert list(t) == row["depths"]
        if "bits" in row:
            assert bits == row["bits"]
        if "theta_printed" in row:
            # the page prints 0.079; the exact water line is the 9th breakpoint
            # g_2 / 8 = 0.079375 approached from above
            assert abs(theta - row["theta_printed"]) < 1e-3
            assert theta >= float(np.float64(g[2]) / 8)


def test_appendix_a_general_bracket_agrees(gold):
    g = _toy_g(gold)
    lo, hi = gold["bracket"]
    for B in (6, 7, 8, 11):
        t1, _, _ = oracle.bisect(g, B, lo, hi, 30)
        t2, _, b2 = oracle.plan_group(g, B)
        assert list(t1) == list(t2)
        assert b2 <= B
    assert list(oracle.plan_group(g, 7)[0]) == [3, 3, 1, 0]
    assert list(oracle.plan_group(g, 11)[0]) == [4, 4, 3, 0]


def test_variance_reading_is_sample_variance(gold):
    """Appendix A's Var for channel 2 (0.127) is the ddof = 1 variance of the
    six printed channel-2 values (ddof = 0 would give 0.106)."""
    v = np.array(gold["channel2_values"], dtype=np.float16).reshape(1, 6, 1)
    var = fathom_inputs.channel_variance(v)[0, 0]
    assert abs(var - gold["var"][2]) < 5e-4


def test_depth_rule_matches_literal_eq4():
    """t = clip(round(log4(g/theta)), 0, 4) computed with a logarithm equals the
    threshold form, away from exact half-way points."""
    rng = np.random.default_rng(5)
    n_checked = 0
    for _ in range(20000):
        g = 10 ** rng.uniform(-6, 6)
        theta = 10 ** rng.uniform(-6, 6)
        x = math.log(g / theta) / math.log(4.0)
        if abs((x + 0.5) - round(x + 0.5)) < 1e-9:
            continue
        lit = min(4, max(0, math.floor(x + 0.5)))
        assert oracle.depth_one(g, theta) == lit
        n_checked += 1
    assert n_checked > 19000
    assert oracle.depth_one(0.0, 1.0) == 0


def _objective(g, t):
    return float(sum(gj * 4.0 ** (-int(tj)) for gj, tj in zip(g, t)))


@pytest.mark.parametrize("d", [3, 4, 5, 6])
def test_brute_force_optimum(d):
    """§3.3: the plan minimises sum_j g_j 4^-t_j subject to sum_j t_j <= B;
    brute force over all 5^d integer plans."""
    rng = np.random.default_rng(10 + d)
    plans = np.array(list(itertools.product(range(5), repeat=d)), dtype=np.int64)
    sums = plans.sum(axis=1)
    for trial in range(30 if d < 6 else 8):
        g = 10 ** rng.uniform(-3, 3, d)
        if trial % 5 == 0:
            g[rng.integers(d)] = 0.0
        cost = (g[None, :] * 4.0 ** (-plans)).sum(axis=1)
        for B in range(0, 4 * d + 1):
            best = cost[sums <= B].min()
            t, _, bits = oracle.plan_group(g, B)
            assert bits <= B
            assert _objective(g, t) == pytest.approx(best, rel=1e-12, abs=1e-300)


def test_breakpoint_closed_form():
    """sum_j t_j(theta) counts the breakpoints g_j / 2^(2m-1) >= theta, so the
    plan is the B largest breakpoints when breakpoints B and B+1 are apart."""
    rng = np.random.default_rng(7)
    for _ in range(50):
        d = 128
        g = np.exp(rng.standard_normal(d) * 2) * rng.uniform(0.5, 2)
        bp = sorted(((g[j] / 2.0 ** (2 * m - 1), j) for j in range(d) for m in range(1, 5)),
                    reverse=True)
        for B in (1, 17, 48, 68, 92, 136, 300, 511):
            if bp[B - 1][0] / bp[B][0] - 1 < 1e-6:
                continue
            expect = np.zeros(d, dtype=np.int64)
            for _, j in bp[:B]:
                expect[j] += 1
            t, theta, bits = oracle.plan_group(g, B)
            assert np.array_equal(t.astype(np.int64), expect)
            assert bits == B
            assert bp[B][0] < theta <= bp[B - 1][0] * (1 + 1e-12)


def test_sum_of_depths_is_monotone_in_theta():
    rng = np.random.default_rng(8)
    g = np.exp(rng.standard_normal(128) * 2)
    thetas = np.geomspace(g.min() / 1000, g.max() * 10, 2000)
    sums = [oracle.depths_at(g, th)[1] for th in thetas]
    assert all(a >= b for a, b in zip(sums, sums[1:]))
    assert sums[0] == 512 and sums[-1] == 0


def test_special_cases():
    g = np.array([3.0, 0.0, 1.0, 0.5], dtype=np.float64)
    t, theta, bits = oracle.plan_group(g, 0)
    assert list(t) == [0, 0, 0, 0] and bits == 0
    t, theta, bits = oracle.plan_group(g, 12)          # = 4 * #{g > 0}
    assert list(t) == [4, 0, 4, 4] and bits == 12
    t, theta, bits = oracle.plan_group(g, 16)
    assert list(t) == [4, 0, 4, 4] and bits == 12
    t, theta, bits = oracle.plan_group(np.zeros(5), 7)
    assert list(t) == [0] * 5 and bits == 0 and theta == 0.0


def test_plan_batch_matches_group_plans():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((5, 4, 128)).astype(np.float32)
    var = np.exp(rng.standard_normal((5, 128))).astype(np.float32)
    depths, theta, bits = oracle.plan(q, var, 92)
    for i in range(5):
        g = oracle.importance(q[i], var[i])
        t, th, b = oracle.plan_group(g, 92)
        assert np.array_equal(depths[i], t) and theta[i] == th and bits[i] == b


def test_active_channels_at_48_bits_soft_check():
    """§3.3 / Tab. 21: at 48 code bits a read touches 30-34 of 128 channels on
    the models measured.  The synthetic recipe lands nearby (soft check)."""
    ins = fathom_inputs.make_inputs(8, 4, 4096, seed=11)
    depths, _, bits = oracle.plan(ins.q, ins.var, 48)
    active = (depths > 0).sum(axis=1).mean()
    assert np.all(bits <= 48)
    assert 20 <= active <= 40, active


# --------------------------------------------------------------------------
# Fixed-depth plans (§2 comparison points)
# --------------------------------------------------------------------------

def test_thumbnail_reads_288_bits_per_token():
    """The 2-bit thumbnail reads all 128 channels at two planes: 256 code bits
    plus the 16-bit scale per 64 tokens of each channel = 288 bits (§2)."""
    t = oracle.plan_fixed("uniform", 2, groups=3)
    assert t.shape == (3, 128) and (t == 2).all()
    code = int(t[0].astype(int).sum())
    assert code + 128 * 16 // 64 == 288


@pytest.mark.parametrize("r,total", [(16, 68), (32, 136)])
def test_sparq_budgets_are_the_pages_68_and_136_bits(r, total):
    """r channels at 4 bits plus their scales: 68 and 136 bits per token, the
    scan widths of the pages' Table 1 comparison."""
    q = np.random.default_rng(r).standard_normal((2, 4, 128)).astype(np.float32)
    t = oracle.plan_fixed("sparq", r, q=q)
    assert ((t == 4).sum(axis=1) == r).all() and ((t == 0) | (t == 4)).all()
    assert 4 * r + r * 16 // 64 == total


def test_sparq_selects_largest_head_sums():
    """|q_hj| grows with j in every head, so the top r are the last r channels."""
    G, d = 4, 128
    base = np.arange(1, d + 1, dtype=np.float32)
    q = np.stack([base * (h + 1) * (-1) ** h for h in range(G)])[None]
    t = oracle.plan_fixed("sparq", 10, q=q)
    assert (np.nonzero(t[0])[0] == np.arange(d - 10, d)).all()


def test_sparq_ties_take_lower_channels():
    q = np.ones((1, 4, 128), dtype=np.float32)
    q[0, :, 64:] = -1.0                     # |q| equal everywhere
    t = oracle.plan_fixed("sparq", 7, q=q)
    assert (np.nonzero(t[0])[0] == np.arange(7)).all()


def test_topstat_brute_force_small():
    """Against the best r-subset found by enumeration (d = 8): the largest sum,
    and among equal sums the lexicographically smallest index set."""
    import itertools
    rng = np.random.default_rng(5)
    for trial in range(40):
        d = 8
        stat = rng.integers(0, 4, size=(1, d)).astype(np.float32)   # many ties
        for r in range(d + 1):
            t = oracle.plan_fixed("topstat", r, stat=stat, d=d)
            best = max(itertools.combinations(range(d), r),
                       key=lambda c: (sum(stat[0, list(c)]), [-i for i in c]))
            assert sorted(np.nonzero(t[0])[0].tolist()) == sorted(best), (trial, r)
