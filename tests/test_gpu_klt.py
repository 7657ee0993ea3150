"""GPU parity of the KLT-rotated store (fathom_klt_fit, fathom_klt_rotate_keys,
fathom_klt_rotate_queries) against the CPU oracle.

The fit is an eigendecomposition, so it is compared within tolerances: the
mean to fp32 rounding, eigenvalues within 1e-5 of the largest, eigenvectors
through orthonormality, the residual C V - V Lambda against the oracle's fp64
covariance, and column by column where the eigenvalue gap makes a column
well defined; on the planted basis of closed-form eigenpairs, directly.  The
rotations are bit-exact (fixed fp32 fold order, binary16 nearest-even); the
rotated store then runs encode, plan, scan and top-k with the same bit-exact
parity as the raw store.
"""
import numpy as np
import pytest

import fathom_inputs
import oracle
from gpu_util import first_mismatch, say, to_dev, to_host
from topk_check import assert_scores_within_band, assert_topk_valid
from klt_cases import D, expected_basis, planted

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import sparse_top_kv_fathom_amd as fk
    fk.lib()
    return fk


def _fit(fk, k):
    import torch
    mu, V, lam = fk.klt_fit(to_dev(k))
    torch.cuda.synchronize()
    return to_host(mu), to_host(V), to_host(lam)


def test_fit_planted(fk):
    """Closed-form eigenpairs: mean mu0, eigenvalues 4 sigma_j^2 / (n - 1)
    descending, eigenvectors the columns of the block-Hadamard R."""
    k, mu0, R, sigma = planted(seed=5)
    n = k.shape[1]
    say("klt fit planted n=%d" % n)
    mu, V, lam = _fit(fk, k)
    assert np.array_equal(mu[0], mu0.astype(np.float32))
    le = np.sort(4 * sigma ** 2 / (n - 1))[::-1]
    assert np.all(np.abs(lam[0] - le) <= 1e-6 * le[0] + 2.0 ** -23 * le)
    Ve = expected_basis(R, sigma)
    assert np.max(np.abs(V[0].astype(np.float64) - Ve)) < 1e-5


@pytest.mark.parametrize("groups,n", [(3, 64 * 70), (2, 64 * 1000), (1, 64), (5, 64 * 33)])
def test_fit_matches_oracle(fk, groups, n):
    ins = fathom_inputs.make_inputs(groups, 4, n, seed=900 + groups)
    say("klt fit groups=%d n=%d" % (groups, n))
    mu, V, lam = _fit(fk, ins.k)
    rmu, rV, rlam = oracle.klt_fit(ins.k)
    for g in range(groups):
        x = ins.k[g].astype(np.float64)
        amax = np.abs(x).max()
        assert np.all(np.abs(mu[g] - rmu[g]) <= 2.0 ** -24 * np.abs(rmu[g]) + 1e-12 * amax)
        lmax = rlam[g][0]
        assert np.all(np.abs(lam[g] - rlam[g]) <= 1e-5 * lmax), np.max(np.abs(lam[g] - rlam[g]))
        Vg = V[g].astype(np.float64)
        assert np.max(np.abs(Vg.T @ Vg - np.eye(D))) < 1e-5
        if n > 1:
            xc = x - rmu[g]
            C = (xc.T @ xc) / (n - 1)
            assert np.max(np.abs(C @ Vg - Vg * rlam[g])) < 1e-5 * lmax
        # columns whose eigenvalue is separated from the others by >= 1% of
        # the largest are determined up to the sign rule: compare them
        gaps = np.array([np.min(np.abs(np.delete(rlam[g], j) - rlam[g][j])) for j in range(D)])
        for j in np.flatnonzero(gaps >= 1e-2 * lmax):
            assert np.max(np.abs(Vg[:, j] - rV[g][:, j])) < 1e-3, (g, j)


@pytest.mark.parametrize("groups,n", [(2, 64 * 37), (1, 64), (3, 64 * 16)])
def test_rotations_bit_exact(fk, groups, n):
    """Rotated keys and queries equal the oracle's folds bit for bit, with
    the basis the GPU fitted (several 16-tile workgroups plus a ragged one)."""
    import torch
    ins = fathom_inputs.make_inputs(groups, 4, n, seed=950 + n)
    say("klt rotate groups=%d n=%d" % (groups, n))
    mu_d, V_d, lam_d = fk.klt_fit(to_dev(ins.k))
    kr = fk.klt_rotate_keys(to_dev(ins.k), mu_d, V_d)
    qr = fk.klt_rotate_queries(to_dev(ins.q), V_d)
    torch.cuda.synchronize()
    mu, V = to_host(mu_d), to_host(V_d)
    ref = oracle.klt_rotate_keys(ins.k, mu, V)
    got = to_host(kr)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16)), first_mismatch(got, ref)
    rq = oracle.klt_rotate_queries(ins.q, V)
    gq = to_host(qr)
    assert np.array_equal(gq.view(np.uint32), rq.view(np.uint32)), first_mismatch(gq, rq)


def test_rotated_store_end_to_end(fk):
    """fit -> rotate keys -> encode; rotate queries -> plan(q V, lambda) ->
    scan -> top-k, every stage bit-exact against the oracle run on the GPU's
    inputs to that stage."""
    import torch
    groups, G, n, B, k = 2, 4, 64 * 100, 92, 128
    ins = fathom_inputs.make_inputs(groups, G, n, seed=977)
    say("klt end to end groups=%d n=%d B=%d k=%d" % (groups, n, B, k))
    mu_d, V_d, lam_d = fk.klt_fit(to_dev(ins.k))
    kr_d = fk.klt_rotate_keys(to_dev(ins.k), mu_d, V_d)
    planes_d, scales_d = fk.encode(kr_d)
    qr_d = fk.klt_rotate_queries(to_dev(ins.q), V_d)
    dep_d = fk.plan(qr_d, lam_d, B)
    sc_d = fk.scan(planes_d, scales_d, dep_d, qr_d, n)
    idx_d = fk.topk(sc_d, k)
    torch.cuda.synchronize()
    kr, lam, qr = to_host(kr_d), to_host(lam_d), to_host(qr_d)
    planes, scales, _ = oracle.encode(kr)
    assert np.array_equal(to_host(planes_d), planes)
    assert np.array_equal(to_host(scales_d), scales)
    depths, _, _ = oracle.plan(qr, lam, B)
    assert np.array_equal(to_host(dep_d), depths)
    ref = oracle.scan_ref32(planes, scales, depths, qr, n)
    sc = to_host(sc_d)
    assert np.array_equal(sc.view(np.uint32), ref.view(np.uint32)), first_mismatch(sc, ref)
    gi = to_host(idx_d)
    assert np.array_equal(gi, oracle.topk(ref.reshape(groups * G, n), k))
    s64, l1 = oracle.scan_f64(planes, scales, depths, qr, n)
    assert_scores_within_band(sc, s64, l1)
    assert_topk_valid(gi, s64, l1, k)
