"""Pins of the oracle's KLT-rotated store (§3.5 of "Fathom: Per-Query Read
Depth for Sparse Decoding over Offloaded KV Caches"; the calibration-free fit
of its Appendix D).

The fit is pinned on a planted basis whose covariance is known exactly: keys
+-sigma_j R[:, j] around a dyadic mean, with R a permuted block-Hadamard
rotation (entries 0 and +-1/2), so the mean, the eigenvalues 4 sigma_j^2 /
(n - 1), the eigenvectors (the columns of R), their order and their signs are
all known in closed form.  The rotation folds are pinned by exact cases
(identity, the planted basis, where every product and sum is exact) and by
the fp32 error bound against an fp64 product on random data; the rotated
store end to end by the score identity q.(k - mu) = (qV).((k - mu)V).
"""
import numpy as np
import pytest

import fathom_inputs
import oracle

from klt_cases import D, expected_basis, planted


def test_fit_planted_basis():
    k, mu0, R, sigma = planted()
    n = k.shape[1]
    mu, V, lam = oracle.klt_fit(k)
    assert np.array_equal(mu[0], mu0)
    le = np.sort(4 * sigma ** 2 / (n - 1))[::-1]
    assert np.allclose(lam[0], le, rtol=1e-12, atol=1e-13 * le[0])     # eigh: ~eps * |C|
    Ve = expected_basis(R, sigma)
    assert np.max(np.abs(V[0] - Ve)) < 1e-10


def test_fit_invariants_random():
    ins = fathom_inputs.make_inputs(2, 4, 4096, seed=11)
    mu, V, lam = oracle.klt_fit(ins.k)
    for g in range(2):
        x = ins.k[g].astype(np.float64)
        C = np.cov(x, rowvar=False, ddof=1)
        assert np.allclose(mu[g], x.mean(axis=0), rtol=0, atol=1e-12 * np.abs(x).max())
        assert np.max(np.abs(V[g].T @ V[g] - np.eye(D))) < 1e-12
        assert np.max(np.abs(C @ V[g] - V[g] * lam[g])) < 1e-10 * lam[g][0]
        assert np.all(np.diff(lam[g]) <= 0) and np.all(lam[g] >= 0)
        assert abs(lam[g].sum() - np.trace(C)) < 1e-10 * np.trace(C)
        # the channel variances the raw store plans with are C's diagonal
        assert np.allclose(np.diag(C), ins.var[g].astype(np.float64), rtol=1e-6)


def test_fit_sign_and_order_rule():
    """Order by eigenvalue descending; sign by the first component of
    magnitude >= 1/(2 sqrt(d)) = 1/4 at d = 4, not by the largest one."""
    lam = np.array([1.0, 3.0, 2.0, -1e-18])
    E = np.array([[0.2, 0.0, -0.8, 0.0], [-0.6, 0.0, -0.6, 0.1],
                  [0.0, -1.0, 0.0, 0.0], [0.77459666924148, 0.0, 0.0, -0.99498743710662]])
    l2, V2 = oracle.klt_order_and_sign(lam, E)
    assert list(l2) == [3.0, 2.0, 1.0, 0.0]
    assert np.array_equal(V2[:, 0], [0, 0, 1, 0])
    assert np.array_equal(V2[:, 1], [0.8, 0.6, 0, 0])
    assert np.array_equal(V2[:, 2], [-0.2, 0.6, 0, -0.77459666924148])
    assert np.array_equal(V2[:, 3], [0, -0.1, 0, 0.99498743710662])


def test_rotate_identity():
    ins = fathom_inputs.make_inputs(2, 4, 256, seed=12)
    eye = np.broadcast_to(np.eye(D, dtype=np.float32), (2, D, D))
    zero = np.zeros((2, D), np.float32)
    kr = oracle.klt_rotate_keys(ins.k, zero, eye)
    assert np.array_equal(kr.astype(np.float32), ins.k.astype(np.float32))   # -0 reads +0
    qr = oracle.klt_rotate_queries(ins.q, eye)
    assert np.array_equal(qr, ins.q)


def test_rotate_planted_exact():
    """On the planted keys every product and partial sum of the fold is a
    short dyadic number, so the rotated keys are exactly +-sigma_j on one
    coordinate and 0 elsewhere."""
    k, mu0, R, sigma = planted(seed=3)
    Ve = expected_basis(R, sigma)
    kr = oracle.klt_rotate_keys(k, mu0[None].astype(np.float32), Ve[None].astype(np.float32))
    exact = (k[0].astype(np.float64) - mu0) @ Ve
    assert np.array_equal(kr[0].astype(np.float64), exact)
    nz = (exact != 0).sum(axis=1)
    assert np.all(nz == 1)


def test_rotate_error_bound_random():
    """fp32 fold within (d + 2) * 2^-24 * sum_c |k_c - mu_c| |V_cj| of the fp64
    product; the binary16 result within half an ulp of the fp32 fold."""
    ins = fathom_inputs.make_inputs(1, 4, 512, seed=13)
    mu, V, lam = oracle.klt_fit(ins.k)
    mu32, V32 = mu.astype(np.float32), V.astype(np.float32)
    raw = oracle.klt_rotate_keys(ins.k, mu32, V32, raw=True)[0].astype(np.float64)
    xc = ins.k[0].astype(np.float64) - mu32[0].astype(np.float64)
    exact = xc @ V32[0].astype(np.float64)
    bound = (D + 2) * 2.0 ** -24 * (np.abs(xc) @ np.abs(V32[0].astype(np.float64)))
    assert np.all(np.abs(raw - exact) <= bound)
    kr = oracle.klt_rotate_keys(ins.k, mu32, V32)[0]
    assert np.array_equal(kr, raw.astype(np.float32).astype(np.float16))
    qr = oracle.klt_rotate_queries(ins.q, V32)[0].astype(np.float64)
    qe = ins.q[0].astype(np.float64) @ V32[0].astype(np.float64)
    qb = (D + 1) * 2.0 ** -24 * (np.abs(ins.q[0]).astype(np.float64) @ np.abs(V32[0].astype(np.float64)))
    assert np.all(np.abs(qr - qe) <= qb)


def test_rotated_store_score_identity():
    """At full depth the rotated store's scores approximate q.(k - mu): the
    difference stays within the 4-bit quantisation bound of the rotated keys
    plus their binary16 rounding and the fp32 basis' departure from
    orthogonality."""
    ins = fathom_inputs.make_inputs(1, 4, 1024, seed=14)
    n = 1024
    mu, V, lam = oracle.klt_fit(ins.k)
    mu32, V32 = mu.astype(np.float32), V.astype(np.float32)
    kr = oracle.klt_rotate_keys(ins.k, mu32, V32)
    qr = oracle.klt_rotate_queries(ins.q, V32)
    planes, scales, _ = oracle.encode(kr)
    depths = np.full((1, D), 4, np.uint8)
    s64, _ = oracle.scan_f64(planes, scales, depths, qr, n)
    xc = ins.k[0].astype(np.float64) - mu32[0].astype(np.float64)
    truth = ins.q[0].astype(np.float64) @ xc.T                       # [G][n]
    a = np.array([[oracle.f16_to_f64(int(b)) for b in row] for row in scales[0].view(np.uint16)])
    amax = np.repeat(a, 64, axis=1)                                    # [d][n] block scales
    quant = np.abs(qr[0]).astype(np.float64) @ (amax / 16.0)          # sum_j |q'_j| a_j / 16
    r16 = np.abs(qr[0]).astype(np.float64) @ (np.abs(kr[0].astype(np.float64)).T * 2.0 ** -11)
    orth = 1e-5 * np.linalg.norm(ins.q[0], axis=1)[:, None] * np.linalg.norm(xc, axis=1)[None]
    err = np.abs(s64[0] - truth)
    assert np.all(err <= quant + r16 + orth)
