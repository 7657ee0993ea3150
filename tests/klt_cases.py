"""Planted KLT cases shared by the oracle pins and the GPU parity tests: keys
whose covariance, mean and eigenbasis are known in closed form."""
import numpy as np

D = 128
H4 = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]], dtype=np.float64) / 2


def planted(seed=0, reps=2):
    """Keys with an exactly known covariance: returns (k fp16 [1][n][d],
    mu0 [d], R [d][d], sigma [d])."""
    rng = np.random.default_rng(seed)
    Hb = np.kron(np.eye(D // 4), H4)
    R = Hb[rng.permutation(D)][:, rng.permutation(D)]          # orthogonal, entries 0, +-1/2
    sigma = (np.arange(D) + 1) / 16.0                           # distinct, dyadic
    mu0 = (np.arange(D) % 7 - 3).astype(np.float64)
    rows = []
    for j in range(D):
        for _ in range(reps):
            rows.append(mu0 + sigma[j] * R[:, j])
            rows.append(mu0 - sigma[j] * R[:, j])
    x = np.array(rows)[rng.permutation(len(rows))]
    k = x.astype(np.float16)
    assert np.array_equal(k.astype(np.float64), x)             # exact in binary16
    return k[None], mu0, R, sigma


def expected_basis(R, sigma):
    """R's columns by sigma descending, each with its first nonzero entry
    (+-1/2, above the 1/(2 sqrt(128)) threshold) positive."""
    order = np.argsort(-sigma)
    V = R[:, order].copy()
    for j in range(D):
        r = int(np.flatnonzero(V[:, j])[0])
        if V[r, j] < 0:
            V[:, j] *= -1
    return V
