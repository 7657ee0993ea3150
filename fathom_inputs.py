"""Seeded synthetic inputs for the Fathom key scan (shared by tests and bench).

This module only draws random arrays; it holds none of the method's
arithmetic, so both the GPU path and the CPU oracle can be fed from it.

Recipe (stand-in for Qwen3-8B K caches: 8 KV heads x 128 channels, 4 query
heads per KV head, contexts of 256k and 1M tokens — the model shape of §1 and
the context lengths of Tab. 2 of "Fathom: Per-Query Read Depth for Sparse
Decoding over Offloaded KV Caches"; the pages themselves time the long
contexts on synthetic KV):

* per group (one KV head of one layer / session): channel scale
  sigma_j = exp(z_j), z_j ~ N(0, 1), and 4 distinct outlier channels whose
  sigma is multiplied by 10;
* keys K_ij = fp16(sigma_j * x_ij), x_ij ~ N(0, 1) drawn in fp32, rounded to
  nearest-even by numpy;
* query heads q_hj ~ N(0, 1) in fp32;
* channel variance Var_j = the fp64 sample variance (ddof = 1) of the fp16
  column over all n keys of the group, cast to fp32.  (Appendix A's 0.127 for
  its channel 2 is the ddof = 1 variance of that channel's six values.)
* budget sweep: 36 layers of the 1M-key shape, seed 5 + layer, with 32
  needle keys per KV head aligned with the query heads in turn (cosine 0.6,
  norm |sigma|_2), for recall against exact scores.

Generator: numpy PCG64 via ``default_rng``; each group draws from its own
child of ``SeedSequence(seed)`` so groups can be generated in parallel.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

D = 128
G_QWEN3 = 4
KV_HEADS = 8
OUTLIERS = 4
OUTLIER_GAIN = 10.0


@dataclass(frozen=True)
class Workload:
    name: str
    groups: int           # KV heads x sessions (x layers) in one call
    G: int                # query heads per KV head
    n: int                # keys per group
    budgets: tuple        # code-bit budgets B
    k: int                # top-k per query head
    seed: int
    d: int = D
    note: str = ""


# The workloads: tiny (oracle-sized), Qwen3-8B-shaped 256k and 1M single
# layers, 16 resident sessions of 128k.  (The full 36-layer budget sweep is
# generated layer by layer with seed 5 + layer.)
WORKLOADS = {
    "tiny": Workload("tiny", 1, 4, 4096, (92,), 64, 1,
                     note="1 KV head, GQA 4, n=4096"),
    "q256k": Workload("q256k", 8, 4, 262_144, (68, 92, 136), 2048, 2,
                      note="Qwen3-8B-shaped layer, 8 KV heads, n=262144"),
    "q1m": Workload("q1m", 8, 4, 1_048_576, (68, 92, 136), 4096, 3,
                    note="Qwen3-8B-shaped layer, 8 KV heads, n=1048576"),
    "s16": Workload("s16", 128, 4, 131_072, (92,), 1024, 4,
                    note="16 sessions x 8 KV heads, n=131072 each"),
}


def _children(seed: int, count: int):
    return np.random.SeedSequence(seed).spawn(count)


def _threads(count: int) -> int:
    env = os.environ.get("FATHOM_GEN_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(count, os.cpu_count() or 1, 16))


def _one_group(ss: np.random.SeedSequence, n: int, d: int):
    rng = np.random.default_rng(ss)
    sigma = np.exp(rng.standard_normal(d)).astype(np.float32)
    out = rng.choice(d, size=OUTLIERS, replace=False)
    sigma[out] *= np.float32(OUTLIER_GAIN)
    k = np.empty((n, d), dtype=np.float16)
    step = 1 << 16
    for s in range(0, n, step):
        e = min(n, s + step)
        x = rng.standard_normal((e - s, d), dtype=np.float32)
        x *= sigma[None, :]
        k[s:e] = x.astype(np.float16)
    return k, sigma


def make_keys(groups: int, n: int, seed: int, d: int = D):
    """K [groups][n][d] fp16 and the channel scales sigma [groups][d] fp32."""
    k = np.empty((groups, n, d), dtype=np.float16)
    sigma = np.empty((groups, d), dtype=np.float32)
    kids = _children(seed, 2 * groups)

    def work(g):
        kg, sg = _one_group(kids[g], n, d)
        k[g] = kg
        sigma[g] = sg

    nt = _threads(groups)
    if nt == 1:
        for g in range(groups):
            work(g)
    else:
        with _cf.ThreadPoolExecutor(nt) as ex:
            list(ex.map(work, range(groups)))
    return k, sigma


def make_queries(groups: int, G: int, seed: int, d: int = D) -> np.ndarray:
    """q [groups][G][d] fp32, N(0, 1)."""
    kids = _children(seed, 2 * groups)
    q = np.empty((groups, G, d), dtype=np.float32)
    for g in range(groups):
        rng = np.random.default_rng(kids[groups + g])
        q[g] = rng.standard_normal((G, d), dtype=np.float32)
    return q


def channel_variance(k: np.ndarray) -> np.ndarray:
    """fp64 sample variance (ddof=1) of every fp16 column, as fp32 [groups][d]."""
    groups, n, d = k.shape
    var = np.empty((groups, d), dtype=np.float32)
    step = 1 << 16

    def one(g):
        s = np.zeros(d, dtype=np.float64)
        for a in range(0, n, step):
            s += k[g, a:a + step].astype(np.float64).sum(axis=0)
        mean = s / n
        ss = np.zeros(d, dtype=np.float64)
        for a in range(0, n, step):
            x = k[g, a:a + step].astype(np.float64) - mean
            ss += (x * x).sum(axis=0)
        var[g] = (ss / max(n - 1, 1)).astype(np.float32)

    nt = _threads(groups)
    if nt == 1 or groups == 1:
        for g in range(groups):
            one(g)
    else:
        with _cf.ThreadPoolExecutor(nt) as ex:
            list(ex.map(one, range(groups)))
    return var


@dataclass
class Inputs:
    k: np.ndarray        # [groups][n][d] fp16
    q: np.ndarray        # [groups][G][d] fp32
    var: np.ndarray      # [groups][d] fp32
    sigma: np.ndarray    # [groups][d] fp32
    extra: dict = field(default_factory=dict)


def make_inputs(groups: int, G: int, n: int, seed: int, d: int = D,
                query_seed: int | None = None) -> Inputs:
    """Keys, queries and variances of one workload.  ``query_seed`` lets a
    decode loop draw a fresh query group per step over the same keys."""
    k, sigma = make_keys(groups, n, seed, d)
    q = make_queries(groups, G, seed if query_seed is None else query_seed, d)
    var = channel_variance(k)
    return Inputs(k=k, q=q, var=var, sigma=sigma)


# The budget sweep: 36 layers of the 1M-key layer shape (seed 5 + layer),
# budgets 32..256 code bits in steps of 16, k = 4096, 32 planted needles per
# KV head.
SWEEP_LAYERS = 36
SWEEP_BUDGETS = tuple(range(32, 257, 16))
SWEEP_K = 4096
SWEEP_NEEDLES = 32
SWEEP_COSINE = 0.6


def sweep_seed(layer: int) -> int:
    return 5 + layer


def plant_needles(ins: Inputs, seed: int, count: int = SWEEP_NEEDLES,
                  cosine: float = SWEEP_COSINE) -> np.ndarray:
    """Overwrite `count` keys per group, at distinct uniformly drawn
    positions, with needles aligned to the group's query heads in turn
    (needle i to head i % G): k = |sigma|_2 (c qhat_h + sqrt(1 - c^2) w), w a
    random unit vector orthogonal to qhat_h, built in fp64 and rounded to
    fp16.  The channel variances are then recomputed over the keys that hold
    the needles.  Returns the positions, [groups][count] int64."""
    groups, n, d = ins.k.shape
    G = ins.q.shape[1]
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x6e656564]))
    pos = np.empty((groups, count), dtype=np.int64)
    s = np.sqrt(1.0 - cosine * cosine)
    for g in range(groups):
        pos[g] = rng.choice(n, size=count, replace=False)
        norm = float(np.sqrt(np.sum(ins.sigma[g].astype(np.float64) ** 2)))
        for i in range(count):
            qh = ins.q[g, i % G].astype(np.float64)
            qh /= np.linalg.norm(qh)
            w = rng.standard_normal(d)
            w -= (w @ qh) * qh
            w /= np.linalg.norm(w)
            ins.k[g, pos[g, i]] = (norm * (cosine * qh + s * w)).astype(np.float16)
    ins.var[...] = channel_variance(ins.k)
    ins.extra["needles"] = pos
    return pos


def sweep_inputs(layer: int) -> Inputs:
    """One layer of the budget sweep: the 1M-key layer shape with needles."""
    w = WORKLOADS["q1m"]
    ins = make_inputs(w.groups, w.G, w.n, sweep_seed(layer), w.d)
    plant_needles(ins, sweep_seed(layer))
    return ins


def workload_inputs(name: str) -> Inputs:
    w = WORKLOADS[name]
    return make_inputs(w.groups, w.G, w.n, w.seed, w.d)


def random_scores(rows: int, n: int, seed: int, kind: str = "normal") -> np.ndarray:
    """Score rows for top-k tests: 'normal' (N(0,1) fp32), 'ties' (values on a
    coarse grid so many keys tie), 'grid64' (N(0,1) rounded to multiples of
    1/64: a few hundred ties per value near the top-k boundary of a 1M row),
    'const' (all equal), 'signed_zero' (a mix of +0 and -0 with a few larger
    values)."""
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return rng.standard_normal((rows, n), dtype=np.float32)
    if kind == "ties":
        return (rng.integers(-8, 8, size=(rows, n)).astype(np.float32) * np.float32(0.25))
    if kind == "grid64":
        return (np.round(rng.standard_normal((rows, n)) * 64.0) / 64.0).astype(np.float32)
    if kind == "const":
        return np.full((rows, n), np.float32(1.5), dtype=np.float32)
    if kind == "signed_zero":
        s = np.where(rng.random((rows, n)) < 0.5, np.float32(0.0), np.float32(-0.0))
        s = s.astype(np.float32)
        m = rng.random((rows, n)) < 0.01
        s[m] = rng.standard_normal(int(m.sum())).astype(np.float32)
        return s
    raise ValueError(kind)
