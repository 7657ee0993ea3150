"""GPU parity of fathom_scan and fathom_topk against the CPU oracle.

Scores: bit-exact against the oracle's fp32 evaluation order, and within
1e-4 of the fp64 definition relative to sum_j |q_hj khat_ij|.  Top-k index
sets: bit-exact (score descending, lower index first on ties, ascending
output), and a valid top-k of the fp64 scores up to that band (the leg that
does not depend on the fp32 order).  The end-to-end case runs the 1M-key
Qwen3-shaped layer at B = 92 with k = 4096 in the launch configuration the
benchmark times.
"""
import numpy as np
import pytest

import fathom_inputs
import oracle
from gpu_util import HipEvent, first_mismatch, say, to_dev, to_host
from topk_check import assert_scores_within_band, assert_topk_valid

pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.fixture(scope="module")
def fk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import sparse_top_kv_fathom_amd as fk
    fk.lib()
    return fk


def _scan(fk, planes, scales, depths, q, n):
    import torch
    s = fk.scan(to_dev(planes), to_dev(scales), to_dev(depths), to_dev(q), n)
    torch.cuda.synchronize()
    return to_host(s)


def _check_scores(gpu, planes, scales, depths, q, n):
    ref = oracle.scan_ref32(planes, scales, depths, q, n)
    assert np.array_equal(gpu.view(np.uint32), ref.view(np.uint32)), first_mismatch(gpu, ref)
    s64, l1 = oracle.scan_f64(planes, scales, depths, q, n)
    err = np.abs(gpu.astype(np.float64) - s64)
    assert np.all(err <= TOL * l1), float(np.max(err / np.maximum(l1, 1e-300)))


def test_scan_tiny(fk):
    w = fathom_inputs.WORKLOADS["tiny"]
    ins = fathom_inputs.workload_inputs("tiny")
    planes, scales, _ = oracle.encode(ins.k)
    depths, _, _ = oracle.plan(ins.q, ins.var, 92)
    say("scan tiny B=92")
    _check_scores(_scan(fk, planes, scales, depths, ins.q, w.n), planes, scales, depths, ins.q, w.n)


@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 8])
def test_scan_shapes_and_budgets(fk, G):
    """Several tiles plus a ragged tail tile (n = 64 * 101), every G, budgets
    from 0 (no active channel) to 512 (all channels at full depth)."""
    n = 64 * 101
    ins = fathom_inputs.make_inputs(3, G, n, seed=300 + G)
    planes, scales, _ = oracle.encode(ins.k)
    for B in (0, 3, 17, 92, 136, 512):
        depths, _, _ = oracle.plan(ins.q, ins.var, B)
        say("scan G=%d n=%d B=%d" % (G, n, B))
        gpu = _scan(fk, planes, scales, depths, ins.q, n)
        _check_scores(gpu, planes, scales, depths, ins.q, n)


def test_scan_random_depths_and_store_capacity(fk):
    """Arbitrary depth vectors (not from a plan) and a store larger than the
    scanned range (nb_store > n/64, scanning a prefix)."""
    rng = np.random.default_rng(31)
    ins = fathom_inputs.make_inputs(2, 4, 64 * 70, seed=31)
    planes, scales, _ = oracle.encode(ins.k, nb_store=90)
    for n in (64, 64 * 33, 64 * 70):
        depths = rng.integers(0, 5, size=(2, 128)).astype(np.uint8)
        say("scan random depths n=%d nb_store=90" % n)
        gpu = _scan(fk, planes, scales, depths, ins.q, n)
        _check_scores(gpu, planes, scales, depths, ins.q, n)


def _misaligned(t, elems):
    """The same values in a contiguous device view whose first element sits
    `elems` elements past a fresh allocation's (aligned) start."""
    import torch
    flat = torch.empty(t.numel() + elems, dtype=t.dtype, device=t.device)
    v = flat[elems:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("nb_extra,scale_shift", [(3, 0), (8, 2), (5, 6)])
def test_scan_odd_capacity_and_unaligned_scales(fk, nb_extra, scale_shift):
    """The main kernel on stores whose scale rows are not 16-byte aligned: a
    capacity that is not a multiple of 8 blocks (n/64 + 3, n/64 + 5), and
    scales starting 4 or 12 bytes past a 16-byte boundary; whole rounds plus a
    tail (n = 64 * 1000)."""
    import torch
    n = 64 * 1000
    ins = fathom_inputs.make_inputs(2, 4, n, seed=47 + nb_extra)
    planes, scales, _ = oracle.encode(ins.k, nb_store=n // 64 + nb_extra)
    depths, _, _ = oracle.plan(ins.q, ins.var, 92)
    ds = to_dev(scales)
    if scale_shift:
        ds = _misaligned(ds, scale_shift)
        assert ds.data_ptr() % 16 != 0
    say("scan nb_store=%d scale shift %d" % (n // 64 + nb_extra, scale_shift))
    s = fk.scan(to_dev(planes), ds, to_dev(depths), to_dev(ins.q), n)
    torch.cuda.synchronize()
    _check_scores(to_host(s), planes, scales, depths, ins.q, n)


def test_scan_timed_same_scores(fk):
    """fathom_scan_timed: the same scores bit for bit, and a positive kernel
    time in its events, with the main kernel only (n = 64 * 64), the main
    and the tail kernel (64 * 101) and the tail kernel only (64 * 5), on a
    store of 104 blocks (a multiple of 8: 16-byte scale rows)."""
    import torch
    ins = fathom_inputs.make_inputs(2, 4, 64 * 101, seed=41)
    planes, scales, _ = oracle.encode(ins.k, nb_store=104)
    depths, _, _ = oracle.plan(ins.q, ins.var, 92)
    dp, ds, dd, dq = to_dev(planes), to_dev(scales), to_dev(depths), to_dev(ins.q)
    for n in (64 * 64, 64 * 101, 64 * 5):
        say("scan timed n=%d" % n)
        e0, e1 = HipEvent(), HipEvent()
        s = fk.scan(dp, ds, dd, dq, n, events=(e0.h, e1.h))
        torch.cuda.synchronize()
        gpu = to_host(s)
        ref = oracle.scan_ref32(planes, scales, depths, ins.q, n)
        assert np.array_equal(gpu.view(np.uint32), ref.view(np.uint32)), first_mismatch(gpu, ref)
        assert e0.elapsed_ms(e1) > 0.0


def test_scan_random_shapes_sweep(fk):
    """24 seeded random cases: groups 1-3, G 1-8, n up to 25,600 keys, store
    capacities with and without the main kernel's alignment (nb_store a
    multiple of 8 or not), depth vectors from all-zero to all-four, half of
    them through fathom_scan_timed; scores equal the oracle's bit for bit."""
    import torch
    rng = np.random.default_rng(2024)
    for case in range(24):
        groups, G = int(rng.integers(1, 4)), int(rng.integers(1, 9))
        n = 64 * int(rng.integers(1, 401))
        nb_store = n // 64 + int(rng.integers(0, 40))
        kind = case % 4
        if kind == 0:
            depths = rng.integers(0, 5, size=(groups, 128))
        elif kind == 1:
            depths = np.where(rng.random((groups, 128)) < 0.6, 0, rng.integers(1, 5, (groups, 128)))
        elif kind == 2:
            depths = np.full((groups, 128), int(rng.integers(0, 5)))
        else:
            depths = np.where(rng.random((groups, 128)) < 0.5, 1, 4)
        depths = depths.astype(np.uint8)
        ins = fathom_inputs.make_inputs(groups, G, n, seed=5000 + case)
        planes, scales, _ = oracle.encode(ins.k, nb_store=nb_store)
        say("scan sweep case %d: groups=%d G=%d n=%d nb_store=%d kind=%d"
            % (case, groups, G, n, nb_store, kind))
        args = (to_dev(planes), to_dev(scales), to_dev(depths), to_dev(ins.q), n)
        if case % 2:
            e0, e1 = HipEvent(), HipEvent()
            s = fk.scan(*args, events=(e0.h, e1.h))
        else:
            s = fk.scan(*args)
        torch.cuda.synchronize()
        gpu = to_host(s)
        ref = oracle.scan_ref32(planes, scales, depths, ins.q, n)
        assert np.array_equal(gpu.view(np.uint32), ref.view(np.uint32)), first_mismatch(gpu, ref)


def test_topk_random_shapes_sweep(fk):
    """20 seeded random cases: rows 1-6, n from 1 to 60,000 (any n), k from 1
    to n, scores normal, heavy-tailed or rounded to few values (many ties);
    indices equal the oracle's."""
    rng = np.random.default_rng(77)
    for case in range(20):
        rows = int(rng.integers(1, 7))
        n = int(rng.integers(1, 60001))
        k = int(rng.integers(1, n + 1)) if case % 3 else int(rng.integers(1, min(n, 64) + 1))
        kind = case % 3
        if kind == 0:
            sc = rng.standard_normal((rows, n)).astype(np.float32)
        elif kind == 1:
            sc = rng.standard_t(2, (rows, n)).astype(np.float32)
        else:
            sc = np.round(rng.standard_normal((rows, n)) * 4).astype(np.float32)
        say("topk sweep case %d: rows=%d n=%d k=%d kind=%d" % (case, rows, n, k, kind))
        got = _topk(fk, sc, k)
        ref = oracle.topk(sc, k)
        assert np.array_equal(got, ref), first_mismatch(got, ref)


def _topk(fk, scores, k):
    import torch
    idx = fk.topk(to_dev(scores), k)
    torch.cuda.synchronize()
    return to_host(idx)


TOPK_CASES = [
    (4, 4096, 64), (3, 1000, 7), (2, 8192 * 3 + 17, 1000), (1, 100, 100), (5, 20000, 1),
    (2, 70000, 4096), (1, 8192, 8192), (3, 1, 1), (2, 8193, 8000),
]


@pytest.mark.parametrize("kind", ["normal", "ties", "const", "signed_zero"])
def test_topk_matches_oracle(fk, kind):
    for rows, n, k in TOPK_CASES:
        scores = fathom_inputs.random_scores(rows, n, seed=rows * 7 + n, kind=kind)
        say("topk kind=%s rows=%d n=%d k=%d" % (kind, rows, n, k))
        gpu = _topk(fk, scores, k)
        ref = oracle.topk(scores, k)
        assert np.array_equal(gpu, ref), first_mismatch(gpu, ref)


@pytest.mark.parametrize("kind", ["normal", "grid64"])
def test_topk_full_rows(fk, kind):
    """Rows of 1M scores, k = 4096 (the q1m shape): the candidate path, with
    a few hundred keys tied at the boundary for grid64."""
    rows, n, k = 4, 1 << 20, 4096
    scores = fathom_inputs.random_scores(rows, n, seed=77, kind=kind)
    say("topk full rows kind=%s rows=%d n=%d k=%d" % (kind, rows, n, k))
    gpu = _topk(fk, scores, k)
    ref = oracle.topk(scores, k)
    assert np.array_equal(gpu, ref), first_mismatch(gpu, ref)


@pytest.mark.parametrize("n", [1 << 21, 3 * (1 << 20) + 4099])
def test_topk_long_rows(fk, n):
    """Rows of 2M keys (256 chunks: the selection from registers with 64
    slots per chunk) and of 3M + 4099 keys (385 chunks, more than the
    registers cover: the candidates staged in LDS, 8 chunks per wave at a
    time, the last chunk partial), k = 4096."""
    rows, k = 2, 4096
    scores = fathom_inputs.random_scores(rows, n, seed=81, kind="normal")
    say("topk long rows rows=%d n=%d k=%d" % (rows, n, k))
    gpu = _topk(fk, scores, k)
    ref = oracle.topk(scores, k)
    assert np.array_equal(gpu, ref), first_mismatch(gpu, ref)


def test_topk_cut_never_published_falls_back(fk):
    """fathom_topk's cut workgroups store the cuts without publishing them
    (fathom_test_cut_hooks) and the compaction gives up after 4 polls: every
    chunk stamps a cut no row has, so every row is selected from its scores,
    with the same result.  The hooks are restored and a second call checks
    the candidate path again."""
    rows, n, k = 3, (1 << 17) + 4099, 700
    scores = fathom_inputs.random_scores(rows, n, seed=83, kind="normal")
    ref = oracle.topk(scores, k)
    say("topk cut never published rows=%d n=%d k=%d" % (rows, n, k))
    fk.test_cut_hooks(publish=False, spin_limit=4)
    try:
        gpu = _topk(fk, scores, k)
    finally:
        fk.test_cut_hooks(publish=True, spin_limit=2048)
    assert np.array_equal(gpu, ref), first_mismatch(gpu, ref)
    gpu = _topk(fk, scores, k)
    assert np.array_equal(gpu, ref), first_mismatch(gpu, ref)


def test_topk_crowded_chunks(fk):
    """Rows of 1M scores with 300 and 200 large scores planted in two chunks
    of 8192 keys that the cut's sample does not read (chunks 3 and 77): those
    chunks hold more candidates than the 128 per chunk the resolve stages
    straight from the loads it issues with the chunk counts, and fewer than a
    chunk's region holds, so the rest of them are staged afterwards."""
    rows, n, k = 2, 1 << 20, 4096
    scores = fathom_inputs.random_scores(rows, n, seed=79, kind="normal")
    rng = np.random.default_rng(80)
    sd = float(scores.std())
    for r in range(rows):
        for chunk, count in ((3, 300), (77, 200)):
            pos = chunk * 8192 + rng.choice(8192, count, replace=False)
            scores[r, pos] = (sd * rng.uniform(3.0, 5.0, count)).astype(np.float32)
    say("topk crowded chunks rows=%d n=%d k=%d" % (rows, n, k))
    gpu = _topk(fk, scores, k)
    ref = oracle.topk(scores, k)
    assert np.array_equal(gpu, ref), first_mismatch(gpu, ref)


def test_scan_repeatable(fk):
    """Three scans of the same inputs give the same bits (no order that
    depends on scheduling), at a size that fills the chip several times."""
    n = 1 << 18
    ins = fathom_inputs.make_inputs(4, 4, n, seed=43)
    planes, scales, _ = oracle.encode(ins.k)
    depths, _, _ = oracle.plan(ins.q, ins.var, 92)
    say("scan repeat x3 n=%d" % n)
    a = _scan(fk, planes, scales, depths, ins.q, n)
    for _ in range(2):
        b = _scan(fk, planes, scales, depths, ins.q, n)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), first_mismatch(a, b)


def test_topk_repeatable(fk):
    scores = fathom_inputs.random_scores(8, 50000, seed=41, kind="ties")
    say("topk repeat x3")
    a = _topk(fk, scores, 2048)
    for _ in range(2):
        assert np.array_equal(a, _topk(fk, scores, 2048))


@pytest.mark.timeout(900)
def test_end_to_end_q1m_b92(fk):
    """1M keys x 8 KV heads, GQA 4, B = 92, k = 4096: GPU encode -> plan ->
    scan -> top-k against the oracle, every output compared in full."""
    import torch
    w = fathom_inputs.WORKLOADS["q1m"]
    ins = fathom_inputs.workload_inputs("q1m")
    say("e2e q1m encode")
    kd = to_dev(ins.k)
    planes, scales = fk.encode(kd)
    say("e2e q1m plan/scan/topk")
    depths = fk.plan(to_dev(ins.q), to_dev(ins.var), 92)
    scores = fk.scan(planes, scales, depths, to_dev(ins.q), w.n)
    idx = fk.topk(scores, w.k)
    torch.cuda.synchronize()
    del kd
    gp, gs, gd, gsc, gi = (to_host(planes), to_host(scales), to_host(depths), to_host(scores),
                           to_host(idx))
    op, os_, _ = oracle.encode(ins.k)
    assert np.array_equal(gp, op), first_mismatch(gp, op)
    assert np.array_equal(gs, os_), first_mismatch(gs, os_)
    od, _, _ = oracle.plan(ins.q, ins.var, 92)
    assert np.array_equal(gd, od), first_mismatch(gd, od)
    ref = oracle.scan_ref32(op, os_, od, ins.q, w.n)
    assert np.array_equal(gsc.view(np.uint32), ref.view(np.uint32)), first_mismatch(gsc, ref)
    oi = oracle.topk(ref.reshape(-1, w.n), w.k)
    assert np.array_equal(gi, oi), first_mismatch(gi, oi)
    # every score against the fp64 definition, every set against its top-k
    say("e2e q1m fp64 leg")
    s64, l1 = oracle.scan_f64(op, os_, od, ins.q, w.n)
    assert_scores_within_band(gsc, s64, l1)
    assert_topk_valid(gi, s64, l1, w.k)


@pytest.mark.parametrize("mode,param", [("uniform", 2), ("uniform", 4), ("sparq", 16), ("sparq", 32)])
def test_fixed_plans_through_the_scan(fk, mode, param):
    """The comparison plans (2-bit thumbnail, full 4-bit, SparQ at 68 and 136
    bits) read through the same store, scan and top-k as the water-filled plan."""
    groups, G, n, k = 2, 4, 1 << 16, 256
    ins = fathom_inputs.make_inputs(groups, G, n, seed=81)
    say("fixed plan %s %d" % (mode, param))
    planes, scales = fk.encode(to_dev(ins.k))
    if mode == "uniform":
        depths = fk.plan_fixed(mode, param, groups=groups, G=G)
        od = oracle.plan_fixed(mode, param, groups=groups)
    else:
        depths = fk.plan_fixed(mode, param, q=to_dev(ins.q))
        od = oracle.plan_fixed(mode, param, q=ins.q)
    scores = fk.scan(planes, scales, depths, to_dev(ins.q), n)
    idx = fk.topk(scores, k)
    gd, gsc, gi = to_host(depths), to_host(scores), to_host(idx)
    assert np.array_equal(gd, od), first_mismatch(gd, od)
    op, os_, _ = oracle.encode(ins.k)
    ref = oracle.scan_ref32(op, os_, od, ins.q, n)
    assert np.array_equal(gsc.view(np.uint32), ref.view(np.uint32)), first_mismatch(gsc, ref)
    oi = oracle.topk(ref.reshape(-1, n), k)
    assert np.array_equal(gi, oi), first_mismatch(gi, oi)
    s64, l1 = oracle.scan_f64(op, os_, od, ins.q, n)
    assert_scores_within_band(gsc, s64, l1)
    assert_topk_valid(gi, s64, l1, k)


def _scan_topk_case(fk, groups, n, k, budget, seed, depths=None, write_scores=True, ins=None,
                    nb_store=None, scale_shift=0, G=4):
    """fathom_scan_topk against the oracle's scan and top-k (scores compared
    when the call writes them; index sets always, and against the fp64
    definition).  nb_store / scale_shift: the store built by the oracle with
    that capacity, its scales `scale_shift` elements past an aligned start."""
    if ins is None:
        ins = fathom_inputs.make_inputs(groups, G, n, seed=seed)
    if nb_store is None:
        planes, scales = fk.encode(to_dev(ins.k))
    else:
        hp, hs, _ = oracle.encode(ins.k, nb_store=nb_store)
        planes, scales = to_dev(hp), to_dev(hs)
    if scale_shift:
        scales = _misaligned(scales, scale_shift)
    if depths is None:
        dd = fk.plan(to_dev(ins.q), to_dev(ins.var), budget)
        od, _, _ = oracle.plan(ins.q, ins.var, budget)
    else:
        dd = to_dev(depths)
        od = depths
    scores, idx = fk.scan_topk(planes, scales, dd, to_dev(ins.q), n, k, write_scores=write_scores)
    gi = to_host(idx)
    op, os_, _ = oracle.encode(ins.k, nb_store=nb_store)
    ref = oracle.scan_ref32(op, os_, od, ins.q, n)
    if write_scores:
        gsc = to_host(scores)
        assert np.array_equal(gsc.view(np.uint32), ref.view(np.uint32)), first_mismatch(gsc, ref)
    else:
        assert scores is None
    oi = oracle.topk(ref.reshape(-1, n), k)
    assert np.array_equal(gi, oi), first_mismatch(gi, oi)
    s64, l1 = oracle.scan_f64(op, os_, od, ins.q, n)
    assert_topk_valid(gi, s64, l1, k)


@pytest.mark.parametrize("write_scores", [True, False])
@pytest.mark.parametrize("groups,n,k", [(2, 1 << 17, 512), (3, 1 << 16, 64), (1, 1 << 18, 4096),
                                        (2, 3 * 4096, 100), (1, 65536 + 2048, 300),
                                        (2, 65536 + 64 * 37, 500), (1, 1 << 21, 4096),
                                        (1, (1 << 21) - 64, 4096)])
def test_scan_topk_matches_scan_then_topk(fk, groups, n, k, write_scores):
    """Fused (64k <= n <= 2M: whole rounds in the main kernel, the rest, down
    to a partial last tile, in the tail kernel) and unfused (shorter rows)
    paths, with and without a score buffer."""
    say("scan_topk groups=%d n=%d k=%d write_scores=%s" % (groups, n, k, write_scores))
    _scan_topk_case(fk, groups, n, k, 92, seed=90 + groups, write_scores=write_scores)


@pytest.mark.parametrize("G", [1, 2, 3, 8])
def test_scan_topk_query_heads_per_group(fk, G):
    """The fused path for other group sizes (the sample's per-head partial
    sums, the candidate regions of every head), with a ragged n."""
    n, k = 65536 + 64 * 9, 300
    say("scan_topk G=%d n=%d" % (G, n))
    _scan_topk_case(fk, 2, n, k, 92, seed=110 + G, write_scores=(G % 2 == 0), G=G)


@pytest.mark.parametrize("write_scores", [True, False])
@pytest.mark.parametrize("nb_extra,scale_shift", [(3, 0), (0, 2)])
def test_scan_topk_odd_capacity_and_unaligned_scales(fk, nb_extra, scale_shift, write_scores):
    """The fused path on a store of n/64 + 3 blocks (8-byte plane loads,
    2-byte scale loads in the sample) and on scales 4 bytes past a 16-byte
    boundary, with a ragged n (whole rounds plus a tail)."""
    n, k = 65536 + 64 * 45, 700
    say("scan_topk nb_store=n/64+%d scale shift %d write_scores=%s"
        % (nb_extra, scale_shift, write_scores))
    _scan_topk_case(fk, 2, n, k, 92, seed=95, write_scores=write_scores,
                    nb_store=n // 64 + nb_extra, scale_shift=scale_shift)


@pytest.mark.parametrize("write_scores", [True, False])
def test_scan_topk_heavy_ties_fall_back(fk, write_scores):
    """One active channel at depth 1: every score takes one of two values per
    block, so the candidate regions overflow and rows are selected from their
    scores (the caller's, or a second scan into the workspace)."""
    n, k = 1 << 17, 1000
    depths = np.zeros((2, 128), dtype=np.uint8)
    depths[:, 5] = 1
    say("scan_topk heavy ties write_scores=%s" % write_scores)
    _scan_topk_case(fk, 2, n, k, 0, seed=97, depths=depths, write_scores=write_scores)


@pytest.mark.parametrize("write_scores", [True, False])
def test_scan_topk_unrepresentative_sample_falls_back(fk, write_scores):
    """Keys aligned with the queries planted in every sampled run (the 8
    runs of 1024 keys every 16384 keys at n = 2^17): the cut taken from the
    sample lies above all but a few hundred keys of the row, fewer than k, so
    the rows are selected from their scores."""
    groups, G, n, k = 2, 4, 1 << 17, 2000
    ins = fathom_inputs.make_inputs(groups, G, n, seed=99)
    rng = np.random.default_rng(98)
    run, stride = 1024, n // 8
    for g in range(groups):
        qn = ins.q[g].astype(np.float64).sum(axis=0)
        qn /= np.abs(qn).max()
        top = 4.0 * float(np.abs(ins.k[g]).max())
        for s0 in range(0, n, stride):
            mag = top * rng.uniform(0.5, 1.0, run)
            ins.k[g, s0:s0 + run] = (mag[:, None] * qn[None, :]).astype(np.float16)
    say("scan_topk unrepresentative sample write_scores=%s" % write_scores)
    _scan_topk_case(fk, groups, n, k, 92, seed=0, write_scores=write_scores, ins=ins)


@pytest.mark.parametrize("write_scores", [True, False])
@pytest.mark.parametrize("width", [300, 420])
def test_scan_topk_clustered_window(fk, width, write_scores):
    """Top keys crowded into one stretch of the row, away from the sampled
    runs: `width` keys aligned with the group's queries inside the 2048-key
    round at keys 4096..6143 (the sample reads keys 0..1023, 16384..17407,
    ...).  With the round's other candidates (about 50 at this k) they fit
    the round's 512 slots, so these rows are selected from the candidates,
    through a round far fuller than the others; the result is the same as
    scan then top-k."""
    groups, G, n, k = 2, 4, 1 << 17, 2000
    ins = fathom_inputs.make_inputs(groups, G, n, seed=121)
    rng = np.random.default_rng(122)
    s0 = 4096 + 300
    for g in range(groups):
        qn = ins.q[g].astype(np.float64).sum(axis=0)
        qn /= np.abs(qn).max()
        top = 4.0 * float(np.abs(ins.k[g]).max())
        mag = top * rng.uniform(0.5, 1.0, width)
        ins.k[g, s0:s0 + width] = (mag[:, None] * qn[None, :]).astype(np.float16)
    say("scan_topk clustered window width=%d write_scores=%s" % (width, write_scores))
    _scan_topk_case(fk, groups, n, k, 92, seed=0, write_scores=write_scores, ins=ins)


@pytest.mark.parametrize("groups,n,k,write_scores", [(2, (1 << 17) + 64 * 5, 700, True),
                                                     (2, (1 << 17) + 64 * 5, 700, False),
                                                     (1, 1 << 21, 4096, False)])
def test_scan_topk_cut_never_published_falls_back(fk, groups, n, k, write_scores):
    """The scan's cut workgroups store the cuts but do not publish them
    (fathom_test_cut_hooks), and the waves give up after 4 polls: every row
    is flagged by the scan and selected from its scores (the caller's, or a
    second scan into the workspace: at 2^21 keys the largest fused row), with
    the same result.  The hooks are restored afterwards, and a second call
    checks that the fused path is back."""
    say("scan_topk cut never published groups=%d n=%d write_scores=%s" % (groups, n, write_scores))
    fk.test_cut_hooks(publish=False, spin_limit=4)
    try:
        _scan_topk_case(fk, groups, n, k, 92, seed=101, write_scores=write_scores)
    finally:
        fk.test_cut_hooks(publish=True, spin_limit=2048)
    _scan_topk_case(fk, groups, n, k, 92, seed=102, write_scores=write_scores)
