"""GPU parity of fathom_gather: the depth-selected runs of a pinned host store
copied into the device store.

The host store is the oracle's encoding of seeded keys.  After a gather under
a depth vector, every plane row p < t_j and every scale row with t_j > 0 must
equal the host's over blocks [0, n/64); every other word of the device store
must still hold the sentinel it was filled with.  A scan over the gathered
store must then give bit for bit the scores of a scan over the whole store.
"""
import numpy as np
import pytest

import fathom_inputs
import oracle
from gpu_util import first_mismatch, say, to_dev, to_host

pytestmark = pytest.mark.gpu

SENT64 = np.uint64(0xA5A5_5A5A_C3C3_3C3C)
SENT16 = np.uint16(0xBEEF)


@pytest.fixture(scope="module")
def fk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import sparse_top_kv_fathom_amd as fk
    fk.lib()
    return fk


def _pinned(a: np.ndarray):
    t = to_dev(a).cpu()
    return t.pin_memory()


def _expected(planes, scales, depths, nblk):
    """Sentinel store with the runs the depths select copied in."""
    ep = np.full_like(planes, SENT64)
    es = np.full_like(scales, SENT16)
    groups, d = depths.shape
    for g in range(groups):
        for j in range(d):
            t = int(depths[g, j])
            ep[g, j, :t, :nblk] = planes[g, j, :t, :nblk]
            if t > 0:
                es[g, j, :nblk] = scales[g, j, :nblk]
    return ep, es


def _gather(fk, hp, hs, depths, n, shape_p, shape_s):
    import torch
    dp = to_dev(np.full(shape_p, SENT64, dtype=np.uint64))
    ds = to_dev(np.full(shape_s, SENT16, dtype=np.uint16))
    fk.gather(hp, hs, to_dev(depths), n, dp, ds)
    torch.cuda.synchronize()
    return to_host(dp), to_host(ds)


@pytest.mark.parametrize("groups,n,nb_store", [(2, 64 * 40, 40), (3, 64 * 37, 48),
                                               (1, 64 * 9000, 9000), (2, 64, 8)])
def test_gather_runs(fk, groups, n, nb_store):
    """Planned depths, random depths, a store larger than the range gathered,
    more blocks than one 8192-block segment, a single block."""
    ins = fathom_inputs.make_inputs(groups, 4, n, seed=700 + groups)
    planes, scales, _ = oracle.encode(ins.k, nb_store=nb_store)
    hp, hs = _pinned(planes), _pinned(scales)
    rng = np.random.default_rng(groups * 1000 + n)
    cases = [oracle.plan(ins.q, ins.var, 92)[0],
             rng.integers(0, 5, size=(groups, 128)).astype(np.uint8),
             np.zeros((groups, 128), np.uint8), np.full((groups, 128), 4, np.uint8)]
    for ci, depths in enumerate(cases):
        say("gather groups=%d n=%d nb_store=%d case=%d" % (groups, n, nb_store, ci))
        gp, gs = _gather(fk, hp, hs, depths, n, planes.shape, scales.shape)
        ep, es = _expected(planes, scales, depths, n // 64)
        assert np.array_equal(gp, ep), first_mismatch(gp, ep)
        assert np.array_equal(gs, es), first_mismatch(gs, es)


def test_gather_then_scan(fk):
    """The scan reads only what the gather brought in: scores over the
    gathered store equal the scores over the complete store, bit for bit, and
    the oracle's."""
    import torch
    groups, G, n = 2, 4, 64 * 300
    ins = fathom_inputs.make_inputs(groups, G, n, seed=77)
    planes, scales, _ = oracle.encode(ins.k, nb_store=304)
    hp, hs = _pinned(planes), _pinned(scales)
    for B in (17, 92, 136):
        depths, _, _ = oracle.plan(ins.q, ins.var, B)
        say("gather+scan B=%d" % B)
        dp = to_dev(np.full(planes.shape, SENT64, dtype=np.uint64))
        ds = to_dev(np.full(scales.shape, SENT16, dtype=np.uint16))
        dd, dq = to_dev(depths), to_dev(ins.q)
        fk.gather(hp, hs, dd, n, dp, ds)
        s_gather = fk.scan(dp, ds, dd, dq, n)
        s_full = fk.scan(to_dev(planes), to_dev(scales), dd, dq, n)
        torch.cuda.synchronize()
        a, b = to_host(s_gather), to_host(s_full)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), first_mismatch(a, b)
        ref = oracle.scan_ref32(planes, scales, depths, ins.q, n)
        assert np.array_equal(a.view(np.uint32), ref.view(np.uint32)), first_mismatch(a, ref)


def test_gather_rejects_pageable(fk):
    """Pageable host memory is refused before any copy is issued."""
    import torch
    planes = np.zeros((1, 128, 4, 8), np.uint64)
    scales = np.zeros((1, 128, 8), np.uint16)
    hp = to_dev(planes).cpu()
    hs = to_dev(scales).cpu()
    dp, ds = to_dev(planes), to_dev(scales)
    dd = to_dev(np.full((1, 128), 2, np.uint8))
    st = fk.lib().fathom_gather(hp.data_ptr(), hs.data_ptr(), 8, dd.data_ptr(), 1, 128, 512,
                                dp.data_ptr(), ds.data_ptr(), None)
    torch.cuda.synchronize()
    assert st == -8
