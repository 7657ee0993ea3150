"""GPU parity at the full sizes of the workloads: the 256k-key layer at every
budget, the 1M-key layer at the budgets the 92-bit test does not cover and
through the fused call, and the 16-session case (128 groups of 131,072 keys)
with every output of a spread of groups compared.

Everything is bit-exact against the oracle: encodings, plans, scores (the
fixed fp32 order) and top-k index sets.  Every compared score is also within
the 1e-4 band of the fp64 definition and every compared set a valid top-k of
the fp64 scores up to that band.
"""
import numpy as np
import pytest

import fathom_inputs
import oracle
from gpu_util import first_mismatch, say, to_dev, to_host
from topk_check import assert_scores_within_band, assert_topk_valid

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import sparse_top_kv_fathom_amd as fk
    fk.lib()
    return fk


def _check_layer(fk, ins, n, k, budgets, planes, scales, op, os_, fused=False):
    import torch
    q_d, var_d = to_dev(ins.q), to_dev(ins.var)
    for B in budgets:
        say("layer n=%d B=%d k=%d fused=%s" % (n, B, k, fused))
        depths = fk.plan(q_d, var_d, B)
        scores = fk.scan(planes, scales, depths, q_d, n)
        idx = fk.topk(scores, k)
        if fused:
            fs, fi = fk.scan_topk(planes, scales, depths, q_d, n, k)
            _, fi2 = fk.scan_topk(planes, scales, depths, q_d, n, k, write_scores=False)
        torch.cuda.synchronize()
        gd, gsc, gi = to_host(depths), to_host(scores), to_host(idx)
        od, _, _ = oracle.plan(ins.q, ins.var, B)
        assert np.array_equal(gd, od), first_mismatch(gd, od)
        ref = oracle.scan_ref32(op, os_, od, ins.q, n)
        assert np.array_equal(gsc.view(np.uint32), ref.view(np.uint32)), first_mismatch(gsc, ref)
        oi = oracle.topk(ref.reshape(-1, n), k)
        assert np.array_equal(gi, oi), first_mismatch(gi, oi)
        s64, l1 = oracle.scan_f64(op, os_, od, ins.q, n)
        assert_scores_within_band(gsc, s64, l1)
        assert_topk_valid(gi, s64, l1, k)
        if fused:
            assert np.array_equal(to_host(fs).view(np.uint32), ref.view(np.uint32))
            assert np.array_equal(to_host(fi), oi)
            assert np.array_equal(to_host(fi2), oi)


@pytest.mark.timeout(600)
def test_q256k_every_budget(fk):
    w = fathom_inputs.WORKLOADS["q256k"]
    ins = fathom_inputs.workload_inputs("q256k")
    say("q256k encode")
    planes, scales = fk.encode(to_dev(ins.k))
    op, os_, _ = oracle.encode(ins.k)
    assert np.array_equal(to_host(planes), op)
    assert np.array_equal(to_host(scales), os_)
    _check_layer(fk, ins, w.n, w.k, w.budgets, planes, scales, op, os_, fused=True)


@pytest.mark.timeout(900)
def test_q1m_other_budgets_and_fused(fk):
    """B = 68 and 136 (92 has its own test), and the fused call at B = 92."""
    w = fathom_inputs.WORKLOADS["q1m"]
    ins = fathom_inputs.workload_inputs("q1m")
    say("q1m encode")
    planes, scales = fk.encode(to_dev(ins.k))
    op, os_, _ = oracle.encode(ins.k)
    assert np.array_equal(to_host(planes), op)
    _check_layer(fk, ins, w.n, w.k, (68, 136), planes, scales, op, os_)
    _check_layer(fk, ins, w.n, w.k, (92,), planes, scales, op, os_, fused=True)


@pytest.mark.timeout(900)
def test_sixteen_sessions(fk):
    """128 groups (16 sessions x 8 KV heads, each with its own channel scales,
    variances and queries) of 131,072 keys, B = 92, k = 1024 per query head:
    the GPU runs every group in one call per step; groups at both ends and in
    the middle are compared in full, and every group's plan."""
    import torch
    w = fathom_inputs.WORKLOADS["s16"]
    say("s16 inputs")
    ins = fathom_inputs.workload_inputs("s16")
    say("s16 gpu")
    q_d = to_dev(ins.q)
    planes, scales = fk.encode(to_dev(ins.k))
    depths = fk.plan(q_d, to_dev(ins.var), 92)
    scores = fk.scan(planes, scales, depths, q_d, w.n)
    idx = fk.topk(scores, w.k)
    torch.cuda.synchronize()
    gd = to_host(depths)
    od, _, _ = oracle.plan(ins.q, ins.var, 92)
    assert np.array_equal(gd, od), first_mismatch(gd, od)
    gp, gs, gsc, gi = to_host(planes), to_host(scales), to_host(scores), to_host(idx)
    G = w.G
    for g in (0, 1, 63, 64, 126, 127):
        say("s16 group %d" % g)
        kg = np.ascontiguousarray(ins.k[g:g + 1])
        op, os_, _ = oracle.encode(kg)
        assert np.array_equal(gp[g:g + 1], op), g
        assert np.array_equal(gs[g:g + 1], os_), g
        ref = oracle.scan_ref32(op, os_, od[g:g + 1], ins.q[g:g + 1], w.n)
        assert np.array_equal(gsc[g:g + 1].view(np.uint32), ref.view(np.uint32)), g
        oi = oracle.topk(ref.reshape(-1, w.n), w.k)
        assert np.array_equal(gi[g * G:(g + 1) * G], oi), g
        s64, l1 = oracle.scan_f64(op, os_, od[g:g + 1], ins.q[g:g + 1], w.n)
        assert_scores_within_band(gsc[g:g + 1], s64, l1)
        assert_topk_valid(gi[g * G:(g + 1) * G], s64, l1, w.k)
