"""GPU parity on the budget sweep's layers (the 1M-key layer shape with 32
planted needles per KV head), sampled at layers 0, 17 and 35 and every
budget from 32 to 256 code bits: the encoding bit-exact in full, plans
bit-exact, scores of a slice of blocks of every group bit-exact, top-k index
sets bit-exact against the oracle's selection over the same scores; every
score within the 1e-4 band of the fp64 definition and every set a valid
top-k of the fp64 scores up to that band.
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


@pytest.mark.timeout(900)
@pytest.mark.parametrize("layer", [0, 17, 35])
def test_sweep_layer_every_budget(fk, layer):
    import torch
    w = fathom_inputs.WORKLOADS["q1m"]
    n, k = w.n, fathom_inputs.SWEEP_K
    say("sweep layer %d inputs" % layer)
    ins = fathom_inputs.sweep_inputs(layer)
    planes, scales = fk.encode(to_dev(ins.k))
    q_d, var_d = to_dev(ins.q), to_dev(ins.var)
    b0, b1 = 7000, 7040                       # a slice of blocks of every group
    torch.cuda.synchronize()
    gp, gs = to_host(planes), to_host(scales)
    say("sweep layer %d oracle encode" % layer)
    fp, fs, _ = oracle.encode(ins.k)
    assert np.array_equal(gp, fp) and np.array_equal(gs, fs)
    op = np.ascontiguousarray(fp[..., b0:b1])
    os_ = np.ascontiguousarray(fs[..., b0:b1])
    for B in fathom_inputs.SWEEP_BUDGETS:
        say("sweep layer %d B=%d" % (layer, B))
        depths = fk.plan(q_d, var_d, B)
        scores = fk.scan(planes, scales, depths, q_d, n)
        idx = fk.topk(scores, k)
        torch.cuda.synchronize()
        gd, gsc, gi = to_host(depths), to_host(scores), to_host(idx)
        od, _, _ = oracle.plan(ins.q, ins.var, B)
        assert np.array_equal(gd, od), first_mismatch(gd, od)
        ref = oracle.scan_ref32(op, os_, od, ins.q, (b1 - b0) * 64)
        got = np.ascontiguousarray(gsc[:, :, b0 * 64:b1 * 64])
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), first_mismatch(got, ref)
        oi = oracle.topk(gsc.reshape(-1, n), k)
        assert np.array_equal(gi, oi), first_mismatch(gi, oi)
        s64, l1 = oracle.scan_f64(fp, fs, od, ins.q, n)
        assert_scores_within_band(gsc, s64, l1)
        assert_topk_valid(gi, s64, l1, k)
