"""GPU parity of fathom_encode and fathom_plan against the CPU oracle.

Bit-exact: plane words, scales, depth vectors, water lines (fp64 bits) and
bit counts.  Inputs come from the seeded generator; every case is printed
before its GPU step.
"""
import json
import os

import numpy as np
import pytest

import fathom_inputs
import oracle
from gpu_util import first_mismatch, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import sparse_top_kv_fathom_amd as fk
    fk.lib()
    return fk


def _gpu_encode(fk, k, nb_store=None, block_offset=0, planes=None, scales=None):
    import torch
    kd = to_dev(k)
    if planes is None:
        pd, sd = fk.empty_store(k.shape[0], nb_store or k.shape[1] // 64)
        pd.zero_()
        sd.zero_()
    else:
        pd, sd = to_dev(planes), to_dev(scales)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    fk.encode(kd, pd, sd, block_offset=block_offset, nonfinite_flag=flag)
    torch.cuda.synchronize()
    return to_host(pd), to_host(sd), int(flag.item())


# Up to 64 blocks per call the column-split kernel runs, above it the
# block-per-wave kernel: both are covered.
@pytest.mark.parametrize("groups,nblk", [(1, 64), (3, 37), (2, 1), (5, 6), (2, 65), (1, 203)])
def test_encode_matches_oracle(fk, groups, nblk):
    n = 64 * nblk
    say("encode groups=%d n=%d" % (groups, n))
    k, _ = fathom_inputs.make_keys(groups, n, seed=100 + nblk)
    gp, gs, flag = _gpu_encode(fk, k)
    op, os_, bad = oracle.encode(k)
    assert flag == 0 and bad == 0
    assert np.array_equal(gp, op), first_mismatch(gp, op)
    assert np.array_equal(gs, os_), first_mismatch(gs, os_)


def test_encode_appends_into_store(fk):
    say("encode append nb_store=50 offset=5")
    k, _ = fathom_inputs.make_keys(2, 64 * 20, seed=7)
    sentinel_p = np.full((2, 128, 4, 50), 0x0123456789ABCDEF, dtype=np.uint64)
    sentinel_s = np.full((2, 128, 50), 0x5A5A, dtype=np.uint16)
    gp, gs, _ = _gpu_encode(fk, k, block_offset=5, planes=sentinel_p, scales=sentinel_s)
    op, os_, _ = oracle.encode(k, nb_store=50, block_offset=5, planes=sentinel_p.copy(),
                               scales=sentinel_s.copy())
    assert np.array_equal(gp, op), first_mismatch(gp, op)
    assert np.array_equal(gs, os_), first_mismatch(gs, os_)


@pytest.mark.parametrize("reps", [1, 9])
def test_encode_edge_values(fk, reps):
    """Zero blocks, +-a, -0, fp16 max, subnormal block maxima, exact cell edges
    (8 blocks: column-split kernel; repeated 9 times: block-per-wave kernel)."""
    say("encode edge values x%d" % reps)
    rng = np.random.default_rng(8)
    k = np.zeros((1, 64 * 8, 128), dtype=np.float16)
    k[0, 64:128] = rng.standard_normal((64, 128)).astype(np.float16)
    k[0, 64, :] = np.float16(-0.0)
    k[0, 128:192] = np.float16(65504.0) * np.sign(rng.standard_normal((64, 128))).astype(np.float16)
    k[0, 192:256] = (rng.integers(-20, 20, (64, 128)) * 2.0 ** -24).astype(np.float16)
    a = np.float16(3.0)
    grid = (np.arange(-8, 9) * (float(a) / 8)).astype(np.float16)
    blk = np.resize(grid, (64, 128)).astype(np.float16)
    k[0, 256:320] = blk
    k[0, 320:384] = np.nextafter(blk, np.float16(np.inf))
    k[0, 384:448] = -blk
    k[0, 448:512] = rng.standard_normal((64, 128)).astype(np.float16) * np.float16(1e-3)
    k = np.ascontiguousarray(np.tile(k, (1, reps, 1)))
    gp, gs, flag = _gpu_encode(fk, k)
    op, os_, bad = oracle.encode(k)
    assert flag == 0 and bad == 0
    assert np.array_equal(gp, op), first_mismatch(gp, op)
    assert np.array_equal(gs, os_), first_mismatch(gs, os_)


@pytest.mark.parametrize("nblk", [4, 80])
def test_encode_nonfinite_flag(fk, nblk):
    say("encode non-finite flag nblk=%d" % nblk)
    k, _ = fathom_inputs.make_keys(2, 64 * nblk, seed=9)
    _, _, flag = _gpu_encode(fk, k)
    assert flag == 0
    k[1, 130, 17] = np.float16(np.inf)
    _, _, flag = _gpu_encode(fk, k)
    assert flag == 1
    k[1, 130, 17] = np.float16(np.nan)
    _, _, flag = _gpu_encode(fk, k)
    assert flag == 1


def _gpu_plan(fk, q, var, B):
    import torch
    groups = q.shape[0]
    theta = torch.zeros(groups, dtype=torch.float64, device="cuda")
    bits = torch.zeros(groups, dtype=torch.int32, device="cuda")
    dep = fk.plan(to_dev(q), to_dev(var), B, theta=theta, bits_used=bits)
    torch.cuda.synchronize()
    return to_host(dep), to_host(theta), to_host(bits)


def test_plan_appendix_a(fk, golden_dir):
    """The Appendix A example embedded in 128 channels (the other 124 have
    zero variance, so g = 0 and t = 0)."""
    gold = json.load(open(os.path.join(golden_dir, "appendix_a.json")))
    q = np.zeros((1, 2, 128), dtype=np.float32)
    q[0, 0, :4] = gold["q_A"]
    q[0, 1, :4] = gold["q_B"]
    var = np.zeros((1, 128), dtype=np.float32)
    var[0, :4] = gold["var"]
    for row in gold["plans"]:
        say("plan appendix A B=%d" % row["budget"])
        dep, theta, bits = _gpu_plan(fk, q, var, row["budget"])
        assert list(dep[0, :4]) == row["depths"] and not dep[0, 4:].any()
        od, ot, ob = oracle.plan(q, var, row["budget"])
        assert np.array_equal(dep, od) and theta[0] == ot[0] and bits[0] == ob[0]


@pytest.mark.parametrize("G", [1, 2, 3, 4, 8])
def test_plan_matches_oracle(fk, G):
    rng = np.random.default_rng(200 + G)
    groups = 64
    q = rng.standard_normal((groups, G, 128)).astype(np.float32)
    var = np.exp(rng.standard_normal((groups, 128)) * 2).astype(np.float32)
    var[3, :] = 0.0                                   # all g = 0
    var[5, 10:] = 0.0                                 # 10 positive channels
    q[7, :, 20:40] = 0.0
    for B in (0, 1, 2, 5, 17, 40, 48, 68, 92, 136, 300, 511, 512):
        say("plan G=%d B=%d" % (G, B))
        dep, theta, bits = _gpu_plan(fk, q, var, B)
        od, ot, ob = oracle.plan(q, var, B)
        assert np.array_equal(dep, od), first_mismatch(dep, od)
        assert np.array_equal(theta.view(np.uint64), ot.view(np.uint64)), first_mismatch(theta, ot)
        assert np.array_equal(bits, ob)
        assert np.all(bits <= B)


def test_plan_q1m_queries(fk):
    """Plans of the 1M-key Qwen3-shaped workload's queries and variances."""
    w = fathom_inputs.WORKLOADS["q256k"]
    ins = fathom_inputs.make_inputs(w.groups, w.G, 4096, w.seed)
    for B in w.budgets:
        say("plan q256k-shaped B=%d" % B)
        dep, theta, bits = _gpu_plan(fk, ins.q, ins.var, B)
        od, ot, ob = oracle.plan(ins.q, ins.var, B)
        assert np.array_equal(dep, od) and np.array_equal(theta, ot) and np.array_equal(bits, ob)


# --------------------------------------------------------------------------
# Fixed-depth plans
# --------------------------------------------------------------------------

@pytest.mark.parametrize("G", [1, 4, 8])
def test_plan_fixed_matches_oracle(fk, G):
    import torch
    rng = np.random.default_rng(60 + G)
    groups = 9
    q = rng.standard_normal((groups, G, 128)).astype(np.float32)
    q[1] = np.round(q[1])                      # many equal |q| sums
    q[2] = 1.0                                 # all equal
    stat = rng.integers(0, 5, size=(groups, 128)).astype(np.float32)
    say("plan_fixed G=%d" % G)
    for t in range(5):
        got = to_host(fk.plan_fixed("uniform", t, groups=groups, G=G))
        torch.cuda.synchronize()
        assert np.array_equal(got, oracle.plan_fixed("uniform", t, groups=groups))
    for r in (0, 1, 16, 32, 127, 128):
        got = to_host(fk.plan_fixed("sparq", r, q=to_dev(q)))
        ref = oracle.plan_fixed("sparq", r, q=q)
        assert np.array_equal(got, ref), (r, first_mismatch(got, ref))
        got = to_host(fk.plan_fixed("topstat", r, stat=to_dev(stat), G=G))
        ref = oracle.plan_fixed("topstat", r, stat=stat)
        assert np.array_equal(got, ref), (r, first_mismatch(got, ref))


# --------------------------------------------------------------------------
# The decode step's append and plan as one call
# --------------------------------------------------------------------------

@pytest.mark.parametrize("G,nblk_new,offset", [(1, 1, 69), (4, 3, 10), (8, 1, 0), (4, 65, 2)])
def test_append_plan_matches_two_calls(fk, G, nblk_new, offset):
    """fathom_append_plan against fathom_encode then fathom_plan on copies of
    the same store, bit for bit: every plane word and scale of the store, the
    depths, water lines and bit counts.  One launch for appends of 1 and 3
    blocks; 65 blocks (more than 64) takes the two launches."""
    import torch
    groups, nb_store, B = 3, 70 + 64, 92
    ins = fathom_inputs.make_inputs(groups, G, 64 * nb_store, seed=300 + G)
    base = torch.from_numpy(ins.k[:, :64 * nb_store].copy()).cuda()
    p0, s0 = fk.encode(base)                               # a full store to append into
    new = torch.from_numpy(ins.k[:, ::-1][:, :64 * nblk_new].copy()).cuda()
    q, var = to_dev(ins.q), to_dev(ins.var)
    say("append_plan G=%d blocks=%d offset=%d" % (G, nblk_new, offset))
    pa, sa = p0.clone(), s0.clone()
    pb, sb = p0.clone(), s0.clone()
    da = torch.empty((groups, 128), dtype=torch.uint8, device="cuda")
    ta = torch.empty(groups, dtype=torch.float64, device="cuda")
    ba = torch.empty(groups, dtype=torch.int32, device="cuda")
    fk.append_plan(new, pa, sa, offset, q, var, B, depths=da, theta=ta, bits_used=ba)
    tb = torch.empty(groups, dtype=torch.float64, device="cuda")
    bb = torch.empty(groups, dtype=torch.int32, device="cuda")
    fk.encode(new, pb, sb, block_offset=offset)
    db = fk.plan(q, var, B, theta=tb, bits_used=bb)
    torch.cuda.synchronize()
    assert torch.equal(pa, pb) and torch.equal(sa, sb)
    assert not torch.equal(pa, p0)                         # the append wrote the store
    assert torch.equal(da, db) and torch.equal(ba, bb)
    assert np.array_equal(to_host(ta).view(np.uint64), to_host(tb).view(np.uint64))
    od, ot, ob = oracle.plan(ins.q, ins.var, B)
    assert np.array_equal(to_host(da), od)
