"""fathom_topk_noalloc (the top-k for callers that cannot allocate) against
fathom_topk with a caller workspace, through the C ABI: two calls in a row on
the library's fixed scratch, the second smaller than the first, each equal
to fathom_topk bit for bit (and to the oracle's selection)."""
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


def test_noalloc_matches_workspace_call(fk):
    import torch
    cases = [(32, 1 << 20, 4096, "normal", 11), (3, 70000, 1000, "ties", 12)]
    for rows, n, k, kind, seed in cases:
        scores = fathom_inputs.random_scores(rows, n, seed=seed, kind=kind)
        sd = to_dev(scores)
        idx_a = torch.empty((rows, k), dtype=torch.int32, device=sd.device)
        idx_b = torch.full((rows, k), -1, dtype=torch.int32, device=sd.device)
        say("topk noalloc rows=%d n=%d k=%d kind=%s" % (rows, n, k, kind))
        fk.topk(sd, k, indices=idx_a)
        fk.topk_noalloc(sd, k, idx_b)
        torch.cuda.synchronize()
        a, b = to_host(idx_a), to_host(idx_b)
        assert np.array_equal(a, b), first_mismatch(a, b)
        ref = oracle.topk(scores, k)
        assert np.array_equal(b, ref), first_mismatch(b, ref)


def test_noalloc_rejects_too_large(fk):
    """A call beyond the fixed scratch returns FATHOM_ERR_TOO_LARGE before
    any GPU work."""
    import torch
    rows, n, k = 512, 131072, 1024
    assert fk.topk_workspace_bytes(rows, n, k) > fk.lib().fathom_topk_noalloc_max_bytes()
    sd = torch.zeros((rows, n), dtype=torch.float32, device="cuda")
    idx = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    with pytest.raises(fk.FathomError) as e:
        fk.topk_noalloc(sd, k, idx)
    assert e.value.status == -9
