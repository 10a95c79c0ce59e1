"""coli_moe_block_noalloc -- the expert block on the library's static device
scratch (for callers that cannot allocate) -- against coli_moe_block with a
caller workspace and against the oracle, on two calls in a row, the second
smaller than the first (the scratch keeps the first call's contents)."""
import numpy as np
import pytest
import torch

import bit_gemv_coli_amd as coli
from gpu_util import TOL_FP32, need_gpu, qtensor, to_dev
from test_gpu_moe import _check_moe, _moe_inputs

pytestmark = pytest.mark.gpu


def _both(G, U, Dn, sh, x, ids, w):
    """(out from coli_moe_block_noalloc, out from coli_moe_block)."""
    S, K = ids.shape
    E, F, D = G.n, G.O, G.I
    tg, tu, td = qtensor(G, True), qtensor(U, True), qtensor(Dn, True)
    ts = [qtensor(m, True) for m in sh] if sh is not None else [None, None, None]
    xd, idd, wd = to_dev(x), to_dev(ids.astype(np.int32)), to_dev(w.astype(np.float32))
    a = torch.full((S, D), float("nan"), device="cuda")
    coli.check(coli.coli_moe_block_noalloc(tg, tu, td, xd, S, idd, wd, K, ts[0], ts[1], ts[2], a),
               "coli_moe_block_noalloc")
    wsb = coli.coli_moe_workspace_bytes(E, S, K, F, D, sh is not None)
    assert 0 < wsb <= coli.COLI_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    b = torch.full((S, D), float("nan"), device="cuda")
    coli.check(coli.coli_moe_block(tg, tu, td, xd, S, idd, wd, K, ts[0], ts[1], ts[2], b, ws, wsb),
               "coli_moe_block")
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


def test_noalloc_matches_workspace_block_two_calls(orc):
    need_gpu()
    # first call: S = 4, K = 8, shared expert; second: S = 1, K = 3, no shared
    cases = [(901, 4, 8, 16, 1024, 512, True), (902, 1, 3, 9, 512, 256, False)]
    for seed, S, K, E, D, F, shared in cases:
        G, U, Dn, sh, x, ids, w = _moe_inputs(seed, 4, S, K, E, D, F, 64, shared)
        a, b = _both(G, U, Dn, sh, x, ids, w)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (S, K)
        _check_moe(orc, G, U, Dn, sh, x, ids, w, a, None, TOL_FP32)


def test_noalloc_declines_beyond_the_scratch():
    """A block whose workspace exceeds the static scratch is declined on the
    host before anything is enqueued (tiny device buffers stand behind the
    descriptors: nothing reads them)."""
    need_gpu()
    E, D, F, S, K, gs = 256, 6144, 2048, 544, 8, 128
    assert coli.coli_moe_workspace_bytes(E, S, K, F, D, 0) > coli.COLI_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(16, dtype=torch.uint8, device="cuda")
    s = torch.zeros(16, dtype=torch.float32, device="cuda")
    tg = coli.QTensor(4, q, s, F, D, gs, n=E)
    td = coli.QTensor(4, q, s, D, F, gs, n=E)
    x = torch.zeros(64, device="cuda")
    ids = torch.zeros(64, dtype=torch.int32, device="cuda")
    out = torch.full((4,), 7.0, device="cuda")
    calls0 = coli.coli_stats()[2]
    rc = coli.coli_moe_block_noalloc(tg, tg, td, x, S, ids, x, K, None, None, None, out)
    assert rc == coli.COLI_DECLINED
    assert "scratch" in coli.coli_last_reason()
    torch.cuda.synchronize()
    assert coli.coli_stats()[2] == calls0  # no launch
    assert torch.all(out == 7.0)
