"""GPU router and exact top-K (colibri-strix commit log, full decode layer commit: router matvec + sigmoid, greedy argmax over
sigmoid + bias with the CPU's tie order, top-p truncation, norm_topk,
routed_scale) against the oracle: the picks bit-exact (both sides decide on
f64 keys), the f32 weights within the rounding of an f64 value."""
import numpy as np
import pytest
import torch

import bit_gemv_coli_amd as coli
import synthdata as sd
from gpu_util import need_gpu, to_dev

pytestmark = pytest.mark.gpu


def _gpu_router(x, R, bias, K, topp, norm, scale):
    S, D = x.shape
    E = R.shape[0]
    ids = torch.full((S, K), 12345, dtype=torch.int32, device="cuda")
    w = torch.full((S, K), float("nan"), device="cuda")
    wsb = coli.coli_moe_router_workspace_bytes(S, E)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    b = None if bias is None else to_dev(bias)
    coli.check(coli.coli_moe_router(to_dev(x), S, D, to_dev(R), b, E, K, topp, norm, scale, ids, w,
                                    ws, wsb), "coli_moe_router")
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def _check(orc, x, R, bias, K, topp, norm, scale):
    gi, gw = _gpu_router(x, R, bias, K, topp, norm, scale)
    oi, ow, _ = orc.moe_router(x, R, bias, K, topp, norm, scale)
    assert np.array_equal(gi, oi), f"picks differ in rows {np.nonzero((gi != oi).any(axis=1))[0][:5]}"
    err = np.abs(gw.astype(np.float64) - ow)
    assert np.all(err <= 2.0 ** -23 * np.abs(ow)), float(np.max(err))


CASES = [  # (S, D, E, K, topp, norm_topk, routed_scale, bias scale)
    (1, 6144, 256, 8, 0.0, True, 1.0, 0.05),     # decode at the block's shape
    (4, 6144, 256, 8, 0.6, True, 2.5, 0.05),
    (3, 100, 37, 5, 0.7, False, 2.5, 0.2),       # D not a multiple of 4, ragged E
    (17, 512, 64, 16, 0.9, True, 1.5, 0.3),      # K at its limit
    (2, 64, 512, 16, 0.0, True, 1.0, 0.1),       # E at its limit
    (9, 33, 1, 1, 0.5, True, 1.0, 0.0),          # one expert
    (40, 256, 96, 6, 1.0, False, 1.0, 0.0),      # topp = 1 keeps all, no bias
]


@pytest.mark.parametrize("case", CASES, ids=["S{}-D{}-E{}-K{}-p{}-n{}-sc{}-b{}".format(*c) for c in CASES])
def test_router_matches_oracle(orc, case):
    need_gpu()
    S, D, E, K, topp, norm, scale, bs = case
    r = sd.rng(1000 + S + E + K)
    x = sd.gen_x(r, S, D)
    R = (r.standard_normal((E, D)) / np.sqrt(D)).astype(np.float32)
    bias = (r.standard_normal(E) * bs).astype(np.float32) if bs > 0 else None
    _check(orc, x, R, bias, K, topp, norm, scale)


def test_router_prefill_rows(orc):
    """S = 544 rows at the block's shape (E 256, D 6144, K 8); 24 rows checked
    (every row's picks depend only on that row)."""
    need_gpu()
    S, D, E, K = 544, 6144, 256, 8
    r = sd.rng(544)
    x = sd.gen_x(r, S, D)
    R = (r.standard_normal((E, D)) / np.sqrt(D)).astype(np.float32)
    bias = (r.standard_normal(E) * 0.05).astype(np.float32)
    gi, gw = _gpu_router(x, R, bias, K, 0.0, True, 2.5)
    rows = np.sort(sd.rng(5).choice(S, 24, replace=False))
    oi, ow, _ = orc.moe_router(x[rows], R, bias, K, 0.0, True, 2.5)
    assert np.array_equal(gi[rows], oi)
    assert np.all(np.abs(gw[rows].astype(np.float64) - ow) <= 2.0 ** -23 * np.abs(ow))
    assert np.all((gi >= 0) & (gi < E)) and np.all([len(set(row)) == K for row in gi])


def test_router_exact_ties(orc):
    """Zero rows (every logit 0, every key 1/2 + bias) and duplicated router
    rows: equal keys go to the smaller expert index on both sides."""
    need_gpu()
    S, D, E, K = 6, 64, 40, 8
    r = sd.rng(77)
    x = sd.gen_x(r, S, D)
    x[0] = 0.0
    x[3] = 0.0
    R = (r.standard_normal((E, D)) / 8).astype(np.float32)
    R[5] = R[30]
    R[12] = R[30]
    R[2] = R[39]
    bias = np.zeros(E, np.float32)
    bias[[7, 19, 33]] = 0.25
    _check(orc, x, R, bias, K, 0.0, True, 1.0)
    _check(orc, x, R, None, K, 0.25, False, 1.0)  # at x = 0 the first pick reaches topp exactly
    # the same ties where the logits go through the matrix-core path with
    # the inputs split over several workgroups (partial sums added in order)
    S, D = 40, 1024
    x = sd.gen_x(r, S, D)
    x[[0, 17, 39]] = 0.0
    R = (r.standard_normal((E, D)) / 32).astype(np.float32)
    R[5] = R[30]
    R[12] = R[30]
    R[2] = R[39]
    _check(orc, x, R, bias, K, 0.0, True, 1.0)


def test_router_feeds_block(orc):
    """The router's ids and weights (with top-p drops) go straight into the
    expert block on the device."""
    need_gpu()
    from test_gpu_moe import _check_moe, _moe_inputs
    from gpu_util import TOL_FP32, qtensor
    S, K, E, D, F = 3, 4, 8, 256, 128
    G, U, Dn, sh, x, _, _ = _moe_inputs(606, 4, S, K, E, D, F, 64, False)
    r = sd.rng(7)
    R = (r.standard_normal((E, D)) / 16).astype(np.float32)
    gi, gw = _gpu_router(x, R, None, K, 0.8, True, 1.0)
    tg, tu, td = qtensor(G, True), qtensor(U, True), qtensor(Dn, True)
    wsb = coli.coli_moe_workspace_bytes(E, S, K, F, D, 0)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.full((S, D), float("nan"), device="cuda")
    coli.check(coli.coli_moe_block(tg, tu, td, to_dev(x), S, to_dev(gi), to_dev(gw), K, None, None,
                                   None, out, ws, wsb), "coli_moe_block")
    torch.cuda.synchronize()
    _check_moe(orc, G, U, Dn, None, x, gi, gw, out.cpu().numpy(), None, TOL_FP32)


def test_router_declines():
    need_gpu()
    x = torch.zeros((2, 16), device="cuda")
    R = torch.zeros((600, 16), device="cuda")
    ids = torch.zeros((2, 8), dtype=torch.int32, device="cuda")
    w = torch.zeros((2, 8), device="cuda")
    ws = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    assert coli.coli_moe_router(x, 2, 16, R, None, 600, 8, 0, 1, 1, ids, w, ws, 1 << 16) == coli.COLI_DECLINED
    assert coli.coli_moe_router(x, 2, 16, R, None, 32, 17, 0, 1, 1, ids, w, ws, 1 << 16) == coli.COLI_DECLINED
    assert coli.coli_moe_router(x, 2, 16, R, None, 32, 8, 1.5, 1, 1, ids, w, ws, 1 << 16) == coli.COLI_DECLINED
    assert coli.coli_moe_router(x, 2, 16, R, None, 32, 8, 0, 1, 1, ids, w, ws, 16) == coli.COLI_DECLINED
