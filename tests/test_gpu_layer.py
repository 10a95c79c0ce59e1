"""GPU parity of the steps around the expert block (colibri-strix commit
log, full decode layer commit: post-attention
RMSNorm, router with the exact top-K, shared + routed experts, residual add)
against the oracle.

  * coli_rmsnorm: every output within the f32 rounding of the oracle's f64
    value (both take the mean of squares and the product in f64);
  * the same norm, router and top-K called step by step: picks bit-exact
    against the oracle's on the oracle's normed rows;
  * coli_moe_layer end to end, in place (out = h): out - h against the
    oracle's block on the oracle's normed rows and picks, within the block's
    bound (the f32 add of h rounds once more, by at most 2^-24 |out|)."""
import numpy as np
import pytest
import torch

import bit_gemv_coli_amd as coli
import synthdata as sd
from gpu_util import TOL_BF16, TOL_FP32, need_gpu, qtensor, to_dev
from test_gpu_moe import _check_moe, _moe_inputs

pytestmark = pytest.mark.gpu

NORM = [  # (S, D, eps, weighted, misaligned)
    (1, 6144, 1e-6, True, False),
    (4, 6144, 1e-6, True, False),
    (5, 100, 1e-5, False, False),
    (3, 33, 0.0, True, False),
    (2, 512, 1e-6, True, True),
    (544, 256, 1e-6, True, False),
]


@pytest.mark.parametrize("case", NORM, ids=["S{}-D{}-eps{}-w{}-mis{}".format(*c) for c in NORM])
def test_rmsnorm_matches_oracle(orc, case):
    need_gpu()
    S, D, eps, weighted, mis = case
    r = sd.rng(2000 + S + D)
    x = (sd.gen_x(r, S, D) * r.uniform(0.01, 30.0, (S, 1))).astype(np.float32)
    w = r.uniform(0.5, 1.5, D).astype(np.float32) if weighted else None
    if mis:  # rows starting 4 bytes past a 16-byte boundary (the scalar path)
        buf = torch.zeros(S * D + 1, device="cuda")
        buf[1:] = to_dev(x.reshape(-1))
        xd = buf[1:]
        yb = torch.full((S * D + 1,), float("nan"), device="cuda")
        yd = yb[1:]
    else:
        xd = to_dev(x)
        yd = torch.full((S, D), float("nan"), device="cuda")
    wd = None if w is None else to_dev(w)
    coli.check(coli.coli_rmsnorm(xd, S, D, wd, eps, yd), "coli_rmsnorm")
    torch.cuda.synchronize()
    y = yd.cpu().numpy().reshape(S, D).astype(np.float64)
    ref = orc.rmsnorm(x, w, eps)
    err = np.abs(y - ref)
    assert np.all(err <= 2.0 ** -24 * np.abs(ref) * 1.0001), float(np.max(err / np.abs(ref)))


def test_rmsnorm_in_place_and_declines(orc):
    need_gpu()
    S, D = 3, 256
    x = sd.gen_x(sd.rng(5), S, D)
    xd = to_dev(x)
    coli.check(coli.coli_rmsnorm(xd, S, D, None, 1e-6, xd), "coli_rmsnorm in place")
    torch.cuda.synchronize()
    ref = orc.rmsnorm(x, None, 1e-6)
    assert np.all(np.abs(xd.cpu().numpy() - ref) <= 2.0 ** -24 * np.abs(ref) * 1.0001)
    y = torch.empty((S, D), device="cuda")
    assert coli.coli_rmsnorm(xd, S, D, None, -1.0, y) == coli.COLI_DECLINED
    assert coli.coli_rmsnorm(xd, 0, D, None, 1e-6, y) == coli.COLI_DECLINED
    assert coli.coli_rmsnorm(None, S, D, None, 1e-6, y) == coli.COLI_DECLINED


LAYER = [  # (S, K, E, D, F, gs, shared, topp, pack)
    (1, 8, 16, 256, 128, 64, True, 0.0, True),
    (1, 4, 32, 512, 128, 32, False, 0.7, False),
    (3, 4, 12, 256, 96, 32, True, 0.0, True),
    (4, 6, 64, 512, 128, 64, True, 0.9, True),
    (24, 4, 16, 256, 128, 64, True, 0.0, True),   # prefill path (bf16 matrix cores)
    (40, 8, 32, 512, 256, 128, False, 0.8, True),
]


def _layer_inputs(case, seed):
    S, K, E, D, F, gs, shared, topp, pack = case
    G, U, Dn, sh, x, _, _ = _moe_inputs(seed, 4, S, K, E, D, F, gs, shared)
    r = sd.rng(seed + 1)
    h = (x * 3.0).astype(np.float32)
    ln_w = r.uniform(0.5, 1.5, D).astype(np.float32)
    R = (r.standard_normal((E, D)) / np.sqrt(D)).astype(np.float32)
    bias = (r.standard_normal(E) * 0.05).astype(np.float32)
    return G, U, Dn, sh, h, ln_w, R, bias


@pytest.mark.parametrize("case", LAYER, ids=["S{}-K{}-E{}-D{}-F{}-g{}-sh{}-p{}-pk{}".format(*c)
                                             for c in LAYER])
def test_moe_layer_matches_oracle(orc, case):
    need_gpu()
    S, K, E, D, F, gs, shared, topp, pack = case
    eps, norm, scale = 1e-6, True, 2.5
    G, U, Dn, sh, h, ln_w, R, bias = _layer_inputs(case, 3000 + S + E)
    out_ref, st = orc.moe_layer(h, ln_w, eps, R, bias, K, topp, norm, scale, G, U, Dn, shared=sh)
    tg, tu, td = qtensor(G, pack), qtensor(U, pack), qtensor(Dn, pack)
    ts = [qtensor(m, pack) for m in sh] if sh is not None else [None, None, None]
    hd, lnd, Rd, bd = to_dev(h), to_dev(ln_w), to_dev(R), to_dev(bias)
    # the steps one by one: normed rows and picks
    xn = torch.full((S, D), float("nan"), device="cuda")
    coli.check(coli.coli_rmsnorm(hd, S, D, lnd, eps, xn), "coli_rmsnorm")
    ids = torch.empty((S, K), dtype=torch.int32, device="cuda")
    w = torch.empty((S, K), device="cuda")
    rwb = coli.coli_moe_router_workspace_bytes(S, E)
    rws = torch.empty(rwb, dtype=torch.uint8, device="cuda")
    coli.check(coli.coli_moe_router(xn, S, D, Rd, bd, E, K, topp, norm, scale, ids, w, rws, rwb),
               "coli_moe_router")
    # the layer in one call, in place (out = h)
    wsb = coli.coli_moe_layer_workspace_bytes(E, S, K, F, D, sh is not None)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = hd.clone()
    coli.check(coli.coli_moe_layer(tg, tu, td, out, S, lnd, eps, Rd, bd, K, topp, norm, scale,
                                   ts[0], ts[1], ts[2], out, ws, wsb), "coli_moe_layer")
    torch.cuda.synchronize()
    xn_g = xn.cpu().numpy()
    assert np.all(np.abs(xn_g - st["xn"]) <= 2.0 ** -24 * np.abs(st["xn"]) * 1.0001)
    assert np.array_equal(ids.cpu().numpy(), st["ids"])
    # inside the layer call (workspace: normed rows, then the picks) the norm
    # may be folded into the router: the same bits as the separate steps
    wsh = ws.cpu().numpy()
    xn_l = wsh[:S * D * 4].view(np.float32).reshape(S, D)
    at = (S * D * 4 + 255) // 256 * 256
    ids_l = wsh[at:at + S * K * 4].view(np.int32).reshape(S, K)
    assert np.array_equal(xn_l.view(np.uint32), xn_g.view(np.uint32)), "layer's normed rows"
    assert np.array_equal(ids_l, st["ids"]), "layer's picks"
    y_est = out.cpu().numpy().astype(np.float64) - h.astype(np.float64)
    tau = TOL_FP32 if S <= 4 else TOL_BF16
    # the f32 add of h rounds once more (<= 2^-24 |out|), far inside the bound
    _check_moe(orc, G, U, Dn, sh, st["xn"], st["ids"], st["w"].astype(np.float32), y_est, None, tau)


def test_moe_layer_declines():
    need_gpu()
    case = LAYER[0]
    S, K, E, D, F, gs, shared, topp, pack = case
    G, U, Dn, sh, h, ln_w, R, bias = _layer_inputs(case, 77)
    tg, tu, td = qtensor(G, pack), qtensor(U, pack), qtensor(Dn, pack)
    hd, Rd = to_dev(h), to_dev(R)
    wsb = coli.coli_moe_layer_workspace_bytes(E, S, K, F, D, False)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(hd)
    args = lambda **kw: dict(dict(K=K, topp=0.0, ws=ws, wsb=wsb, R=Rd, eps=1e-6), **kw)
    def call(a):
        return coli.coli_moe_layer(tg, tu, td, hd, S, None, a["eps"], a["R"], None, a["K"],
                                   a["topp"], 1, 1.0, None, None, None, out, a["ws"], a["wsb"])
    assert call(args()) == coli.COLI_OK
    assert call(args(K=17)) == coli.COLI_DECLINED
    assert call(args(topp=1.5)) == coli.COLI_DECLINED
    assert call(args(eps=-1.0)) == coli.COLI_DECLINED
    assert call(args(R=None)) == coli.COLI_DECLINED
    assert call(args(wsb=wsb - 1)) == coli.COLI_DECLINED
    torch.cuda.synchronize()
