"""Parity of the 75-layer decode stream's layers 0 and 74, drawn exactly as
the benchmark draws them (same seeded device generators): the grouped launch
of the four attention projections at their full shapes (q_a 1536x6144, q_b
16384x1536, kv_a 576x6144, o_proj 6144x16384, one coli_qmatmul_group call on
packed copies) and the expert block with 8 routed experts from a pool of 20
plus the shared expert, all fmt 4 gs 64, S = 1 (colibri-strix commit log,
full decode layer commit: a layer's projections and its block go to the GPU
together).  Bounds: the decode GEMV bound with the matrix-core term, and the
expert block's staged bound (test_gpu_moe)."""
import numpy as np
import pytest
import torch

import bit_gemv_coli_amd as coli
import synthdata as sd
from gpu_util import TOL_FP32, assert_within, need_gpu, rep_allowance
from oracle import QMat
from test_gpu_moe import _check_moe

pytestmark = pytest.mark.gpu

D, F, K, GS, POOL = 6144, 2048, 8, 64, 20
PROJS = [(1536, 6144), (16384, 1536), (576, 6144), (6144, 16384)]


@pytest.mark.parametrize("layer", [0, 74])
def test_layer_stream_layer_matches_oracle(orc, layer):
    need_gpu()
    dev = "cuda"
    # the benchmark's draws for this layer
    P = [sd.pool_on_device(1000 + 10 * layer + i, 4, 1, o, i_, GS) for i, (o, i_) in enumerate(PROJS)]
    TP = [coli.QTensor(4, q[0], s[0], o, i_, GS, n=1) for (q, s), (o, i_) in zip(P, PROJS)]
    for t in TP:
        assert t.pack()
    g = torch.Generator(device=dev)
    g.manual_seed(4242 + layer)
    xs = [torch.randn((1, i_), device=dev, generator=g) for _, i_ in PROJS]
    ys = [torch.full((1, o), float("nan"), device=dev) for o, _ in PROJS]
    coli.check(coli.coli_qmatmul_group(TP, xs, ys, 1), "coli_qmatmul_group")
    torch.cuda.synchronize()
    for (q, s), (o, i_), x, y in zip(P, PROJS, xs, ys):
        W = QMat(4, o, i_, GS, q[0].cpu().numpy(), s[0].cpu().numpy())
        xh = x.cpu().numpy()
        yr, A = orc.qmatmul(W, xh)
        assert_within(y.cpu().numpy(), yr, A, TOL_FP32, f"layer {layer} proj {o}x{i_}",
                      rep_allowance(orc, W, xh))
    del P, TP
    # the expert block: 8 of the 20 pooled experts and the shared one
    mg = sd.pool_on_device(5000 + 4 * layer, 4, POOL + 1, F, D, GS)
    mu = sd.pool_on_device(5001 + 4 * layer, 4, POOL + 1, F, D, GS)
    md = sd.pool_on_device(5002 + 4 * layer, 4, POOL + 1, D, F, GS)
    tg = coli.QTensor(4, mg[0][:POOL], mg[1][:POOL], F, D, GS)
    tu = coli.QTensor(4, mu[0][:POOL], mu[1][:POOL], F, D, GS)
    td = coli.QTensor(4, md[0][:POOL], md[1][:POOL], D, F, GS)
    sg = coli.QTensor(4, mg[0][POOL], mg[1][POOL], F, D, GS, n=1)
    su = coli.QTensor(4, mu[0][POOL], mu[1][POOL], F, D, GS, n=1)
    sdn = coli.QTensor(4, md[0][POOL], md[1][POOL], D, F, GS, n=1)
    for t in (tg, tu, td, sg, su, sdn):
        assert t.pack()
    r = sd.rng(75)
    routes = [sd.gen_routing_uniform(r, 1, K, POOL) for _ in range(75)]
    ids, w = routes[layer]
    x = torch.randn((1, D), device=dev, generator=g)
    out = torch.full((1, D), float("nan"), device=dev)
    wsb = coli.coli_moe_workspace_bytes(POOL, 1, K, F, D, 1)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    idd, wd = torch.from_numpy(ids).to(dev), torch.from_numpy(w).to(dev)
    coli.check(coli.coli_moe_block(tg, tu, td, x, 1, idd, wd, K, sg, su, sdn, out, ws, wsb),
               "coli_moe_block")
    h = torch.full((K + 1, F), float("nan"), device=dev)
    coli.check(coli.coli_moe_hidden(tg, tu, x, 1, idd, K, sg, su, h, ws, wsb), "coli_moe_hidden")
    torch.cuda.synchronize()
    sel = torch.from_numpy(ids[0].astype(np.int64)).to(dev)
    G = QMat(4, F, D, GS, mg[0][sel].cpu().numpy(), mg[1][sel].cpu().numpy())
    U = QMat(4, F, D, GS, mu[0][sel].cpu().numpy(), mu[1][sel].cpu().numpy())
    Dn = QMat(4, D, F, GS, md[0][sel].cpu().numpy(), md[1][sel].cpu().numpy())
    sh = (QMat(4, F, D, GS, mg[0][POOL].cpu().numpy(), mg[1][POOL].cpu().numpy()),
          QMat(4, F, D, GS, mu[0][POOL].cpu().numpy(), mu[1][POOL].cpu().numpy()),
          QMat(4, D, F, GS, md[0][POOL].cpu().numpy(), md[1][POOL].cpu().numpy()))
    local = np.arange(K, dtype=np.int32)[None, :]
    _check_moe(orc, G, U, Dn, sh, x.cpu().numpy(), local, w, out.cpu().numpy(), h.cpu().numpy(),
               TOL_FP32)
