"""The expert block and the matmul inside a captured HIP graph (the pages'
full decode layer commit: a block is one submission).  Each
graph is replayed several times with eager library work and host
synchronisations between the replays, and every replay must reproduce the
eager result bit for bit (the kernels are deterministic; nothing in the
library records a memset or an allocation)."""
import numpy as np
import pytest
import torch

import bit_gemv_coli_amd as coli
from gpu_util import make_case, need_gpu, qtensor, to_dev
from test_gpu_moe import _moe_inputs

pytestmark = pytest.mark.gpu


def _replays_match(run, outs, reps=3, between=None):
    """Capture run() (which writes the tensors in outs), compare every replay
    with the eager values."""
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for r in range(reps):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else -7)
        if between is not None:
            between()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(o.view(torch.int32), e.view(torch.int32)), f"replay {r} differs"
    del g


def _block(S, pack, seed):
    G, U, Dn, sh, x, ids, w = _moe_inputs(seed, 4, S, 4, 8, 256, 128, 64 if S <= 4 else 128, True)
    tg, tu, td = qtensor(G, pack), qtensor(U, pack), qtensor(Dn, pack)
    ts = [qtensor(m, pack) for m in sh]
    xd, idd, wd = to_dev(x), to_dev(ids.astype(np.int32)), to_dev(w.astype(np.float32))
    ws_bytes = coli.coli_moe_workspace_bytes(8, S, 4, 128, 256, 1)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((S, 256), device="cuda")

    def run():
        coli.check(coli.coli_moe_block(tg, tu, td, xd, S, idd, wd, 4, ts[0], ts[1], ts[2], out, ws,
                                       ws_bytes, torch.cuda.current_stream()), "coli_moe_block")
    return run, out, (tg, tu, td, ts, xd, idd, wd, ws)


@pytest.mark.parametrize("S,pack", [(1, True), (3, True), (1, False), (40, True), (40, False)],
                         ids=["decode-S1-packed", "decode-S3-packed", "decode-S1-plain",
                              "prefill-S40-packed", "prefill-S40-plain"])
def test_moe_block_graph_replays(S, pack):
    need_gpu()
    run, out, keep = _block(S, pack, 900 + S)
    # eager work between replays: another block on the same stream
    run2, out2, keep2 = _block(2, True, 7)
    _replays_match(run, [out], between=run2)


@pytest.mark.parametrize("S", [1, 4, 96])
def test_qmatmul_graph_replays(S):
    need_gpu()
    W, x = make_case(4, 640, 1024, 64, S, seed=31 + S)
    T = qtensor(W, pack=True)
    xd = to_dev(x.astype(np.float32))
    y = torch.empty((S, 640), device="cuda")
    W2, x2 = make_case(4, 64, 256, 64, 2, seed=5)
    T2 = qtensor(W2, pack=True)
    x2d = to_dev(x2.astype(np.float32))
    y2 = torch.empty((2, 64), device="cuda")

    def run():
        coli.check(coli.coli_qmatmul(T, xd, y, S, torch.cuda.current_stream()), "coli_qmatmul")

    def between():
        coli.check(coli.coli_qmatmul(T2, x2d, y2, 2), "coli_qmatmul")
    _replays_match(run, [y], between=between)


@pytest.mark.parametrize("S", [1, 4, 96])
def test_router_graph_replays(S):
    """The router and top-K (decode rows, and many rows through the split
    matrix-core logits) replayed from a graph."""
    need_gpu()
    import synthdata as sd
    E, D, K = 64, 512, 6
    r = sd.rng(300 + S)
    x = to_dev(sd.gen_x(r, S, D))
    R = to_dev((r.standard_normal((E, D)) / np.sqrt(D)).astype(np.float32))
    bias = to_dev((r.standard_normal(E) * 0.05).astype(np.float32))
    ids = torch.empty((S, K), dtype=torch.int32, device="cuda")
    w = torch.empty((S, K), device="cuda")
    wsb = coli.coli_moe_router_workspace_bytes(S, E)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")

    def run():
        coli.check(coli.coli_moe_router(x, S, D, R, bias, E, K, 0.7, 1, 2.5, ids, w, ws, wsb,
                                        torch.cuda.current_stream()), "coli_moe_router")
    _replays_match(run, [ids, w], between=lambda: ws.fill_(0xFF))


def test_moe_layer_graph_replays():
    """Norm, router, top-K, shared + routed experts and the residual add of
    the expert half of a layer, replayed from one graph (in place on a copy
    of h restored before each replay)."""
    need_gpu()
    import synthdata as sd
    S, K, E, D, F = 1, 8, 16, 256, 128
    G, U, Dn, sh, x, _, _ = _moe_inputs(808, 4, S, K, E, D, F, 64, True)
    r = sd.rng(809)
    tg, tu, td = qtensor(G, True), qtensor(U, True), qtensor(Dn, True)
    ts = [qtensor(m, True) for m in sh]
    h0 = to_dev(x)
    h = h0.clone()
    lnw = to_dev(r.uniform(0.5, 1.5, D).astype(np.float32))
    R = to_dev((r.standard_normal((E, D)) / 16).astype(np.float32))
    wsb = coli.coli_moe_layer_workspace_bytes(E, S, K, F, D, True)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(h)

    def run():
        coli.check(coli.coli_moe_layer(tg, tu, td, h, S, lnw, 1e-6, R, None, K, 0.0, 1, 2.5,
                                       ts[0], ts[1], ts[2], out, ws, wsb,
                                       torch.cuda.current_stream()), "coli_moe_layer")
    _replays_match(run, [out], between=lambda: ws.fill_(0x7F))


@pytest.mark.parametrize("S", [1, 4])
def test_graph_grouped_gemv(S):
    """coli_qmatmul_group (one launch for independent matrices, the way the
    layer stream captures a layer's projections) replayed from a graph, with
    single-matrix calls on other data between the replays."""
    need_gpu()
    shapes = [(1536, 640), (1024, 1536), (576, 640), (640, 2048)]
    Ts, xs, ys = [], [], []
    for j, (O, I) in enumerate(shapes):
        W, x = make_case(4, O, I, 64, S, seed=60 + j)
        Ts.append(qtensor(W, pack=True))
        xs.append(to_dev(x))
        ys.append(torch.empty((1, S, O), device="cuda"))
    Wb, xb = make_case(4, 512, 1024, 64, S, seed=70)
    Tb, xbd = qtensor(Wb, pack=True), to_dev(xb)
    yb = torch.empty((1, S, 512), device="cuda")

    def run():
        coli.check(coli.coli_qmatmul_group(Ts, xs, ys, S), "coli_qmatmul_group")

    def between():
        coli.check(coli.coli_qmatmul(Tb, xbd, yb, S), "coli_qmatmul")

    _replays_match(run, ys, between=between)


@pytest.mark.parametrize("S", [1, 40])
def test_graph_two_phase_block(S):
    """coli_moe_block_begin and coli_moe_block_end captured together and
    replayed, with a one-submission block on other data between replays."""
    need_gpu()
    K, E, D, F = 4, 8, 256, 128
    gs = 64 if S <= 4 else 128
    G, U, Dn, sh, x, ids, w = _moe_inputs(90 + S, 4, S, K, E, D, F, gs, True)
    tg, tu, td = qtensor(G, True), qtensor(U, True), qtensor(Dn, True)
    ts = [qtensor(m, True) for m in sh]
    xd, idd, wd = to_dev(x), to_dev(ids), to_dev(w)
    late = to_dev((np.arange(S * K).reshape(S, K) % 3 == 1).astype(np.int32))
    wsb = coli.coli_moe_block_two_phase_workspace_bytes(E, S, K, F, D, True)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty((S, D), device="cuda")
    G2, U2, D2, sh2, x2, ids2, w2 = _moe_inputs(91 + S, 4, S, K, E, D, F, gs, False)
    t2 = [qtensor(m, True) for m in (G2, U2, D2)]
    x2d, ids2d, w2d = to_dev(x2), to_dev(ids2), to_dev(w2)
    wsb2 = coli.coli_moe_workspace_bytes(E, S, K, F, D, 0)
    ws2 = torch.empty(wsb2, dtype=torch.uint8, device="cuda")
    out2 = torch.empty((S, D), device="cuda")

    def run():
        coli.check(coli.coli_moe_block_begin(tg, tu, td, xd, S, idd, wd, K, late, ts[0], ts[1], ts[2],
                                             out, ws, wsb), "begin")
        coli.check(coli.coli_moe_block_end(tg, tu, td, xd, S, wd, K, True, out, ws, wsb), "end")

    def between():
        coli.check(coli.coli_moe_block(t2[0], t2[1], t2[2], x2d, S, ids2d, w2d, K, None, None, None,
                                       out2, ws2, wsb2), "coli_moe_block")

    _replays_match(run, [out], between=between)


def test_layer_decode_graph_replays():
    """A whole decode layer (attention with its cache writes, residual, expert
    half) captured as one graph: every replay reproduces the eager output and
    cache rows bit for bit, with an eager layer on other buffers between the
    replays."""
    need_gpu()
    from test_gpu_mla import SMALL, _setup as setup_attention
    S, pb, E, F, K = 3, 6, 8, 64, 4
    D = SMALL["D"]

    def make(seed):
        W, layer, x, Lc, Rc, T = setup_attention(seed, S, pb, SMALL)
        G, U, Dn, sh, _, _, _ = _moe_inputs(seed + 1, 4, S, K, E, D, F, 32, True)
        R = (np.random.default_rng(seed).standard_normal((E, D)) / np.sqrt(D)).astype(np.float32)
        tg, tu, td = qtensor(G, True), qtensor(U, True), qtensor(Dn, True)
        ts = [qtensor(m, True) for m in sh]
        total = coli.coli_layer_decode_workspace_bytes(layer, tg, S, K, T, True)
        ws = torch.empty(total, dtype=torch.uint8, device="cuda")
        xd, Rd, Lc_d, Rc_d = to_dev(x), to_dev(R), to_dev(Lc), to_dev(Rc)
        out = torch.empty((S, D), device="cuda")

        def run():
            coli.check(coli.coli_layer_decode(layer, None, tg, tu, td, None, Rd, None, K, 0.0, 1,
                                              1.0, ts[0], ts[1], ts[2], 1e-6, xd, S, pb, Lc_d,
                                              Rc_d, T, out, ws, total,
                                              torch.cuda.current_stream()), "coli_layer_decode")
        return run, [out, Lc_d, Rc_d], (layer, tg, tu, td, ts, ws, xd, Rd)
    run, outs, keep = make(950)
    run2, _, keep2 = make(960)
    out, Lc_d, Rc_d = outs
    # the caches are inputs too (rows below pb): only this call's rows are
    # cleared before each replay
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(float("nan"))
        Lc_d[pb:pb + S].fill_(float("nan"))
        Rc_d[pb:pb + S].fill_(float("nan"))
        run2()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(o.view(torch.int32), e.view(torch.int32)), f"replay {r} differs"
    del g
