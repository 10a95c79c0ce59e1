"""GPU parity of the MoE routing table (bit-exact) and the expert block
(colibri-strix commit log, batched expert-block commit: gate/up -> SiLU ->
down per routed expert, weighted combine; shared-expert fusion commit: the shared
expert adds with weight 1.0 on every row) against the oracle.

Checks per case:
  * hidden h = silu(G x) * (U x) against the oracle within
    eps_j = tau * (1.1 |u_j| A_g,j + |silu(g_j)| A_u,j)  (1.1 >= max |silu'|);
  * stagewise: out against sum_k w_k D_e h_gpu (+ shared), recomputed by the
    oracle from the GPU's own h, within tau * sum_k |w_k| A_D;
  * end to end: |out - out_ref| <= sum_k |w_k| (|D| eps + tau |D| (|h| + eps)).
tau = 1e-5 for the fp32 decode path (S <= 4), 4e-3 for the bf16 prefill path."""
import numpy as np
import pytest
import torch

import bit_gemv_coli_amd as coli
import synthdata as sd
from digit_model import REP_BOUND, block_magnitude
from gpu_util import (TOL_BF16, TOL_FP32, assert_within, decode_kernels, need_gpu, qtensor, to_dev,
                      zero_column)
from oracle import QMat

pytestmark = pytest.mark.gpu


def _moe_inputs(seed, fmt, S, K, E, D, F, gs, shared, routing="uniform"):
    r = sd.rng(seed)
    x = sd.gen_x(r, S, D)
    gq, gsc = sd.gen_matrix(r, fmt, F, D, gs, n=E)
    uq, usc = sd.gen_matrix(r, fmt, F, D, gs, n=E)
    dq, dsc = sd.gen_matrix(r, fmt, D, F, gs, n=E)
    g = 0 if fmt != 4 else gs
    G, U, Dn = QMat(fmt, F, D, g, gq, gsc), QMat(fmt, F, D, g, uq, usc), QMat(fmt, D, F, g, dq, dsc)
    sh = None
    if shared:
        a = sd.gen_matrix(r, fmt, F, D, gs)
        b = sd.gen_matrix(r, fmt, F, D, gs)
        c = sd.gen_matrix(r, fmt, D, F, gs)
        sh = (QMat(fmt, F, D, g, *a), QMat(fmt, F, D, g, *b), QMat(fmt, D, F, g, *c))
    if routing == "zipf":
        ids, w = sd.gen_routing_zipf(r, S, K, E, 1.1)
    else:
        ids, w = sd.gen_routing_uniform(r, S, K, E)
    return G, U, Dn, sh, x, ids, w


def _run_gpu(G, U, Dn, sh, x, ids, w, hidden=True, pack=True):
    S, K = ids.shape
    E, F, D = G.n, G.O, G.I
    tg, tu, td = qtensor(G, pack), qtensor(U, pack), qtensor(Dn, pack)
    ts = [qtensor(m, pack) for m in sh] if sh is not None else [None, None, None]
    xd, idd, wd = to_dev(x), to_dev(ids.astype(np.int32)), to_dev(w.astype(np.float32))
    ws_bytes = coli.coli_moe_workspace_bytes(E, S, K, F, D, sh is not None)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.full((S, D), float("nan"), device="cuda")
    coli.check(coli.coli_moe_block(tg, tu, td, xd, S, idd, wd, K, ts[0], ts[1], ts[2], out, ws,
                                   ws_bytes), "coli_moe_block")
    h = None
    if hidden:
        P = S * K + (S if sh is not None else 0)
        h = torch.full((P, F), float("nan"), device="cuda")
        coli.check(coli.coli_moe_hidden(tg, tu, xd, S, idd, K, ts[0], ts[1], h, ws, ws_bytes),
                   "coli_moe_hidden")
        h = h.cpu().numpy()
    torch.cuda.synchronize()
    return out.cpu().numpy(), h


def _check_moe(orc, G, U, Dn, sh, x, ids, w, out, h_gpu, tau, rows=None, rep=False):
    """rep=True adds the matrix-core decode kernels' input-resolution term
    2^-29 * Ahat to each stage's bound (gate/up on x, down on the GPU's h)."""
    S, K = ids.shape
    E = G.n
    D = Dn.O
    out_ref, inter = orc.moe_block(G, U, Dn, x, ids, w, shared=sh, rows=rows, intermediates=True)
    g, u, h, Ag, Au = (inter[k] for k in ("g", "u", "h", "Ag", "Au"))
    sil = g / (1.0 + np.exp(-g))
    # the bf16 path stores h in bf16 (8 significant bits: relative rounding <= 2^-8)
    hround = 2.0 ** -8 if tau > 1e-4 else 1e-6
    eps = tau * (1.1 * np.abs(u) * Ag + np.abs(sil) * Au) + hround * np.abs(h) + 1e-30
    P = S * K + (S if sh is not None else 0)
    valid = np.ones(P, bool)
    valid[:S * K] = (ids.reshape(-1) >= 0) & (ids.reshape(-1) < E)

    def pair(p):
        if p < S * K:
            e = int(ids.flat[p])
            return p // K, float(w.flat[p]), G.expert(e), U.expert(e), Dn.expert(e)
        return p - S * K, 1.0, sh[0], sh[1], sh[2]

    if rep:
        for p in range(P):
            if valid[p]:
                s_, _, Gm, Um, _ = pair(p)
                xs = x[s_:s_ + 1]
                rg = REP_BOUND * block_magnitude(np.abs(orc.dequant_f64(Gm)), xs)[0]
                ru = REP_BOUND * block_magnitude(np.abs(orc.dequant_f64(Um)), xs)[0]
                eps[p] += 1.1 * np.abs(u[p]) * rg + np.abs(sil[p]) * ru
    # 1. hidden vectors
    if h_gpu is not None:
        err = np.abs(h_gpu.astype(np.float64) - h)
        assert np.all(err[valid] <= eps[valid]), \
            f"hidden: max err/eps = {np.max(err[valid] / eps[valid]):.3e}"
        assert np.all(h_gpu[~valid] == 0.0)
    out_rows = out if rows is None else out[:, rows]
    # 2. stagewise down + combine from the GPU's own h (f32 exactly as stored)
    if h_gpu is not None:
        sel = np.arange(D) if rows is None else np.asarray(rows)
        y_st = np.zeros((S, len(sel)))
        A_st = np.zeros((S, len(sel)))
        R_st = np.zeros((S, len(sel)))
        for p in range(P):
            if not valid[p]:
                continue
            s, wk, _, _, Dm = pair(p)
            Dsel = QMat(Dm.fmt, len(sel), Dm.I, Dm.gs, np.ascontiguousarray(Dm.q[sel]),
                        np.ascontiguousarray(Dm.s[sel]))
            hp = h_gpu[p:p + 1].astype(np.float32)
            yk, Ak = orc.qmatmul(Dsel, hp)
            y_st[s] += wk * yk[0]
            A_st[s] += abs(wk) * Ak[0]
            if rep:
                R_st[s] += abs(wk) * REP_BOUND * block_magnitude(np.abs(orc.dequant_f64(Dsel)), hp)[0]
        assert_within(out_rows, y_st, A_st, tau, "stagewise down+combine", R_st if rep else None)
    # 3. end to end
    sel = np.arange(D) if rows is None else np.asarray(rows)
    bound = np.zeros((S, len(sel)))
    for p in range(P):
        if not valid[p]:
            continue
        s, wk, _, _, Dm = pair(p)
        Dsel = QMat(Dm.fmt, len(sel), Dm.I, Dm.gs, np.ascontiguousarray(Dm.q[sel]),
                    np.ascontiguousarray(Dm.s[sel]))
        Dabs = np.abs(orc.dequant_f64(Dsel))
        bound[s] += abs(wk) * (Dabs @ eps[p] + tau * (Dabs @ (np.abs(h[p]) + eps[p])))
        if rep and h_gpu is not None:
            bound[s] += abs(wk) * REP_BOUND * block_magnitude(Dabs, h_gpu[p:p + 1])[0]
    err = np.abs(out_rows.astype(np.float64) - out_ref)
    assert np.all(err <= bound + 1e-30), f"end to end: max err/bound = {np.max(err / bound):.3e}"


# S = 1 and 2 with long expert rows (F up to 2048) and every scale-slot count
DECODE_LONG_F = [  # (fmt, S, K, E, D, F, gs, shared)
    (4, 1, 8, 16, 256, 512, 64, True),
    (4, 1, 8, 16, 512, 2048, 64, False),
    (4, 1, 5, 9, 160, 1024, 32, True),      # gs 32: four scale slots per block
    (4, 1, 3, 7, 96, 1536, 128, True),      # gs 128: one slot
    (2, 1, 4, 8, 256, 512, 0, True),        # per-row scales
    (4, 1, 16, 40, 128, 512, 64, True),
    # more gate/up workgroups than two per compute unit (the one-quad variant)
    (4, 1, 8, 16, 256, 2048, 64, True),
    (4, 2, 8, 20, 256, 2048, 128, True),
    (2, 1, 12, 16, 128, 2048, 0, False),
]


@pytest.mark.parametrize("case", DECODE_LONG_F,
                         ids=["fmt{}-S{}-K{}-E{}-D{}-F{}-gs{}-sh{}".format(*c) for c in DECODE_LONG_F])
def test_moe_decode_long_rows_with_bad_ids(orc, case):
    need_gpu()
    fmt, S, K, E, D, F, gs, shared = case
    G, U, Dn, sh, x, ids, w = _moe_inputs(1500 + K + E + F, fmt, S, K, E, D, F, gs, shared)
    if K >= 5:  # an invalid id and a duplicate among the picks
        ids = ids.copy()
        ids[0, 1] = E + 3
        ids[0, 3] = ids[0, 2]
    out, h = _run_gpu(G, U, Dn, sh, x, ids, w)
    _check_moe(orc, G, U, Dn, sh, x, ids, w, out, h, TOL_FP32)


DECODE = [  # (fmt, S, K, E, D, F, gs, shared)
    (4, 1, 8, 16, 256, 128, 64, False),
    (4, 1, 8, 16, 256, 128, 64, True),
    (4, 2, 4, 6, 192, 96, 32, True),
    (4, 3, 2, 5, 128, 64, 16, False),
    (4, 4, 8, 12, 2048 + 64, 64, 64, True),
    (4, 4, 3, 9, 96, 2048 + 96, 32, False),
    (4, 1, 1, 1, 64, 32, 128, False),
    (2, 2, 3, 7, 128, 96, 0, True),
    (1, 1, 4, 6, 64, 48, 0, False),
    (1, 3, 2, 4, 160, 64, 0, True),
    (3, 2, 4, 6, 128, 64, 0, True),
    (3, 4, 2, 3, 96, 160, 0, False),
    (2, 3, 4, 6, 224, 64, 0, True),    # 14 down tiles: a ragged last row column
    (4, 2, 5, 7, 352, 96, 64, True),   # 22 down tiles
]


@pytest.mark.parametrize("kmode", [0, 1], ids=["mfma", "valu"])
@pytest.mark.parametrize("case", DECODE, ids=["fmt{}-S{}-K{}-E{}-D{}-F{}-gs{}-sh{}".format(*c) for c in DECODE])
def test_moe_decode_small(orc, case, kmode):
    need_gpu()
    fmt, S, K, E, D, F, gs, shared = case
    G, U, Dn, sh, x, ids, w = _moe_inputs(hash(case) % 997, fmt, S, K, E, D, F, gs, shared)
    with decode_kernels(kmode):
        out, h = _run_gpu(G, U, Dn, sh, x, ids, w, pack=(kmode == 0))
    _check_moe(orc, G, U, Dn, sh, x, ids, w, out, h, TOL_FP32)


@pytest.mark.parametrize("kmode", [0, 1], ids=["mfma", "valu"])
def test_moe_decode_duplicates_invalid_and_zero_weights(orc, kmode):
    need_gpu()
    G, U, Dn, sh, x, ids, w = _moe_inputs(31, 4, 3, 4, 8, 128, 64, 64, True)
    ids = ids.copy()
    w = w.copy()
    ids[0, 1] = ids[0, 0]      # duplicate expert in one row: two independent terms
    ids[1, 2] = 8              # out of range: left out
    ids[2, 0] = -5             # out of range: left out
    w[2, 3] = 0.0              # zero weight
    with decode_kernels(kmode):
        out, h = _run_gpu(G, U, Dn, sh, x, ids, w, pack=(kmode == 0))
    _check_moe(orc, G, U, Dn, sh, x, ids, w, out, h, TOL_FP32)


def test_moe_decode_single_row_shared_invalid_ids(orc):
    """S = 1, K = 7 plus the shared expert (8 pairs) on the matrix-core
    kernels, with an out-of-range id, a negative id, a duplicate and a zero
    weight."""
    need_gpu()
    G, U, Dn, sh, x, ids, w = _moe_inputs(33, 4, 1, 7, 8, 224, 96, 32, True)
    ids = ids.copy()
    w = w.copy()
    ids[0, 1] = 8
    ids[0, 2] = -1
    ids[0, 4] = ids[0, 3]
    w[0, 5] = 0.0
    out, h = _run_gpu(G, U, Dn, sh, x, ids, w)
    _check_moe(orc, G, U, Dn, sh, x, ids, w, out, h, TOL_FP32)


@pytest.mark.parametrize("S", [1, 2, 3, 4])
def test_moe_decode_zero_weight_outlier_in_h(orc, S):
    """One hidden unit j0 of every expert is driven to ~1e13 (its gate and up
    rows have all codes +7 and scales 1e3, on inputs whose first block is
    positive) while the down matrices' column j0 is zero in every row: the
    down kernel's first 128-input block of h then has a huge maximum and no
    weight on it.  Every stage stays within its bound plus the matrix-core
    decode kernels' 2^-29 * Ahat term (gate/up from x, down from the GPU's h)."""
    need_gpu()
    E, D, F, K, gs, j0 = 4, 512, 256, 2, 64, 100
    G, U, Dn, sh, x, ids, w = _moe_inputs(800 + S, 4, S, K, E, D, F, gs, True)
    for m in (G, U, sh[0], sh[1]):
        q = m.q if m.q.ndim == 3 else m.q[None]
        sc = m.s if m.s.ndim == 3 else m.s[None]
        q[:, j0, :] = 0xFF
        sc[:, j0, :] = 1e3
    for m in (Dn, sh[2]):
        q = m.q if m.q.ndim == 3 else m.q[None]
        for e in range(q.shape[0]):
            zero_column(q[e], 4, j0)
    x[:, :128] = 5.0
    out, h = _run_gpu(G, U, Dn, sh, x, ids, w)
    assert np.min(np.abs(h[:, j0])) > 1e12
    _check_moe(orc, G, U, Dn, sh, x, ids, w, out, h, TOL_FP32, rep=True)


def test_moe_decode_repeatable_bitwise(orc):
    need_gpu()
    G, U, Dn, sh, x, ids, w = _moe_inputs(5, 4, 4, 8, 16, 512, 256, 64, True)
    a, _ = _run_gpu(G, U, Dn, sh, x, ids, w, hidden=False)
    b, _ = _run_gpu(G, U, Dn, sh, x, ids, w, hidden=False)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_moe_decode_config2_full(orc):
    """Decode MoE block at its real shape: hidden 6144, 256 experts with gate/up
    2048x6144 and down 6144x2048, fmt 4 gs 64, 8 routed experts chosen
    uniformly, softmax weights.  The expert pool is drawn on the device with a
    seeded generator; the 8 routed experts are copied back for the oracle,
    which evaluates every one of the 6144 output rows."""
    need_gpu()
    E, D, F, gs, K = 256, 6144, 2048, 64, 8
    r = sd.rng(2)
    x = sd.gen_x(r, 1, D)
    ids, w = sd.gen_routing_uniform(r, 1, K, E)
    gq, gsc = sd.pool_on_device(100, 4, E, F, D, gs)
    uq, usc = sd.pool_on_device(101, 4, E, F, D, gs)
    dq, dsc = sd.pool_on_device(102, 4, E, D, F, gs)
    tg = coli.QTensor(4, gq, gsc, F, D, gs)
    tu = coli.QTensor(4, uq, usc, F, D, gs)
    td = coli.QTensor(4, dq, dsc, D, F, gs)
    for t in (tg, tu, td):
        assert t.pack()
    xd, idd, wd = to_dev(x), to_dev(ids), to_dev(w)
    ws_bytes = coli.coli_moe_workspace_bytes(E, 1, K, F, D, 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.full((1, D), float("nan"), device="cuda")
    h = torch.full((K, F), float("nan"), device="cuda")
    coli.check(coli.coli_moe_block(tg, tu, td, xd, 1, idd, wd, K, None, None, None, out, ws,
                                   ws_bytes))
    coli.check(coli.coli_moe_hidden(tg, tu, xd, 1, idd, K, None, None, h, ws, ws_bytes))
    torch.cuda.synchronize()
    # the routed experts, relabelled 0..7, on the host
    sel = torch.from_numpy(ids[0].astype(np.int64)).cuda()
    G = QMat(4, F, D, gs, gq[sel].cpu().numpy(), gsc[sel].cpu().numpy())
    U = QMat(4, F, D, gs, uq[sel].cpu().numpy(), usc[sel].cpu().numpy())
    Dn = QMat(4, D, F, gs, dq[sel].cpu().numpy(), dsc[sel].cpu().numpy())
    local = np.arange(K, dtype=np.int32)[None, :]
    _check_moe(orc, G, U, Dn, None, x, local, w, out.cpu().numpy(), h.cpu().numpy(), TOL_FP32)


ROUTE = [(1, 8, 256), (3, 2, 5), (7, 3, 4), (16, 4, 64), (5, 1, 1), (544, 8, 256),
         (100, 8, 4096), (2000, 2, 37), (4, 64, 300)]


@pytest.mark.parametrize("S,K,E", ROUTE)
def test_route_bit_exact(orc, S, K, E):
    need_gpu()
    r = sd.rng(S * 7 + K + E)
    if S == 544:
        ids, _ = sd.gen_routing_zipf(r, S, K, E, 1.1)
    else:
        ids = r.integers(0, E, size=(S, K)).astype(np.int32)
    _route_compare(orc, ids, E)


def test_route_invalid_ids(orc):
    need_gpu()
    ids = sd.rng(1).integers(-3, 12, size=(50, 4)).astype(np.int32)
    _route_compare(orc, ids, 9)


def _route_compare(orc, ids, E):
    S, K = ids.shape
    counts = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((max(S * K, 1),), -7, dtype=torch.int32, device="cuda")
    bad = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    coli.check(coli.coli_moe_route(to_dev(ids), S, K, E, counts, offsets, perm, bad))
    torch.cuda.synchronize()
    c_ref, o_ref, p_ref, b_ref = orc.moe_route(ids, E)
    assert np.array_equal(counts.cpu().numpy(), c_ref)
    assert np.array_equal(offsets.cpu().numpy(), o_ref)
    assert np.array_equal(perm.cpu().numpy()[:S * K], p_ref)
    assert int(bad.item()) == b_ref


TWO_PHASE = [  # (fmt, S, K, E, D, F, gs, shared, late pattern)
    (4, 1, 8, 16, 256, 128, 64, True, "half"),
    (4, 1, 8, 16, 256, 128, 64, False, "all"),
    (4, 3, 4, 9, 192, 96, 32, True, "half"),
    (2, 2, 3, 7, 128, 96, 0, True, "none"),
    (4, 40, 4, 12, 256, 128, 128, True, "half"),   # S > 4: the prefill kernels
    (4, 24, 2, 6, 256, 128, 64, False, "all"),
]


def _late(pattern, S, K, seed):
    if pattern == "none":
        return np.zeros((S, K), np.int32)
    if pattern == "all":
        return np.ones((S, K), np.int32)
    return (sd.rng(seed).random((S, K)) < 0.5).astype(np.int32)


def _two_phase(G, U, Dn, sh, x, ids, w, late, pack=True):
    S, K = ids.shape
    E, F, D = G.n, G.O, G.I
    tg, tu, td = qtensor(G, pack), qtensor(U, pack), qtensor(Dn, pack)
    ts = [qtensor(m, pack) for m in sh] if sh is not None else [None, None, None]
    xd, idd, wd = to_dev(x), to_dev(ids.astype(np.int32)), to_dev(w.astype(np.float32))
    ld = to_dev(late.astype(np.int32))
    wsb = coli.coli_moe_block_two_phase_workspace_bytes(E, S, K, F, D, sh is not None)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.full((S, D), float("nan"), device="cuda")
    coli.check(coli.coli_moe_block_begin(tg, tu, td, xd, S, idd, wd, K, ld, ts[0], ts[1], ts[2], out,
                                         ws, wsb), "coli_moe_block_begin")
    coli.check(coli.coli_moe_block_end(tg, tu, td, xd, S, wd, K, sh is not None, out, ws, wsb),
               "coli_moe_block_end")
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("case", TWO_PHASE,
                         ids=["fmt{}-S{}-K{}-E{}-D{}-F{}-gs{}-sh{}-{}".format(*c) for c in TWO_PHASE])
def test_moe_two_phase_matches_oracle(orc, case):
    """Resident slots (and the shared expert) in begin, late slots in end: the
    sum equals the whole block within its end-to-end bound; with no late slot
    it equals coli_moe_block itself."""
    need_gpu()
    fmt, S, K, E, D, F, gs, shared, pattern = case
    G, U, Dn, sh, x, ids, w = _moe_inputs(700 + S + K + E, fmt, S, K, E, D, F, gs, shared)
    late = _late(pattern, S, K, seed=S * K)
    out = _two_phase(G, U, Dn, sh, x, ids, w, late)
    tau = TOL_FP32 if S <= coli.coli_gemv_max_rows() else TOL_BF16
    _check_moe(orc, G, U, Dn, sh, x, ids, w, out, None, tau)
    if pattern == "none":
        whole, _ = _run_gpu(G, U, Dn, sh, x, ids, w, hidden=False)
        assert np.array_equal(out, whole)


def test_moe_two_phase_repeatable_and_declines(orc):
    need_gpu()
    G, U, Dn, sh, x, ids, w = _moe_inputs(77, 4, 1, 8, 16, 256, 128, 64, True)
    late = _late("half", 1, 8, seed=3)
    a = _two_phase(G, U, Dn, sh, x, ids, w, late)
    b = _two_phase(G, U, Dn, sh, x, ids, w, late)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    tg, tu, td = qtensor(G, True), qtensor(U, True), qtensor(Dn, True)
    xd, idd, wd = to_dev(x), to_dev(ids), to_dev(w)
    wsb = coli.coli_moe_block_two_phase_workspace_bytes(16, 1, 8, 128, 256, False)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.full((1, 256), 5.0, device="cuda")
    assert coli.coli_moe_block_begin(tg, tu, td, xd, 1, idd, wd, 8, None, None, None, None, out,
                                     ws, wsb) == coli.COLI_DECLINED
    assert "late" in coli.coli_last_reason()
    assert coli.coli_moe_block_begin(tg, tu, td, xd, 1, idd, wd, 8, idd, None, None, None, out,
                                     ws, wsb - 256) == coli.COLI_DECLINED
    assert coli.coli_moe_block_end(tg, tu, td, xd, 1, wd, 8, False, out, ws, wsb - 256) == \
        coli.COLI_DECLINED
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)


def test_moe_two_phase_overlapped_upload(orc):
    """The two-phase block as the pages use it: the late experts' weights
    (codes, scales and the packed copy the decode kernels read) are not on the
    device when begin is enqueued; they are copied from pinned host memory on
    a second stream while begin runs, and end waits for the copies through an
    event.  The result is bit-identical to the same two submissions run after
    the copies have finished, and within the block's bound of the oracle."""
    need_gpu()
    S, K, E, D, F, gs = 1, 8, 16, 1024, 512, 64
    G, U, Dn, sh, x, ids, w = _moe_inputs(931, 4, S, K, E, D, F, gs, True)
    late = np.zeros((S, K), np.int32)
    late[0, 1::2] = 1
    late_e = sorted(set(int(e) for e in ids[0, 1::2]))
    tg, tu, td = qtensor(G, True), qtensor(U, True), qtensor(Dn, True)
    ts = [qtensor(m, True) for m in sh]
    xd, idd, wd = to_dev(x), to_dev(ids.astype(np.int32)), to_dev(w.astype(np.float32))
    ld = to_dev(late)
    wsb = coli.coli_moe_block_two_phase_workspace_bytes(E, S, K, F, D, True)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")

    # the late experts' device slices: original codes, scales, packed copy
    def slices(T):
        d = T.desc
        out = []
        for e in late_e:
            out.append(T.q[e])
            out.append(T.s[e])
            out.append(T.packed[e * d.pk_stride:(e + 1) * d.pk_stride])
        return out
    dev_sl = [t for T in (tg, tu, td) for t in slices(T)]
    host = [torch.empty(t.shape, dtype=t.dtype, pin_memory=True) for t in dev_sl]
    for h_, d_ in zip(host, dev_sl):
        h_.copy_(d_)
    torch.cuda.synchronize()

    def run(overlap):
        for d_ in dev_sl:   # not loaded yet
            d_.zero_()
        out = torch.full((S, D), float("nan"), device="cuda")
        main = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        side.wait_stream(main)
        if not overlap:
            for h_, d_ in zip(host, dev_sl):
                d_.copy_(h_)
        coli.check(coli.coli_moe_block_begin(tg, tu, td, xd, S, idd, wd, K, ld, ts[0], ts[1],
                                             ts[2], out, ws, wsb, main), "begin")
        if overlap:
            with torch.cuda.stream(side):
                for h_, d_ in zip(host, dev_sl):
                    d_.copy_(h_, non_blocking=True)
                ev = torch.cuda.Event()
                ev.record(side)
            main.wait_event(ev)
        coli.check(coli.coli_moe_block_end(tg, tu, td, xd, S, wd, K, True, out, ws, wsb, main),
                   "end")
        torch.cuda.synchronize()
        return out.cpu().numpy()
    serial = run(False)
    overlapped = run(True)
    assert np.array_equal(serial.view(np.uint32), overlapped.view(np.uint32))
    _check_moe(orc, G, U, Dn, sh, x, ids, w, overlapped, None, TOL_FP32)
