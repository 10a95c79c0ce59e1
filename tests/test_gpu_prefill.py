"""GPU parity of the prefill path (S > 4 input rows): the bf16 matrix-core
GEMM for coli_qmatmul and the ragged MoE block (routing table, gathered
inputs, dual gate/up + SiLU, down, combine), against the oracle with the
bf16 tolerance 4e-3 * sum |w||x| (colibri-strix commit log, prefill GEMM routing commit: prefill-sized row batches take a GEMM
path)."""
import numpy as np
import pytest
import torch

import bit_gemv_coli_amd as coli
import synthdata as sd
from gpu_util import TOL_BF16, assert_within, gpu_qmatmul, make_case, need_gpu, qtensor, to_dev
from oracle import QMat
from test_gpu_moe import _check_moe, _moe_inputs, _run_gpu

pytestmark = pytest.mark.gpu

# (fmt, O, I, gs, S, n)
GEMM = [
    (4, 128, 256, 64, 5, 1), (4, 130, 96, 32, 17, 1), (4, 64, 6144, 128, 33, 1),
    (4, 200, 320, 64, 64, 2), (4, 48, 512, 256, 100, 1), (4, 257, 2048, 64, 65, 1),
    (4, 32, 160, 160, 9, 1),
    (2, 100, 256, 0, 7, 1), (2, 64, 96, 0, 129, 1),
    (1, 90, 128, 0, 12, 1), (1, 33, 96, 0, 70, 2),
    (3, 77, 256, 0, 6, 1), (3, 128, 160, 0, 40, 1),
    # > 64 rows: packed fmt-4 tensors with gs <= 128 take the weight-streaming
    # kernel (128 x 128 tiles; ragged rows, columns and a partial last block)
    (4, 300, 384, 128, 200, 1), (4, 130, 256, 32, 130, 2), (4, 96, 160, 32, 77, 1),
    (4, 272, 1024, 64, 129, 1),
]


@pytest.mark.parametrize("pack", [False, True], ids=["plain", "packed"])
@pytest.mark.parametrize("case", GEMM, ids=["fmt{}-O{}-I{}-gs{}-S{}-n{}".format(*c) for c in GEMM])
def test_qmatmul_prefill(orc, case, pack):
    need_gpu()
    fmt, O, I, gs, S, n = case
    W, x = make_case(fmt, O, I, gs, S, seed=200 + hash(case) % 1000, n=n if n > 1 else None)
    T = qtensor(W, pack=pack and coli.coli_packed_bytes(fmt, n, O, I, gs) > 0)
    y = gpu_qmatmul(T, x, n)
    for e in range(n):
        y_ref, A = orc.qmatmul(W.expert(e), x)
        assert_within(y[e], y_ref, A, TOL_BF16, f"{case} expert {e}")


def test_qmatmul_prefill_fallback_layouts(orc):
    """Layouts the matrix cores do not take (odd I, gs % 32 != 0) run the exact
    fp32 path and still meet the bound."""
    need_gpu()
    for fmt, O, I, gs, S in [(4, 20, 130, 64, 9), (4, 16, 96, 16, 6), (2, 9, 33, 0, 12)]:
        W, x = make_case(fmt, O, I, gs, S, seed=O + I)
        y = gpu_qmatmul(qtensor(W), x)[0]
        y_ref, A = orc.qmatmul(W, x)
        assert_within(y, y_ref, A, TOL_BF16, f"fallback {fmt} {I} {gs}")


@pytest.mark.parametrize("pack", [False, True], ids=["plain", "packed"])
@pytest.mark.parametrize("gs", [64, 128])
def test_qmatmul_prefill_dense_544_full(orc, gs, pack):
    """S = 544 x 6144 x 6144 fmt 4: every output of 24 sampled input rows."""
    need_gpu()
    W, x = make_case(4, 6144, 6144, gs, 544, seed=544 + gs)
    y = gpu_qmatmul(qtensor(W, pack=pack), x)[0]
    rows = np.sort(sd.rng(1).choice(544, 24, replace=False))
    y_ref, A = orc.qmatmul(W, x[rows])
    assert_within(y[rows], y_ref, A, TOL_BF16, f"dense 544 g{gs}")
    assert np.all(np.isfinite(y))


PREFILL = [  # (fmt, S, K, E, D, F, gs, shared)
    (4, 5, 2, 6, 128, 64, 32, False),
    (4, 9, 4, 7, 256, 128, 64, True),
    (4, 40, 8, 16, 192, 160, 32, True),
    (4, 33, 3, 3, 128, 96, 128, False),
    (2, 12, 2, 5, 128, 64, 0, True),
    (1, 7, 3, 4, 96, 64, 0, False),
    (3, 20, 2, 6, 128, 96, 0, True),
    (4, 24, 4, 6, 768, 384, 384, True),   # groups of 3 blocks
    (4, 70, 2, 5, 512, 256, 256, False),  # groups of 2 blocks, experts with several tiles
    (2, 45, 3, 4, 160, 96, 0, False),     # K not a multiple of the 128-input block
]


@pytest.mark.parametrize("pack", [True, False], ids=["packed", "unpacked"])
@pytest.mark.parametrize("case", PREFILL, ids=["fmt{}-S{}-K{}-E{}-D{}-F{}-gs{}-sh{}".format(*c) for c in PREFILL])
def test_moe_prefill_small(orc, case, pack):
    """Packed copies take the weight-streaming kernel (32-row tiles), plain
    int4 tensors the producer/consumer kernel (64-row tiles), the other
    formats the generic matrix-core GEMM."""
    need_gpu()
    fmt, S, K, E, D, F, gs, shared = case
    G, U, Dn, sh, x, ids, w = _moe_inputs(300 + hash(case) % 997, fmt, S, K, E, D, F, gs, shared)
    out, h = _run_gpu(G, U, Dn, sh, x, ids, w, pack=pack)
    _check_moe(orc, G, U, Dn, sh, x, ids, w, out, h, TOL_BF16)


def _routing_with_counts(counts, S, K):
    """ids [S][K] in which expert e is routed exactly counts[e] times, never
    twice to one token (every count <= S): the sorted labels fill slot k of
    tokens 0..S-1 in turn."""
    labels = np.repeat(np.arange(len(counts)), counts)
    assert labels.size == S * K and max(counts) <= S
    return labels.reshape(K, S).T.astype(np.int32).copy()


@pytest.mark.parametrize("counts,shared", [
    ([1, 15, 16, 17, 0, 31], False),
    ([32, 33, 15, 0, 0, 0], True),
], ids=["1-15-16-17-0-31", "32-33-15-shared"])
def test_moe_prefill_tile_boundaries(orc, counts, shared):
    """Experts with 1..16 routed rows take one 16-row tile, larger ones 32-row
    tiles (packed experts): counts on both sides of both boundaries."""
    need_gpu()
    S, K = 40, 2
    G, U, Dn, sh, x, _, w = _moe_inputs(77 + len(counts), 4, S, K, len(counts), 256, 128, 64,
                                        shared)
    ids = _routing_with_counts(counts, S, K)
    assert np.array_equal(np.bincount(ids.ravel(), minlength=len(counts)), counts)
    out, h = _run_gpu(G, U, Dn, sh, x, ids, w)
    _check_moe(orc, G, U, Dn, sh, x, ids, w, out, h, TOL_BF16)


def test_moe_prefill_ragged_zipf_invalid(orc):
    """Zipf-skewed routing (some experts with many rows, many with one or
    none), out-of-range ids and duplicates."""
    need_gpu()
    G, U, Dn, sh, x, ids, w = _moe_inputs(41, 4, 70, 4, 12, 256, 128, 64, True, routing="zipf")
    ids = ids.copy()
    ids[3, 1] = 12
    ids[5, 0] = -1
    ids[7, 2] = ids[7, 1]
    out, h = _run_gpu(G, U, Dn, sh, x, ids, w)
    _check_moe(orc, G, U, Dn, sh, x, ids, w, out, h, TOL_BF16)


def test_moe_prefill_repeatable_bitwise(orc):
    need_gpu()
    G, U, Dn, sh, x, ids, w = _moe_inputs(42, 4, 50, 8, 16, 256, 128, 64, True, routing="zipf")
    a, _ = _run_gpu(G, U, Dn, sh, x, ids, w, hidden=False)
    b, _ = _run_gpu(G, U, Dn, sh, x, ids, w, hidden=False)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("pack", [True, False], ids=["packed", "unpacked"])
def test_moe_prefill_config4_full(orc, pack):
    """Prefill MoE at its real shape: S = 544 tokens, 256 experts, top-8 with
    Zipf(1.1) popularity, gate/up 2048x6144 and down 6144x2048 fmt 4 gs 128.
    The pool is drawn on the device; the oracle evaluates 6 sampled tokens
    (each token's output depends only on its own input and routing) at 256
    sampled output rows, with the experts those tokens use copied back."""
    need_gpu()
    E, D, F, gs, K, S = 256, 6144, 2048, 128, 8, 544
    r = sd.rng(4)
    x = sd.gen_x(r, S, D)
    ids, w = sd.gen_routing_zipf(r, S, K, E, 1.1)
    gq, gsc = sd.pool_on_device(200, 4, E, F, D, gs)
    uq, usc = sd.pool_on_device(201, 4, E, F, D, gs)
    dq, dsc = sd.pool_on_device(202, 4, E, D, F, gs)
    tg = coli.QTensor(4, gq, gsc, F, D, gs)
    tu = coli.QTensor(4, uq, usc, F, D, gs)
    td = coli.QTensor(4, dq, dsc, D, F, gs)
    if pack:
        for t in (tg, tu, td):
            t.pack()
    xd, idd, wd = to_dev(x), to_dev(ids), to_dev(w)
    ws_bytes = coli.coli_moe_workspace_bytes(E, S, K, F, D, 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.full((S, D), float("nan"), device="cuda")
    coli.check(coli.coli_moe_block(tg, tu, td, xd, S, idd, wd, K, None, None, None, out, ws,
                                   ws_bytes))
    h = torch.full((S * K, F), float("nan"), device="cuda")
    coli.check(coli.coli_moe_hidden(tg, tu, xd, S, idd, K, None, None, h, ws, ws_bytes))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    h = h.cpu().numpy()
    assert np.all(np.isfinite(out))
    toks = np.sort(sd.rng(5).choice(S, 6, replace=False))
    used = np.unique(ids[toks])
    remap = {int(e): i for i, e in enumerate(used)}
    sel = torch.from_numpy(used.astype(np.int64)).cuda()
    G = QMat(4, F, D, gs, gq[sel].cpu().numpy(), gsc[sel].cpu().numpy())
    U = QMat(4, F, D, gs, uq[sel].cpu().numpy(), usc[sel].cpu().numpy())
    Dn = QMat(4, D, F, gs, dq[sel].cpu().numpy(), dsc[sel].cpu().numpy())
    local = np.vectorize(remap.get)(ids[toks]).astype(np.int32)
    rows = np.sort(sd.rng(6).choice(D, 256, replace=False)).astype(np.int32)
    hsel = h.reshape(S, K, F)[toks].reshape(-1, F)
    _check_moe(orc, G, U, Dn, None, x[toks], local, w[toks], out[toks], hsel, TOL_BF16, rows=rows)


ZW = [(4, 128, True), (4, 256, True), (4, 64, True), (4, 32, True), (4, 128, False), (2, 0, True),
      (2, 0, False)]


@pytest.mark.parametrize("fmt,gs,pack", ZW, ids=[f"fmt{f}-gs{g}-{'packed' if p else 'plain'}"
                                                 for f, g, p in ZW])
def test_qmatmul_prefill_zero_weights_and_outliers(orc, fmt, gs, pack):
    """Rows whose codes are all the zero code give exact zeros, and huge
    inputs at columns whose weights are zero in every row (up to 1e6 times
    the rest) stay within 4e-3 * sum |w||x|: the bound has no term for the
    inputs' spread, so a weight that is zero must contribute exactly nothing."""
    need_gpu()
    from gpu_util import zero_column
    O, I, S = 96, 1024, 130
    r = sd.rng(900 + fmt + gs + pack)
    q, s = sd.gen_matrix(r, fmt, O, I, gs)
    q[5] = 0x88          # zero rows
    q[17] = 0x88
    cols = (3, 200, 640, 1023)
    for c in cols:
        zero_column(q, fmt, c)
    W = QMat(fmt, O, I, gs if fmt == 4 else 0, q, s)
    T = qtensor(W, pack=pack)
    for mag in (1e3, 1e6):
        x = sd.gen_x(r, S, I)
        for t in range(S):
            x[t, cols[t % 4]] = mag if t % 2 else -mag
        y = gpu_qmatmul(T, x)[0]
        y_ref, A = orc.qmatmul(W, x)
        assert np.all(y[:, 5] == 0.0) and np.all(y[:, 17] == 0.0), "zero rows"
        assert_within(y, y_ref, A, TOL_BF16, f"fmt {fmt} gs {gs} outliers {mag:g}")


@pytest.mark.parametrize("gs", [64, 128, 256])
def test_moe_prefill_zero_weight_outliers(orc, gs):
    """S = 40 rows, Zipf routing (experts with 1-16 rows and with more), packed
    experts: inputs up to 1e5 times the rest at hidden columns whose gate and
    up weights are zero in every expert -- the weight-streaming kernels' group
    sums (codes as 2 + q/8 with a -3 correction row for gs >= 128) must make
    those columns contribute nothing, within the staged bf16 bound."""
    need_gpu()
    from gpu_util import zero_column
    E, D, F, K, S = 6, 512, 256, 4, 40
    G, U, Dn, sh, x, ids, w = _moe_inputs(950 + gs, 4, S, K, E, D, F, gs, True, routing="zipf")
    cols = (7, 130, 300, 511)
    for m in (G, U, sh[0], sh[1]):
        q = m.q if m.q.ndim == 3 else m.q[None]
        for e in range(q.shape[0]):
            for c in cols:
                zero_column(q[e], 4, c)
    for t in range(S):
        x[t, cols[t % 4]] = 1e5 if t % 2 else -1e5
    out, h = _run_gpu(G, U, Dn, sh, x, ids, w)
    _check_moe(orc, G, U, Dn, sh, x, ids, w, out, h, TOL_BF16)
