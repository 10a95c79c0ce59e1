"""GPU parity of coli_qmatmul_ws, the prefill GEMM whose input rows are
prepared once in a workspace (bf16, in the matrix cores' order) and whose
workgroups split each 128-input block over their four wavefronts, against
the oracle with the bf16 tolerance 4e-3 * sum |w||x| (colibri-strix commit
log, prefill GEMM routing commit: prefill-sized row batches take a GEMM
path; colibri PR #298: w = scale * (q - 8), the group scale applied per
group)."""
import numpy as np
import pytest
import torch

import bit_gemv_coli_amd as coli
import synthdata as sd
from gpu_util import (DEV, TOL_BF16, assert_within, make_case, need_gpu, qtensor, rep_allowance,
                      to_dev)

pytestmark = pytest.mark.gpu


def gpu_qmatmul_ws(T, x, n=1, ws_extra=0, ws_none=False):
    xd = to_dev(x.astype(np.float32))
    S = x.shape[0]
    y = torch.full((n, S, T.desc.O), float("nan"), device=DEV)
    wsb = coli.coli_qmatmul_workspace_bytes(T, S)
    ws = None if ws_none else torch.full((max(wsb + ws_extra, 256),), 0xFF, dtype=torch.uint8,
                                          device=DEV)
    coli.check(coli.coli_qmatmul_ws(T, xd, y, S, ws, 0 if ws is None else ws.numel()),
               "coli_qmatmul_ws")
    torch.cuda.synchronize()
    return y.cpu().numpy()


# (fmt, O, I, gs, S, n): ragged rows (tiles of 144), outputs (tiles of 96),
# inputs (128-input blocks, block counts not a multiple of 4), stacks
CASES = [
    (4, 96, 512, 128, 5, 1), (4, 100, 384, 128, 17, 1), (4, 257, 1056, 64, 144, 1),
    (4, 200, 160, 32, 145, 2), (4, 192, 2048, 256, 300, 1), (4, 130, 640, 32, 33, 1),
    (4, 64, 6144, 128, 290, 1), (4, 16, 128, 128, 9, 1), (4, 1000, 896, 64, 61, 1),
    (2, 100, 256, 0, 7, 1), (2, 300, 1152, 0, 150, 2),
]


@pytest.mark.parametrize("case", CASES, ids=["fmt{}-O{}-I{}-gs{}-S{}-n{}".format(*c) for c in CASES])
def test_qmatmul_ws(orc, case):
    need_gpu()
    fmt, O, I, gs, S, n = case
    W, x = make_case(fmt, O, I, gs, S, seed=700 + hash(case) % 1000, n=n if n > 1 else None)
    T = qtensor(W, pack=True)
    assert coli.coli_qmatmul_workspace_bytes(T, S) > 0
    y = gpu_qmatmul_ws(T, x, n)
    for e in range(n):
        y_ref, A = orc.qmatmul(W.expert(e), x)
        assert_within(y[e], y_ref, A, TOL_BF16, f"{case} matrix {e}")
    # repeatable: a second call (workspace filled with other bytes) gives the same bits
    y2 = gpu_qmatmul_ws(T, x, n, ws_extra=4096)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("gs", [64, 128])
def test_qmatmul_ws_dense_544_full(orc, gs):
    """S = 544 x 6144 x 6144 fmt 4, the launch the bench times: every output
    of 24 sampled input rows against the oracle, all outputs finite."""
    need_gpu()
    W, x = make_case(4, 6144, 6144, gs, 544, seed=544 + gs)
    T = qtensor(W, pack=True)
    y = gpu_qmatmul_ws(T, x)[0]
    rows = np.sort(sd.rng(2).choice(544, 24, replace=False))
    y_ref, A = orc.qmatmul(W, x[rows])
    assert_within(y[rows], y_ref, A, TOL_BF16, f"dense 544 g{gs}")
    assert np.all(np.isfinite(y))


def test_qmatmul_ws_falls_back(orc):
    """No workspace, an unpacked tensor or decode rows: coli_qmatmul's own
    kernels, within their bounds."""
    need_gpu()
    W, x = make_case(4, 96, 256, 64, 20, seed=5)
    y_ref, A = orc.qmatmul(W, x)
    assert_within(gpu_qmatmul_ws(qtensor(W, pack=True), x, ws_none=True)[0], y_ref, A, TOL_BF16,
                  "no workspace")
    assert_within(gpu_qmatmul_ws(qtensor(W), x)[0], y_ref, A, TOL_BF16, "unpacked")
    W4, x4 = make_case(4, 96, 256, 64, 3, seed=6)
    T4 = qtensor(W4, pack=True)
    assert coli.coli_qmatmul_workspace_bytes(T4, 3) == 0
    y4_ref, A4 = orc.qmatmul(W4, x4)
    assert_within(gpu_qmatmul_ws(T4, x4)[0], y4_ref, A4, 1e-5, "decode rows",
                  extra=rep_allowance(orc, W4, x4))


def test_qmatmul_ws_zero_rows_and_outliers(orc):
    """Rows of zeros give exact zeros; inputs up to 1e6 times the rest at
    columns whose weights are zero in every row contribute nothing; negative
    scales."""
    need_gpu()
    from gpu_util import zero_column
    W, x = make_case(4, 192, 512, 128, 150, seed=9)
    cols = (3, 200, 333, 511)
    for c in cols:
        zero_column(W.q, 4, c)
    W.s[5] = -np.abs(W.s[5])
    x[3] = 0.0
    for t in range(4, 150):
        x[t, cols[t % 4]] = 1e6 if t % 2 else -1e6
    T = qtensor(W, pack=True)
    y = gpu_qmatmul_ws(T, x)[0]
    y_ref, A = orc.qmatmul(W, x)
    assert_within(y, y_ref, A, TOL_BF16, "zeros / outliers")
    assert np.all(y[3] == 0.0)


def test_qmatmul_ws_dominant_product(orc):
    """One product carrying nearly all of sum |w||x| (a large input at a
    nonzero weight): weight and input are each rounded once to bf16, so the
    worst case is (2^-7 + 2^-16) * sum |w||x| (bf16 keeps 8 significant bits);
    that bound holds here."""
    need_gpu()
    W, x = make_case(4, 192, 512, 128, 150, seed=9)
    x[100, 17] = 3.0e4
    T = qtensor(W, pack=True)
    y = gpu_qmatmul_ws(T, x)[0]
    y_ref, A = orc.qmatmul(W, x)
    assert_within(y, y_ref, A, 2.0 ** -7 + 2.0 ** -16 + 1e-5, "dominant product")
