"""GPU parity of coli_qmatmul_group (several independent matrices, each with
its own input and output, in one submission) through the C ABI: every member
against the oracle within the fp32 GEMV bound, and bit-identical to the same
member run alone through coli_qmatmul; mixed members and S > 4 (one launch
per member inside the call) and the declines."""
import numpy as np
import pytest
import torch

import bit_gemv_coli_amd as coli
from gpu_util import TOL_BF16, TOL_FP32, assert_within, make_case, need_gpu, qtensor, to_dev

pytestmark = pytest.mark.gpu

# members: (fmt, O, I, gs); the first group is the attention projections of a
# decode layer at a reduced size plus ragged shapes (O not a multiple of the
# 32-row workgroup tile, I not a multiple of 128)
GROUPS = [
    [(4, 1536, 6144, 64), (4, 2048, 1536, 64), (4, 576, 6144, 64), (4, 6144, 2048, 64)],
    [(4, 37, 4160, 64), (4, 5, 96, 64), (4, 300, 640, 64), (4, 150, 8320, 64), (4, 33, 32, 64),
     (4, 129, 2080, 64), (4, 70, 1024, 64), (4, 1, 256, 64)],
    [(4, 70, 1024, 128), (4, 300, 2560, 256), (4, 17, 6144, 128)],
    [(4, 40, 96, 32), (4, 9, 4096, 32)],
    [(2, 41, 2080, 0), (2, 9, 64, 0), (2, 500, 1536, 0)],
    [(1, 37, 1056, 0), (1, 300, 640, 0), (1, 16, 8320, 0)],
    [(3, 37, 1056, 0), (3, 300, 640, 0), (3, 16, 8320, 0)],
]


def _members(group, S, seed):
    Ws, xs = [], []
    for j, (fmt, O, I, gs) in enumerate(group):
        W, x = make_case(fmt, O, I, gs, S, seed=seed + 17 * j)
        Ws.append(W)
        xs.append(x)
    return Ws, xs


def _run_group(Ts, xs, S, stacks=None):
    xd = [to_dev(x.astype(np.float32)) for x in xs]
    ys = [torch.full(((stacks or [1] * len(Ts))[j], S, T.desc.O), float("nan"), device="cuda")
          for j, T in enumerate(Ts)]
    coli.check(coli.coli_qmatmul_group(Ts, xd, ys, S), "coli_qmatmul_group")
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys], xd


@pytest.mark.parametrize("S", [1, 2, 4])
@pytest.mark.parametrize("gi", range(len(GROUPS)))
def test_group_matches_oracle_and_single_calls(orc, gi, S):
    need_gpu()
    Ws, xs = _members(GROUPS[gi], S, seed=100 * gi + S)
    Ts = [qtensor(W, pack=True) for W in Ws]
    ys, xd = _run_group(Ts, xs, S)
    for j, (W, T) in enumerate(zip(Ws, Ts)):
        y_ref, A = orc.qmatmul(W, xs[j])
        assert_within(ys[j][0], y_ref, A, TOL_FP32, f"group {gi} member {j}")
        alone = torch.full((1, S, W.O), float("nan"), device="cuda")
        coli.check(coli.coli_qmatmul(T, xd[j], alone, S), "coli_qmatmul")
        torch.cuda.synchronize()
        assert np.array_equal(alone.cpu().numpy().view(np.uint32), ys[j].view(np.uint32)), (gi, j)


def test_group_mixed_members_fall_back_per_member(orc):
    """A packed fmt-4 member, an unpacked one, a fmt-1 member and a stack of
    two: not one launch, still one call with every member right."""
    need_gpu()
    S = 3
    spec = [(4, 40, 512, 64, True), (4, 33, 200, 64, False), (1, 20, 130, 0, False),
            (2, 24, 256, 0, True)]
    Ws, xs, Ts = [], [], []
    for j, (fmt, O, I, gs, pk) in enumerate(spec):
        W, x = make_case(fmt, O, I, gs, S, seed=900 + j, n=2 if j == 3 else None)
        Ws.append(W)
        xs.append(x)
        Ts.append(qtensor(W, pack=pk))
    ys, _ = _run_group(Ts, xs, S, stacks=[1, 1, 1, 2])
    for j, W in enumerate(Ws):
        for e in range(2 if j == 3 else 1):
            y_ref, A = orc.qmatmul(W.expert(e) if j == 3 else W, xs[j])
            assert_within(ys[j][e], y_ref, A, TOL_FP32, f"member {j} matrix {e}")


def test_group_prefill_rows(orc):
    """S > 4: every member on the bf16 matrix-core GEMM within its bound."""
    need_gpu()
    S = 20
    Ws, xs = _members([(4, 96, 512, 64), (4, 130, 1024, 128)], S, seed=77)
    Ts = [qtensor(W, pack=True) for W in Ws]
    ys, _ = _run_group(Ts, xs, S)
    for j, W in enumerate(Ws):
        y_ref, A = orc.qmatmul(W, xs[j])
        assert_within(ys[j][0], y_ref, A, TOL_BF16, f"member {j}")


def test_group_declines_leave_outputs_untouched():
    need_gpu()
    W, x = make_case(4, 32, 128, 64, 1, seed=5)
    T = qtensor(W, pack=True)
    xd = to_dev(x.astype(np.float32))
    y = torch.full((1, 1, 32), 7.0, device="cuda")
    assert coli.coli_qmatmul_group([], [], [], 1) == coli.COLI_DECLINED
    assert coli.coli_qmatmul_group([T] * 9, [xd] * 9, [y] * 9, 1) == coli.COLI_DECLINED
    assert coli.coli_qmatmul_group([T, T], [xd, None], [y, y], 1) == coli.COLI_DECLINED
    assert coli.coli_qmatmul_group([T], [xd], [y], 0) == coli.COLI_DECLINED
    bad = coli.coli_qtensor()  # never uploaded
    assert coli.coli_qmatmul_group([T, bad], [xd, xd], [y, y], 1) == coli.COLI_DECLINED
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
