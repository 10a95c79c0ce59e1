"""GPU parity of coli_dequantize (bit-exact) and coli_qmatmul against the
oracle, through the C ABI.

The shape matrix follows the grouped-int4 test commit of colibri PR #298
(I a multiple of gs, partial last group, odd I, gs > I, gs = 16/64/128,
S > 1, nibble extremes) and the Metal commits' tails (non-multiple-of-8
rows/columns, I <= 64), plus the full sizes of the decode workloads."""
import numpy as np
import pytest
import torch

import bit_gemv_coli_amd as coli
import synthdata as sd
from gpu_util import (TOL_BF16, TOL_FP32, assert_within, decode_kernels, gpu_qmatmul, make_case,
                      need_gpu, qtensor, rep_allowance, to_dev, zero_column)
from oracle import QMat

pytestmark = pytest.mark.gpu

# (fmt, O, I, gs, S, n)
SMALL = [
    (4, 8, 128, 64, 1, 1), (4, 5, 130, 64, 1, 1), (4, 3, 129, 64, 2, 1), (4, 4, 37, 64, 1, 1),
    (4, 6, 96, 16, 3, 1), (4, 4, 256, 128, 1, 1), (4, 2, 1, 16, 1, 1), (4, 7, 200, 32, 4, 1),
    (4, 9, 96, 48, 2, 1), (4, 3, 96, 24, 1, 1), (4, 33, 4096 + 64, 64, 4, 1),
    (4, 70, 2048, 64, 1, 3), (4, 17, 6144, 128, 3, 2), (4, 5, 32, 32, 1, 1), (4, 5, 32, 64, 2, 1),
    (2, 5, 130, 0, 2, 1), (2, 3, 33, 0, 1, 1), (2, 41, 2048 + 32, 0, 4, 1), (2, 9, 64, 0, 1, 2),
    (1, 4, 70, 0, 3, 1), (1, 2, 5, 0, 1, 1), (1, 33, 1040, 0, 2, 1), (1, 8, 4096, 0, 4, 2),
    (3, 5, 130, 0, 2, 1), (3, 3, 7, 0, 1, 1), (3, 2, 66, 0, 1, 1), (3, 19, 2080, 0, 4, 1),
    (3, 12, 64, 0, 3, 2),
    # more inputs than one LDS segment holds at S = 4 (6656): the matrix-core
    # kernel restages the inputs between segments
    (4, 150, 8320, 64, 4, 1), (2, 40, 13312 + 32, 0, 4, 1),
]


def _id(c):
    return "fmt{}-O{}-I{}-gs{}-S{}-n{}".format(*c)


@pytest.mark.parametrize("case", SMALL, ids=[_id(c) for c in SMALL])
def test_dequant_bit_exact(orc, case):
    need_gpu()
    fmt, O, I, gs, S, n = case
    W, _ = make_case(fmt, O, I, gs, S, seed=hash(case) % 1000, n=n if n > 1 else None)
    T = qtensor(W)
    w = torch.full((n, O, I), float("nan"), device="cuda")
    coli.check(coli.coli_dequantize(T, w), "coli_dequantize")
    got = w.cpu().numpy()
    for e in range(n):
        ref = orc.dequant_f32(W.expert(e))
        assert np.array_equal(got[e].view(np.uint32), ref.view(np.uint32)), (case, e)


def test_dequant_subnormal_and_extreme_scales(orc):
    need_gpu()
    # products that land in the f32 subnormal range and near the top of it
    q = np.array([[0x00, 0xFF, 0x19, 0x91]], dtype=np.uint8)
    s = np.array([[1e-41, 3.0e38]], dtype=np.float32)
    W = QMat(4, 1, 8, 4, q, s)
    T = qtensor(W)
    w = torch.zeros((1, 1, 8), device="cuda")
    coli.check(coli.coli_dequantize(T, w))
    assert np.array_equal(w.cpu().numpy()[0].view(np.uint32), orc.dequant_f32(W).view(np.uint32))


KERNELS = pytest.mark.parametrize("kmode", [0, 1], ids=["mfma", "valu"])


@KERNELS
@pytest.mark.parametrize("case", SMALL, ids=[_id(c) for c in SMALL])
def test_qmatmul_small(orc, case, kmode):
    need_gpu()
    fmt, O, I, gs, S, n = case
    W, x = make_case(fmt, O, I, gs, S, seed=1 + hash(case) % 1000, n=n if n > 1 else None)
    T = qtensor(W, pack=(kmode == 0))
    with decode_kernels(kmode):
        y = gpu_qmatmul(T, x, n)
    tol = TOL_FP32 if S <= coli.coli_gemv_max_rows() else TOL_BF16
    for e in range(n):
        y_ref, A = orc.qmatmul(W.expert(e), x)
        assert_within(y[e], y_ref, A, tol, f"{case} expert {e}")


@KERNELS
def test_qmatmul_nibble_extremes_and_outliers(orc, kmode):
    """Rows of all 0x00 / all 0xFF bytes (-8 / +7), zero rows (0x88), and
    outlier-heavy rows (one large group scale), S = 1..4."""
    need_gpu()
    coli.coli_set_decode_kernel(kmode)
    r = sd.rng(77)
    O, I, gs = 8, 2048, 64
    q = sd.gen_codes(r, 4, O, I)
    q[0] = 0x00
    q[1] = 0xFF
    q[2] = 0x88
    q[3, : I // 4] = 0x88
    s = sd.gen_scales(r, 4, O, I, gs)
    s[4, 7] = 50.0
    s[5, :] = 1e-3
    s[5, 3] = 1e3
    W = QMat(4, O, I, gs, q, s)
    T = qtensor(W, pack=(kmode == 0))
    for S in (1, 2, 3, 4):
        x = sd.gen_x(r, S, I)
        x[:, 100] = 1e4
        y = gpu_qmatmul(T, x)[0]
        y_ref, A = orc.qmatmul(W, x)
        assert_within(y, y_ref, A, TOL_FP32, f"extremes S={S}")
        assert np.all(y[:, 2] == 0.0)
    coli.coli_set_decode_kernel(0)


@KERNELS
@pytest.mark.parametrize("S", [1, 2, 3, 4])
def test_qmatmul_one_hot_columns_exact(orc, S, kmode):
    """x = e_i picks column i: the GPU result equals s*v exactly."""
    need_gpu()
    W, _ = make_case(4, 64, 2048, 64, 1, seed=5)
    T = qtensor(W, pack=(kmode == 0))
    coli.coli_set_decode_kernel(kmode)
    cols = [0, 31, 32, 1000, 2047][:S]
    x = np.zeros((S, 2048), np.float32)
    for t, c in enumerate(cols):
        x[t, c] = 1.0
    y = gpu_qmatmul(T, x)[0]
    coli.coli_set_decode_kernel(0)
    w = orc.dequant_f32(W)
    for t, c in enumerate(cols):
        assert np.array_equal(y[t], w[:, c]), (S, c)


@KERNELS
def test_qmatmul_config1_full(orc, kmode):
    """Single fmt-4 GEMV: O=1024, I=2048, gs=64, S=1, seed 0, on the packed
    matrix-core path (the one the benchmark times) and the vector-ALU path."""
    need_gpu()
    W, x = make_case(4, 1024, 2048, 64, 1, seed=0)
    with decode_kernels(kmode):
        y = gpu_qmatmul(qtensor(W, pack=(kmode == 0)), x)[0]
    y_ref, A = orc.qmatmul(W, x)
    assert_within(y, y_ref, A, TOL_FP32, "config 1")


ZW = [(4, 64), (4, 128), (2, 0), (1, 0), (3, 0)]


@KERNELS
@pytest.mark.parametrize("fmt,gs", ZW, ids=[f"fmt{f}-gs{g}" for f, g in ZW])
def test_qmatmul_zero_weight_outliers(orc, fmt, gs, kmode):
    """Huge inputs at columns whose weights are zero in every row, among
    N(0,1) inputs (S = 1..4, 1e7 .. 1e30).  The matrix-core kernels give every
    (input row, 128-input block) one power of two, so such a block loses
    resolution: they must stay within 1e-5 A + 2^-29 Ahat.  The vector-ALU
    kernels multiply the floats themselves and hold the plain 1e-5 A."""
    need_gpu()
    O, I = 272, 2176
    r = sd.rng(300 + fmt + gs)
    q, s = sd.gen_matrix(r, fmt, O, I, gs)
    cols = (5, 700, 2100)
    for c in cols:
        zero_column(q, fmt, c)
    W = QMat(fmt, O, I, gs if fmt == 4 else 0, q, s)
    assert np.all(orc.dequant_f64(W)[:, list(cols)] == 0.0)
    T = qtensor(W, pack=(kmode == 0))
    for S in (1, 2, 3, 4):
        for mag in (1e7, 1e12, 1e30):
            x = sd.gen_x(r, S, I)
            for t in range(S):
                x[t, cols[t % 3]] = mag if t % 2 == 0 else -mag
            with decode_kernels(kmode):
                y = gpu_qmatmul(T, x)[0]
            y_ref, A = orc.qmatmul(W, x)
            extra = rep_allowance(orc, W, x) if kmode == 0 else None
            assert_within(y, y_ref, A, TOL_FP32, f"fmt {fmt} S {S} outlier {mag:g}", extra)


SWEEP = [(1, 0), (2, 0), (3, 0), (4, 64), (4, 128)]


@KERNELS
@pytest.mark.parametrize("fmt,gs", SWEEP, ids=[f"fmt{f}-gs{g}" for f, g in SWEEP])
@pytest.mark.parametrize("S", [1, 4])
def test_qmatmul_format_sweep_full(orc, fmt, gs, S, kmode):
    """Format sweep at full size: O = I = 6144, S in {1, 4}."""
    need_gpu()
    W, x = make_case(fmt, 6144, 6144, gs, S, seed=10 + fmt + gs + S)
    with decode_kernels(kmode):
        y = gpu_qmatmul(qtensor(W, pack=(kmode == 0)), x)[0]
    y_ref, A = orc.qmatmul(W, x)
    assert_within(y, y_ref, A, TOL_FP32, f"sweep fmt {fmt} gs {gs} S {S}")


@pytest.mark.parametrize("pack", [True, False], ids=["packed", "plain"])
@pytest.mark.parametrize("O,I", [(1536, 6144), (16384, 1536), (576, 6144), (6144, 16384)])
def test_qmatmul_attention_projection_shapes(orc, O, I, pack):
    """The decode layer's projections (q_a, q_b, kv_a, o_proj), fmt 4 g64."""
    need_gpu()
    W, x = make_case(4, O, I, 64, 1, seed=O + I)
    y = gpu_qmatmul(qtensor(W, pack=pack), x)[0]
    y_ref, A = orc.qmatmul(W, x)
    assert_within(y, y_ref, A, TOL_FP32, f"proj {O}x{I}")


@pytest.mark.parametrize("fmt,gs,S", [(4, 64, 1), (4, 64, 2), (4, 32, 3), (4, 128, 4), (1, 0, 2),
                                      (3, 0, 4), (2, 0, 1)])
def test_qmatmul_long_rows_several_input_segments(orc, fmt, gs, S):
    """Rows of 17056 inputs (a partial last group at gs 64): the matrix-core
    kernel stages the inputs in two or three segments, the next segment's
    first weight requests going out before its restaging."""
    need_gpu()
    W, x = make_case(fmt, 200, 17056, gs, S, seed=40 + fmt + gs + S)
    y = gpu_qmatmul(qtensor(W, pack=True), x)[0]
    y_ref, A = orc.qmatmul(W, x)
    assert_within(y, y_ref, A, TOL_FP32, f"long rows fmt {fmt} gs {gs} S {S}",
                  rep_allowance(orc, W, x))


def test_qmatmul_repeatable_bitwise(orc):
    need_gpu()
    W, x = make_case(4, 3000, 6144, 64, 3, seed=9)
    T = qtensor(W, pack=True)
    a = gpu_qmatmul(T, x)
    b = gpu_qmatmul(T, x)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_qmatmul_unaligned_x_and_stream(orc):
    """An x view at a 4-byte (not 16-byte) offset takes the exact fallback;
    work on a side stream is ordered on that stream."""
    need_gpu()
    W, x = make_case(4, 40, 256, 64, 2, seed=3)
    T = qtensor(W)
    buf = torch.zeros(2 * 256 + 1, device="cuda")
    buf[1:].copy_(torch.from_numpy(x.reshape(-1)))
    xv = buf[1:]
    y = torch.zeros((2, 40), device="cuda")
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        coli.check(coli.coli_qmatmul(T, xv, y, 2, st))
    st.synchronize()
    y_ref, A = orc.qmatmul(W, x)
    assert_within(y.cpu().numpy(), y_ref, A, TOL_FP32, "unaligned x")


def test_fault_injection_writes_nothing(orc):
    need_gpu()
    W, x = make_case(4, 16, 128, 64, 1, seed=4)
    T = qtensor(W)
    xd = to_dev(x)
    y = torch.full((1, 16), 123.0, device="cuda")
    coli.coli_set_fail_after(1)
    try:
        assert coli.coli_qmatmul(T, xd, y, 1) == coli.COLI_OK
        torch.cuda.synchronize()
        y.fill_(123.0)
        assert coli.coli_qmatmul(T, xd, y, 1) == coli.COLI_DECLINED
        torch.cuda.synchronize()
        assert torch.all(y == 123.0)
    finally:
        coli.coli_set_fail_after(-1)


def test_pack_leaves_other_paths_unchanged(orc):
    """A packed tensor still serves the prefill GEMM and the vector-ALU kernels
    from its original codes; results with and without the packed copy agree
    with the oracle."""
    need_gpu()
    W, x = make_case(4, 100, 1024, 128, 9, seed=12)
    T = qtensor(W, pack=True)
    y_ref, A = orc.qmatmul(W, x)
    assert_within(gpu_qmatmul(T, x)[0], y_ref, A, TOL_BF16, "prefill on a packed tensor")
    for S in (1, 3):
        yr, Ar = orc.qmatmul(W, x[:S])
        with decode_kernels(1):
            assert_within(gpu_qmatmul(T, x[:S])[0], yr, Ar, TOL_FP32, "valu on a packed tensor")
        assert_within(gpu_qmatmul(T, x[:S])[0], yr, Ar, TOL_FP32, "mfma on a packed tensor")


@KERNELS
@pytest.mark.parametrize("bad", [float("nan"), float("inf")], ids=["nan", "inf"])
def test_qmatmul_nonfinite_input_propagates(orc, kmode, bad):
    """A NaN or inf input makes every output of its input row non-finite (as
    in the oracle, where NaN*w and inf*0 are NaN); other rows stay exact."""
    need_gpu()
    W, x = make_case(4, 40, 512, 64, 2, seed=21)
    x[0, 300] = bad
    with decode_kernels(kmode):
        y = gpu_qmatmul(qtensor(W, pack=(kmode == 0)), x)[0]
    y_ref, A = orc.qmatmul(W, x)
    assert not np.isfinite(y_ref[0]).any()
    assert not np.isfinite(y[0]).any()
    assert_within(y[1], y_ref[1], A[1], TOL_FP32, "finite row")


@pytest.mark.parametrize("fmt,O,I,gs,S", [(4, 4160, 512, 64, 1), (4, 4160, 640, 64, 4),
                                          (4, 4096, 384, 128, 3), (2, 4112, 256, 0, 2),
                                          (1, 4160, 512, 0, 1), (1, 4096, 384, 0, 4),
                                          (3, 4112, 640, 0, 2), (3, 4096, 256, 0, 4)])
def test_qmatmul_wide_stack(orc, fmt, O, I, gs, S):
    """Stacks with enough rows for 512 or more 64-row workgroups take a
    wider launch shape: every matrix against the oracle; for S >= 2 also
    bit-identical to the same matrix run alone (the narrower shape splits the
    inputs three ways per tile, as the wide S >= 2 shape does; the wide S = 1
    shape splits them two ways, so its sums are grouped differently)."""
    need_gpu()
    n = 8
    W, x = make_case(fmt, O, I, gs, S, seed=4000 + O + I + S, n=n)
    T = qtensor(W, pack=True)
    y = gpu_qmatmul(T, x, n)
    xd = to_dev(x.astype(np.float32))
    for e in range(n):
        y_ref, A = orc.qmatmul(W.expert(e), x)
        assert_within(y[e], y_ref, A, TOL_FP32, f"stack matrix {e}")
        if S == 1:
            continue
        Te = qtensor(W.expert(e), pack=True)
        alone = torch.full((1, S, O), float("nan"), device="cuda")
        coli.check(coli.coli_qmatmul(Te, xd, alone, S), "coli_qmatmul")
        torch.cuda.synchronize()
        assert np.array_equal(alone.cpu().numpy()[0].view(np.uint32), y[e].view(np.uint32)), e


@pytest.mark.parametrize("S", [1, 2, 4])
@pytest.mark.parametrize("fmt", [1, 3])
def test_qmatmul_per_row_packed_extremes(orc, fmt, S):
    """fmt 1 and fmt 3 on the matrix cores (packed copy): int8 codes -128 and
    127 side by side, every 2-bit code, rows of a single repeated code, a
    ragged last tile (O = 37) and inputs past the last whole block
    (I = 416), against the oracle."""
    need_gpu()
    O, I = 37, 416
    r = sd.rng(90 + fmt + S)
    x = sd.gen_x(r, S, I)
    q, s = sd.gen_matrix(r, fmt, O, I, 0)
    q = q.copy()
    if fmt == 1:
        q[0, 0::2], q[0, 1::2] = 0x80, 0x7F   # -128, 127
        q[1, :] = 0x80
        q[2, :] = 0x7F
    else:
        q[0, :] = 0b11100100                  # codes 0, 1, 2, 3 in every byte
        q[1, :] = 0x00                        # every weight -2
        q[2, :] = 0xFF                        # every weight +1
    W = QMat(fmt, O, I, 0, q, s)
    T = qtensor(W, pack=True)
    assert T.desc.flags & 8, "the packed copy should be attached"
    y = gpu_qmatmul(T, x)[0]
    y_ref, A = orc.qmatmul(W, x)
    assert_within(y, y_ref, A, TOL_FP32, f"fmt {fmt} S {S}")
