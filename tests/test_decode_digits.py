"""CPU checks of the matrix-core decode kernels' input representation (the
model in digit_model.py) against the oracle: where the plain bound
|y - y_ref| <= 1e-5 * sum_i |w||x| holds, where it breaks, and the bound that
holds always, |y - y_ref| <= 1e-5 * A + 2^-29 * Ahat.

Tolerances are magnitude-relative (colibri PR #298, matmul_i4_grouped test
commit: the error is judged against the sum of |terms|)."""
import numpy as np
import pytest

import synthdata as sd
from digit_model import REP_BOUND, block_exponents, block_magnitude, byte_digits, represent
from oracle import QMat


def test_byte_digits_reconstruct():
    """The byte split of (X + 0x808080) XOR 0x808080 gives four signed digits
    that sum back to X for every |X| < 2^30 (edges and random values)."""
    edge = [0, 1, -1, 127, 128, 129, -127, -128, -129, 255, 256, -256, 0x7F7F7F, -0x7F7F7F,
            0x808080, -0x808080, 2**23, -2**23, 2**24 - 1, -(2**24 - 1), 2**29, -2**29,
            2**30 - 1, -(2**30 - 1)]
    r = np.random.default_rng(0)
    X = np.concatenate([np.array(edge, np.int64),
                        r.integers(-(2**30) + 1, 2**30, size=200000, dtype=np.int64)])
    d = byte_digits(X)
    assert d.min() >= -128 and d.max() <= 127
    rec = d[:, 0] + (d[:, 1] << 8) + (d[:, 2] << 16) + (d[:, 3] << 24)
    assert np.array_equal(rec, X)


def test_representation_step():
    """|x_rep - x| < 2^-e_b <= 2^-29 max(M_b, 2^-97), and the block's largest
    |X| lies in [2^29, 2^30) whenever M_b is a normal number above 2^-96."""
    r = np.random.default_rng(1)
    S, I = 4, 128 * 9 + 40
    x = (r.standard_normal((S, I)) * np.exp(r.uniform(-80, 80, (S, I)))).astype(np.float32)
    x[0, :128] *= 1e-30                     # a block below 2^-96: capped exponent
    x[1, 128:256] = 0.0                     # an all-zero block
    x[2, 300] = 3.0e38                      # a block near the f32 limit
    x_rep, X, e = represent(x)
    M, _ = block_exponents(x)
    step = np.ldexp(1.0, -e)                # [S][nb]
    stepi = np.repeat(step, 128, axis=1)[:, :I]
    err = np.abs(x_rep - x.astype(np.float64))
    assert np.all((err < stepi) | (x == 0))
    nz = M > 0  # an all-zero block is represented exactly whatever its step
    assert np.all(step[nz] <= REP_BOUND * np.maximum(M[nz], 2.0 ** -97))
    assert np.all(x_rep[1, 128:256] == 0.0)
    big = M > 2.0 ** -96
    Xmax = np.max(np.abs(X), axis=2)
    assert np.all((Xmax[big] >= 2**29) & (Xmax[big] < 2**30))
    assert np.all(Xmax[~big] < 2**30)


def _zero_column(q, fmt, col):
    """Set the codes of input column `col` to the format's zero value in every row."""
    if fmt in (2, 4):
        b, hi = col // 2, col % 2
        q[:, b] = (q[:, b] & 0x0F) | 0x80 if hi else (q[:, b] & 0xF0) | 0x08
    elif fmt == 3:
        b, sh = col // 4, 2 * (col % 4)
        q[:, b] = (q[:, b] & ~np.uint8(3 << sh)) | np.uint8(2 << sh)
    else:
        q[:, col] = 0


def _case(orc, fmt, gs, O, I, S, seed, outlier=None, cols=()):
    r = sd.rng(seed)
    x = sd.gen_x(r, S, I)
    q, s = sd.gen_matrix(r, fmt, O, I, gs)
    for c in cols:
        _zero_column(q, fmt, c)
        if outlier is not None:
            x[:, c] = np.float32(outlier) * np.where(np.arange(S) % 2 == 0, 1, -1)
    W = QMat(fmt, O, I, gs if fmt == 4 else 0, q, s)
    w64 = orc.dequant_f64(W)
    if cols:
        assert np.all(w64[:, list(cols)] == 0.0)
    y_ref, A = orc.qmatmul(W, x)
    x_rep, _, _ = represent(x)
    y_rep = x_rep @ w64.T
    Ahat = block_magnitude(np.abs(w64), x)
    return np.abs(y_rep - y_ref), A, Ahat


@pytest.mark.parametrize("fmt,gs", [(4, 64), (4, 128), (2, 0), (1, 0), (3, 0)])
def test_normal_inputs_far_inside(orc, fmt, gs):
    """N(0,1) inputs (the workloads' activations): the representation alone
    moves outputs by < 1e-7 A, a hundredth of the fp32 budget."""
    err, A, Ahat = _case(orc, fmt, gs, 128, 6144, 4, seed=3 + fmt + gs)
    assert np.all(err <= REP_BOUND * Ahat)
    assert np.max(err / A) < 1e-7
    assert np.max(Ahat / A) < 8.0


@pytest.mark.parametrize("I", [6144, 2048])
def test_zero_weight_outlier_breaks_plain_bound(orc, I):
    """One input column whose weights are zero in every row carries an
    outlier: the block's resolution follows the outlier, the other inputs of
    its 128-input block lose precision.  The bound with Ahat holds at every
    magnitude; the plain 1e-5 A bound holds up to ~1e5 and fails from ~1e7
    (I = 6144) -- the limit the header states."""
    worst = {}
    for mag in (1e3, 1e5, 1e6, 1e7, 1e8, 1e12, 1e30):
        err, A, Ahat = _case(orc, 4, 64, 256, I, 2, seed=11, outlier=mag, cols=(1000,))
        assert np.all(err <= REP_BOUND * Ahat + 1e-12 * A), mag
        worst[mag] = float(np.max(err / A))
    assert worst[1e3] < 1e-7 and worst[1e5] < 1e-5
    assert worst[1e8] > 1e-5 and worst[1e12] > 1e-2
    # the plain bound fails exactly where 2^-29 Ahat outgrows it
    assert worst[1e7] > (1e-5 if I == 2048 else 1e-6)


def test_outlier_with_weight_is_harmless(orc):
    """An outlier where the weights are not zero carries its own term in A:
    the plain bound holds even at 1e30."""
    r = sd.rng(12)
    x = sd.gen_x(r, 2, 6144)
    q, s = sd.gen_matrix(r, 4, 256, 6144, 64)
    x[:, 1000] = 1e30
    W = QMat(4, 256, 6144, 64, q, s)
    w64 = orc.dequant_f64(W)
    live = w64[:, 1000] != 0
    y_ref, A = orc.qmatmul(W, x)
    x_rep, _, _ = represent(x)
    err = np.abs(x_rep @ w64.T - y_ref)
    assert np.max(err[:, live] / A[:, live]) < 1e-7
