"""Shared helpers of the GPU parity tests: upload seeded host inputs, call the
C ABI through the binding, and compare with the oracle under the
magnitude-relative tolerances (colibri PR #298, matmul_i4_grouped test
commit: error is judged against the sum of |terms|, not |result|)."""
from __future__ import annotations

import contextlib

import numpy as np
import pytest
import torch

import bit_gemv_coli_amd as coli
import synthdata as sd
from oracle import QMat

TOL_FP32 = 1e-5   # fp32 GEMV path: |y - y_ref| <= 1e-5 * sum_i |w||x|
TOL_BF16 = 4e-3   # bf16 matrix-core path: |y - y_ref| <= 4e-3 * sum_i |w||x|

DEV = "cuda"


@contextlib.contextmanager
def decode_kernels(mode):
    """Run with the matrix-core (0) or vector-ALU (1) decode kernels."""
    old = coli.coli_set_decode_kernel(mode)
    try:
        yield
    finally:
        coli.coli_set_decode_kernel(old)


def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    if not __import__("os").path.exists(coli.LIB_PATH):
        pytest.fail("libcoli.so is not built")


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def qtensor(W: QMat, pack: bool = False) -> coli.QTensor:
    """Upload a host QMat (single matrix or stack) and describe it; with
    pack=True also attach the packed copy the matrix-core kernels read."""
    q = to_dev(W.q.view(np.uint8))
    s = to_dev(W.s.astype(np.float32))
    n = W.q.shape[0] if W.q.ndim == 3 else 1
    T = coli.QTensor(W.fmt, q, s, W.O, W.I, W.gs if W.fmt == 4 else 0, n=n)
    if pack:
        T.pack()
    return T


def gpu_qmatmul(T: coli.QTensor, x: np.ndarray, n: int = 1) -> np.ndarray:
    xd = to_dev(x.astype(np.float32))
    S = x.shape[0]
    y = torch.full((n, S, T.desc.O), float("nan"), device=DEV)
    coli.check(coli.coli_qmatmul(T, xd, y, S), "coli_qmatmul")
    torch.cuda.synchronize()
    return y.cpu().numpy()


def assert_within(y_gpu, y_ref, A, tol, what="", extra=None):
    """|y_gpu - y_ref| <= tol * A (+ extra, an absolute allowance per output,
    e.g. the matrix-core decode kernels' 2^-29 * Ahat input-resolution term)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    bound = tol * A if extra is None else tol * A + extra
    bad = ~(err <= bound)  # NaN counts as bad
    if bad.any():
        idx = np.argwhere(bad)[:5]
        ratio = np.nanmax(err / np.maximum(bound, 1e-300))
        raise AssertionError(f"{what}: {int(bad.sum())} outputs outside {tol:g}*A"
                             f"{'' if extra is None else ' + extra'}; "
                             f"max err/bound = {ratio:.3e}; first bad {idx.tolist()}")
    return float(np.max(err / np.maximum(A, 1e-300))) if err.size else 0.0


def rep_allowance(orc, W: QMat, x) -> np.ndarray:
    """2^-29 * Ahat per output: how far the matrix-core decode kernels' input
    representation (one power of two per input row and 128-input block) may
    move each output of W x."""
    from digit_model import REP_BOUND, block_magnitude
    return REP_BOUND * block_magnitude(np.abs(orc.dequant_f64(W)), x)


def zero_column(q: np.ndarray, fmt: int, col: int) -> None:
    """Set the codes of input column `col` to the format's zero in every row
    (q: uint8 [O][row_bytes], modified in place)."""
    if fmt in (2, 4):
        b = col // 2
        q[:, b] = (q[:, b] & 0x0F) | 0x80 if col % 2 else (q[:, b] & 0xF0) | 0x08
    elif fmt == 3:
        b, sh = col // 4, 2 * (col % 4)
        q[:, b] = (q[:, b] & np.uint8(~(3 << sh) & 0xFF)) | np.uint8(2 << sh)
    else:
        q[:, col] = 0


def make_case(fmt, O, I, gs, S, seed, n=None):
    r = sd.rng(seed)
    x = sd.gen_x(r, S, I)
    q, s = sd.gen_matrix(r, fmt, O, I, gs, n=n)
    return QMat(fmt, O, I, gs if fmt == 4 else 0, q, s), x
