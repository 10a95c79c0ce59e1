"""A numpy model of how the matrix-core decode kernels represent their inputs
(test infrastructure; it shares no code with the HIP library).

The kernels take every input row in blocks of 128 consecutive inputs counted
from the start of the row.  Per block b with largest magnitude M_b they pick a
power of two 2^e_b with 2^e_b * M_b in [2^29, 2^30) (e_b capped at 126 for
blocks below 2^-96), truncate X_i = trunc(x_i * 2^e_b) toward zero, and split
the int32 X_i into four signed byte digits.  The integer products with the
weight codes are exact, so what the kernels multiply is x_rep_i = X_i * 2^-e_b,
with |x_rep_i - x_i| < 2^-e_b <= 2^-29 * max(M_b, 2^-97).

Consequence for one output: the representation moves it by at most
    2^-29 * Ahat,   Ahat = sum_b max(M_b, 2^-97) * sum_{i in b} |w_i|,
which is small against A = sum_i |w_i||x_i| only while each block's largest
input is not far above the inputs that carry its weight (a huge input where
the weights are zero still sets the block's resolution).
"""
from __future__ import annotations

import numpy as np

BLOCK = 128
E_CAP = 126
FLOOR = 2.0 ** -97  # blocks below this all use 2^-126 as their step


def pad_blocks(x: np.ndarray) -> np.ndarray:
    """x [S][I] -> [S][nb][128] with zeros past I (the kernels read zeros there)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float32))
    S, I = x.shape
    nb = -(-I // BLOCK)
    xp = np.zeros((S, nb * BLOCK), np.float64)
    xp[:, :I] = x
    return xp.reshape(S, nb, BLOCK)


def block_exponents(x: np.ndarray):
    """Per (row, block): the largest magnitude M_b and the exponent e_b."""
    xb = pad_blocks(x)
    M = np.max(np.abs(xb), axis=2)
    _, E = np.frexp(M)             # M = m * 2^E, m in [0.5, 1)
    e = np.minimum(30 - E, E_CAP)
    e = np.where(M > 0, e, 0)
    return M, e.astype(np.int64)


def represent(x: np.ndarray):
    """(x_rep f64 [S][I], X int64 [S][nb][128], e int64 [S][nb])."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float32))
    S, I = x.shape
    xb = pad_blocks(x)
    _, e = block_exponents(x)
    X = np.trunc(np.ldexp(xb, e[:, :, None])).astype(np.int64)
    x_rep = np.ldexp(X.astype(np.float64), -e[:, :, None]).reshape(S, -1)[:, :I]
    return x_rep, X, e


def byte_digits(X: np.ndarray) -> np.ndarray:
    """Four signed byte digits d with X = d0 + 2^8 d1 + 2^16 d2 + 2^24 d3, read
    as the bytes of (X + 0x808080) XOR 0x808080 (|X| < 2^30)."""
    u = ((np.asarray(X, np.int64) + 0x808080) & 0xFFFFFFFF) ^ 0x808080
    b = np.stack([(u >> (8 * k)) & 0xFF for k in range(4)], axis=-1)
    return np.where(b >= 128, b - 256, b).astype(np.int64)


def block_magnitude(w_abs: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Ahat [S][O] for |w| f64 [O][I] and inputs x [S][I]."""
    M, _ = block_exponents(x)
    O, I = w_abs.shape
    nb = M.shape[1]
    wb = np.zeros((O, nb * BLOCK))
    wb[:, :I] = w_abs
    wsum = wb.reshape(O, nb, BLOCK).sum(axis=2)     # [O][nb]
    return np.maximum(M, FLOOR) @ wsum.T


REP_BOUND = 2.0 ** -29  # coefficient of Ahat in the matrix-core decode bound
