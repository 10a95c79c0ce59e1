"""Pins of the CPU oracle to facts other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with what the pages or the mathematics fix:
  - values the pages print (the nibble extremes),
  - closed forms (group sums with power-of-two scales, ramps),
  - invariants (one-hot inputs, zero codes, scale doubling, row independence),
  - special cases that reduce to another format or to a library routine
    (scipy's logistic function, numpy's f64 matmul on an independently
    written decoder),
  - brute force on tiny inputs (routing by sorting).
The same functions run against deliberately broken copies of the oracle in
``test_oracle_mutations.py`` to show that they bite.
"""
from __future__ import annotations

import json
import os

import numpy as np
from scipy.special import expit

import synthdata as sd
from oracle import QMat

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# An independent decoder: vectorised bit slicing with numpy (a different
# construction from the oracle's per-element function).
# ---------------------------------------------------------------------------

def ref_codes(fmt: int, q: np.ndarray, I: int) -> np.ndarray:
    q = q.view(np.uint8)
    O = q.shape[0]
    if fmt == 1:
        return q.view(np.int8).astype(np.int64)[:, :I]
    if fmt in (2, 4):
        both = np.stack([q & 0x0F, q >> 4], axis=-1).reshape(O, -1)
        return both[:, :I].astype(np.int64) - 8
    if fmt == 3:
        shifts = np.array([0, 2, 4, 6], dtype=np.uint8)
        crumbs = (q[:, :, None] >> shifts[None, None, :]) & 0x3
        return crumbs.reshape(O, -1)[:, :I].astype(np.int64) - 2
    raise ValueError(fmt)


def ref_dense(W: QMat) -> np.ndarray:
    """Exact f64 weights from the independent decoder."""
    v = ref_codes(W.fmt, W.q, W.I).astype(np.float64)
    if W.fmt == 4:
        col_scale = np.repeat(W.s.astype(np.float64), W.gs, axis=1)[:, :W.I]
        return v * col_scale
    return v * W.s.astype(np.float64)[:, None]


def make(fmt, O, I, gs=64, seed=0, S=1):
    r = sd.rng(seed)
    x = sd.gen_x(r, S, I)
    q, s = sd.gen_matrix(r, fmt, O, I, gs)
    return QMat(fmt, O, I, gs if fmt == 4 else 0, q, s), x


# The shape matrix of the grouped-int4 test commit (PR #298): I a multiple of
# gs, a partial last group, odd I, gs > I, gs = 16/64/128, S > 1; plus the
# per-row formats on odd / non-multiple-of-4 widths.
SHAPES = [
    (4, 8, 128, 64, 1), (4, 5, 130, 64, 1), (4, 3, 129, 64, 2), (4, 4, 37, 64, 1),
    (4, 6, 96, 16, 3), (4, 4, 256, 128, 1), (4, 2, 1, 16, 1), (4, 7, 200, 32, 4),
    (2, 5, 130, 0, 2), (2, 3, 33, 0, 1), (1, 4, 70, 0, 3), (1, 2, 5, 0, 1),
    (3, 5, 130, 0, 2), (3, 3, 7, 0, 1), (3, 2, 66, 0, 1),
]


def _assert_close_A(y, y_ref, A, rel):
    err = np.abs(y - y_ref)
    bound = rel * A + 1e-300
    assert np.all(err <= bound), f"max err/A = {np.max(err / np.maximum(A, 1e-300)):.3e}"


# ---------------------------------------------------------------------------
# Format pins
# ---------------------------------------------------------------------------

def pin_golden_nibble_extremes(orc):
    """Page-printed values: 0x00 -> -8, 0xFF -> +7 (offset encoding)."""
    with open(os.path.join(GOLDEN, "nibble_extremes.json")) as f:
        g = json.load(f)
    for fmt in (2, 4):
        for case in g["cases"]:
            q = np.array([[case["byte"]]], dtype=np.uint8)
            v = orc.decode_codes(QMat(fmt, 1, 2, 2 if fmt == 4 else 0, q,
                                      np.ones((1, 1) if fmt == 4 else (1,), np.float32)))
            assert v.tolist() == [case["values"]], (fmt, case, v)


def pin_midpoint_and_order(orc):
    """Nibble 8 is zero; byte 0x9F holds 15 in its low nibble (element 0,
    value +7) and 9 in its high nibble (element 1, value +1)."""
    q = np.array([[0x88, 0x9F]], dtype=np.uint8)
    v = orc.decode_codes(QMat(2, 1, 4, 0, q, np.ones(1, np.float32)))
    assert v.tolist() == [[0, 0, 7, 1]], v
    # fmt 3: byte 0b11_10_01_00 holds codes 0,1,2,3 from the lowest bits up
    q3 = np.array([[0b11100100]], dtype=np.uint8)
    v3 = orc.decode_codes(QMat(3, 1, 4, 0, q3, np.ones(1, np.float32)))
    assert v3.tolist() == [[-2, -1, 0, 1]], v3
    # fmt 1: two's complement bytes
    q1 = np.array([[0x7F, 0x80, 0xFF, 0x01]], dtype=np.uint8)
    v1 = orc.decode_codes(QMat(1, 1, 4, 0, q1, np.ones(1, np.float32)))
    assert v1.tolist() == [[127, -128, -1, 1]], v1


def pin_decoder_matches_independent(orc):
    for fmt, O, I, gs, _ in SHAPES:
        W, _ = make(fmt, O, I, gs, seed=fmt * 100 + I)
        assert np.array_equal(orc.decode_codes(W), ref_codes(fmt, W.q, I)), (fmt, O, I)


def pin_dequant_single_rounding(orc):
    """f32 dequant equals one rounding of the exact product s*v."""
    for fmt, O, I, gs, _ in SHAPES:
        W, _ = make(fmt, O, I, gs, seed=7 + I)
        exact = ref_dense(W)
        assert np.array_equal(orc.dequant_f64(W), exact), (fmt, O, I)
        assert np.array_equal(orc.dequant_f32(W).view(np.uint32),
                              exact.astype(np.float32).view(np.uint32)), (fmt, O, I)


# ---------------------------------------------------------------------------
# Matmul pins
# ---------------------------------------------------------------------------

def pin_bruteforce_dense(orc):
    """Dequantise with the independent decoder, then numpy's f64 matmul."""
    for fmt, O, I, gs, S in SHAPES:
        W, x = make(fmt, O, I, gs, seed=11 + I + fmt, S=S)
        y, A = orc.qmatmul(W, x)
        Wd = ref_dense(W)
        y_ref = x.astype(np.float64) @ Wd.T
        A_ref = np.abs(x.astype(np.float64)) @ np.abs(Wd).T
        _assert_close_A(y, y_ref, A_ref, 1e-12)
        assert np.allclose(A, A_ref, rtol=1e-12, atol=0), (fmt, O, I)


def pin_closed_form_group_sums(orc):
    """x = 1, every nibble 15 (value +7), group scales 2^g:
    y = 7 * sum_g 2^g * len_g with the last group holding I - (ng-1)*gs."""
    for I, gs in [(130, 64), (129, 64), (37, 64), (96, 16), (200, 32), (64, 64), (1, 16)]:
        ng = -(-I // gs)
        q = np.full((2, (I + 1) // 2), 0xFF, dtype=np.uint8)
        s = np.tile(np.array([2.0 ** g for g in range(ng)], dtype=np.float32), (2, 1))
        s[1] *= 0.5
        W = QMat(4, 2, I, gs, q, s)
        y, _ = orc.qmatmul(W, np.ones((1, I), np.float32))
        lens = [gs] * (ng - 1) + [I - (ng - 1) * gs]
        expect = 7.0 * sum((2.0 ** g) * lens[g] for g in range(ng))
        assert y[0, 0] == expect and y[0, 1] == expect / 2, (I, gs, y, expect)


def pin_closed_form_ramp(orc):
    """x_i = i, nibbles alternate 0 / 15 (values -8 / +7), scale 1 per row:
    y = sum_even(-8 i) + sum_odd(7 i)."""
    for I in (8, 9, 130, 257):
        q = np.full((1, (I + 1) // 2), 0xF0, dtype=np.uint8)  # low nibble 0, high 15
        W = QMat(2, 1, I, 0, q, np.ones(1, np.float32))
        x = np.arange(I, dtype=np.float32)[None, :]
        y, _ = orc.qmatmul(W, x)
        expect = sum(-8 * i for i in range(0, I, 2)) + sum(7 * i for i in range(1, I, 2))
        assert y[0, 0] == expect, (I, y, expect)


def pin_one_hot_columns(orc):
    for fmt, O, I, gs, _ in SHAPES:
        W, _ = make(fmt, O, I, gs, seed=5 + I)
        Wd = ref_dense(W)
        for i in sorted({0, I // 2, I - 1}):
            x = np.zeros((1, I), np.float32)
            x[0, i] = 1.0
            y, _ = orc.qmatmul(W, x)
            assert np.array_equal(y[0], Wd[:, i]), (fmt, I, i)


def pin_zero_and_unit(orc):
    for I in (1, 7, 64, 130):
        # all nibbles 8 -> every weight 0
        W = QMat(4, 3, I, 16, np.full((3, (I + 1) // 2), 0x88, np.uint8),
                 np.full((3, -(-I // 16)), 0.37, np.float32))
        y, _ = orc.qmatmul(W, np.ones((1, I), np.float32))
        assert np.all(y == 0.0)
        # scale 1, value +1 (nibble 9), x = 1 -> y = I
        W1 = QMat(4, 2, I, 16, np.full((2, (I + 1) // 2), 0x99, np.uint8),
                  np.ones((2, -(-I // 16)), np.float32))
        y1, _ = orc.qmatmul(W1, np.ones((1, I), np.float32))
        assert np.all(y1 == I), (I, y1)


def pin_scale_doubling_and_rows(orc):
    W, x = make(4, 6, 200, 64, seed=3, S=3)
    y, _ = orc.qmatmul(W, x)
    W2 = QMat(4, 6, 200, 64, W.q, W.s * 2)
    y2, _ = orc.qmatmul(W2, x)
    assert np.array_equal(y2, 2 * y)
    for t in range(3):
        yt, _ = orc.qmatmul(W, x[t:t + 1])
        assert np.array_equal(yt[0], y[t])


def pin_cross_format(orc):
    r = sd.rng(21)
    O = 4
    for I in (64, 130, 37):
        x = sd.gen_x(r, 2, I)
        q = sd.gen_codes(r, 2, O, I)
        s = sd.gen_scales(r, 2, O, I, 0)
        y2, _ = orc.qmatmul(QMat(2, O, I, 0, q, s), x)
        # fmt 4 with gs = I, and with gs > I, equals fmt 2 with s[o]
        for gs in (I, I + 5, 4 * I):
            y4, _ = orc.qmatmul(QMat(4, O, I, gs, q, s[:, None].copy()), x)
            assert np.array_equal(y4, y2), (I, gs)
        # equal group scales along a row equal fmt 2
        ng = -(-I // 16)
        y4e, _ = orc.qmatmul(QMat(4, O, I, 16, q, np.repeat(s[:, None], ng, axis=1)), x)
        _assert_close_A(y4e, y2, np.abs(y2) + 1, 1e-13)
        # values in -2..1 give the same result in fmt 1 / 2 / 3
        v = r.integers(-2, 2, size=(O, I))
        q1 = v.astype(np.int8).view(np.uint8)
        nib = (v + 8).astype(np.uint8)
        nib = np.pad(nib, ((0, 0), (0, (-I) % 2)), constant_values=8)
        q2 = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
        cr = (v + 2).astype(np.uint8)
        cr = np.pad(cr, ((0, 0), (0, (-I) % 4)), constant_values=2)
        q3 = (cr[:, 0::4] | (cr[:, 1::4] << 2) | (cr[:, 2::4] << 4) | (cr[:, 3::4] << 6)).astype(np.uint8)
        ya, _ = orc.qmatmul(QMat(1, O, I, 0, q1, s), x)
        yb, _ = orc.qmatmul(QMat(2, O, I, 0, q2, s), x)
        yc, _ = orc.qmatmul(QMat(3, O, I, 0, q3, s), x)
        assert np.array_equal(ya, yb) and np.array_equal(yb, yc), I


# ---------------------------------------------------------------------------
# SiLU and routing pins
# ---------------------------------------------------------------------------

def pin_silu(orc):
    assert orc.silu(0.0) == 0.0
    for z in (0.1, 0.5, 1.0, 3.0, 10.0):
        assert abs(orc.silu(-z) - (orc.silu(z) - z)) <= 1e-15 * (1 + z)
    for z in np.linspace(-30, 30, 121):
        ref = float(z) * float(expit(z))
        assert abs(orc.silu(float(z)) - ref) <= 1e-15 * (1 + abs(ref)), z


def pin_route_bruteforce(orc):
    r = sd.rng(4)
    for S, K, E in [(1, 8, 256), (3, 2, 5), (7, 3, 4), (16, 4, 64), (5, 1, 1), (0, 8, 16)]:
        ids = r.integers(0, E, size=(S, K)).astype(np.int32)
        counts, offsets, perm, bad = orc.moe_route(ids, E)
        assert bad == 0
        pairs = sorted(range(S * K), key=lambda p: (int(ids.flat[p]), p))
        assert perm.tolist() == pairs
        assert counts.tolist() == [int(np.sum(ids == e)) for e in range(E)]
        assert offsets.tolist() == [0] + list(np.cumsum(counts))
        assert offsets[-1] == S * K
    ids = np.array([[0, 9, 2], [-1, 2, 2]], dtype=np.int32)
    counts, offsets, perm, bad = orc.moe_route(ids, 4)
    assert bad == 2 and counts.tolist() == [1, 0, 3, 0]
    assert perm[:4].tolist() == [0, 2, 4, 5]


# ---------------------------------------------------------------------------
# MoE block pins
# ---------------------------------------------------------------------------

def _moe_case(seed, S, K, E, D, F, gs=32, shared=False):
    r = sd.rng(seed)
    x = sd.gen_x(r, S, D)
    gq, gs_ = sd.gen_matrix(r, 4, F, D, gs, n=E)
    uq, us = sd.gen_matrix(r, 4, F, D, gs, n=E)
    dq, ds = sd.gen_matrix(r, 4, D, F, gs, n=E)
    ids, w = sd.gen_routing_uniform(r, S, K, E)
    G, U, Dn = QMat(4, F, D, gs, gq, gs_), QMat(4, F, D, gs, uq, us), QMat(4, D, F, gs, dq, ds)
    sh = None
    if shared:
        a, b = sd.gen_matrix(r, 4, F, D, gs)
        c, d = sd.gen_matrix(r, 4, F, D, gs)
        e_, f_ = sd.gen_matrix(r, 4, D, F, gs)
        sh = (QMat(4, F, D, gs, a, b), QMat(4, F, D, gs, c, d), QMat(4, D, F, gs, e_, f_))
    return G, U, Dn, x, ids, w, sh


def _mlp_dense(G, U, Dn, xs):
    g = ref_dense(G) @ xs
    u = ref_dense(U) @ xs
    h = g * expit(g) * u
    return ref_dense(Dn) @ h, np.abs(ref_dense(Dn)) @ np.abs(h)


def pin_moe_bruteforce(orc):
    """Dense numpy expert MLPs on the independent decoder, weighted by w."""
    for seed, S, K, E, D, F, shared in [(1, 1, 1, 1, 64, 32, False), (2, 3, 2, 5, 70, 40, True),
                                        (3, 2, 4, 6, 96, 33, False)]:
        G, U, Dn, x, ids, w, sh = _moe_case(seed, S, K, E, D, F, shared=shared)
        out = orc.moe_block(G, U, Dn, x, ids, w, shared=sh)
        for s in range(S):
            ref = np.zeros(D)
            mag = np.zeros(D)
            xs = x[s].astype(np.float64)
            for k in range(K):
                e = int(ids[s, k])
                y, m = _mlp_dense(G.expert(e), U.expert(e), Dn.expert(e), xs)
                ref += float(w[s, k]) * y
                mag += abs(float(w[s, k])) * m
            if sh is not None:
                y, m = _mlp_dense(*sh, xs)
                ref += y
                mag += m
            _assert_close_A(out[s], ref, mag, 1e-12)


def pin_moe_invariants(orc):
    G, U, Dn, x, ids, w, sh = _moe_case(9, 3, 3, 7, 64, 48, shared=True)
    out = orc.moe_block(G, U, Dn, x, ids, w)
    # zero weights give zero
    assert np.all(orc.moe_block(G, U, Dn, x, ids, np.zeros_like(w)) == 0.0)
    # doubling w doubles the output exactly
    assert np.array_equal(orc.moe_block(G, U, Dn, x, ids, 2 * w), 2 * out)
    # relabelling the experts (permuting the stack and the ids) changes nothing
    perm = np.array([3, 0, 6, 1, 5, 2, 4])
    inv = np.argsort(perm)
    Gp = QMat(4, G.O, G.I, G.gs, G.q[perm], G.s[perm])
    Up = QMat(4, U.O, U.I, U.gs, U.q[perm], U.s[perm])
    Dp = QMat(4, Dn.O, Dn.I, Dn.gs, Dn.q[perm], Dn.s[perm])
    assert np.array_equal(orc.moe_block(Gp, Up, Dp, x, inv[ids].astype(np.int32), w), out)
    # each row of a batch equals the same row run alone
    for s in range(3):
        assert np.array_equal(orc.moe_block(G, U, Dn, x[s:s + 1], ids[s:s + 1], w[s:s + 1])[0], out[s])
    # the shared expert equals an extra routed expert with weight 1 on every row
    with_sh = orc.moe_block(G, U, Dn, x, ids, w, shared=sh)
    Ge = QMat(4, G.O, G.I, G.gs, np.concatenate([G.q, sh[0].q[None]]), np.concatenate([G.s, sh[0].s[None]]))
    Ue = QMat(4, U.O, U.I, U.gs, np.concatenate([U.q, sh[1].q[None]]), np.concatenate([U.s, sh[1].s[None]]))
    De = QMat(4, Dn.O, Dn.I, Dn.gs, np.concatenate([Dn.q, sh[2].q[None]]), np.concatenate([Dn.s, sh[2].s[None]]))
    ids_e = np.concatenate([ids, np.full((3, 1), 7, np.int32)], axis=1)
    w_e = np.concatenate([w, np.ones((3, 1), np.float32)], axis=1)
    assert np.array_equal(orc.moe_block(Ge, Ue, De, x, ids_e, w_e), with_sh)
    # sampled output rows equal the full evaluation at those rows
    rows = np.array([0, 5, 63, 17], dtype=np.int32)
    assert np.array_equal(orc.moe_block(G, U, Dn, x, ids, w, shared=sh, rows=rows), with_sh[:, rows])


def pin_moe_invalid_ids(orc):
    G, U, Dn, x, ids, w, _ = _moe_case(12, 2, 3, 4, 32, 16)
    bad = ids.copy()
    bad[0, 1] = 4
    bad[1, 2] = -3
    out, inter = orc.moe_block(G, U, Dn, x, bad, w, intermediates=True)
    assert inter["bad"] == 2
    w0 = w.copy()
    w0[0, 1] = 0
    w0[1, 2] = 0
    ids0 = ids.copy()
    ids0[0, 1] = 0
    ids0[1, 2] = 0
    ref = orc.moe_block(G, U, Dn, x, ids0, w0)
    assert np.allclose(out, ref, rtol=0, atol=1e-12 * (1 + np.abs(ref).max()))


def pin_moe_intermediates(orc):
    G, U, Dn, x, ids, w, sh = _moe_case(13, 2, 2, 3, 64, 40, shared=True)
    _, inter = orc.moe_block(G, U, Dn, x, ids, w, shared=sh, intermediates=True)
    for p in range(2 * 2 + 2):
        s = p // 2 if p < 4 else p - 4
        if p < 4:
            e = int(ids.flat[p])
            Gm, Um = G.expert(e), U.expert(e)
        else:
            Gm, Um = sh[0], sh[1]
        g_ref = ref_dense(Gm) @ x[s].astype(np.float64)
        u_ref = ref_dense(Um) @ x[s].astype(np.float64)
        assert np.allclose(inter["g"][p], g_ref, rtol=0, atol=1e-12 * inter["Ag"][p].max())
        assert np.allclose(inter["u"][p], u_ref, rtol=0, atol=1e-12 * inter["Au"][p].max())
        h_ref = g_ref * expit(g_ref) * u_ref
        tol = 1e-12 * (1.1 * np.abs(u_ref) * inter["Ag"][p]
                       + np.abs(g_ref * expit(g_ref)) * inter["Au"][p]) + 1e-15 * np.abs(h_ref)
        assert np.all(np.abs(inter["h"][p] - h_ref) <= tol)


# ---------------------------------------------------------------------------
# Router and exact top-K (colibri-strix commit log, full decode layer commit: router matvec + sigmoid, greedy argmax over sigmoid
# + bias with the CPU's tie order, top-p truncation, norm_topk, routed_scale)
# ---------------------------------------------------------------------------

def ref_router(x, R, bias, K, topp, norm_topk, scale):
    """Independent statement: numpy's f64 matmul, scipy's logistic function, a
    stable sort by (-key, index) for the greedy picks, a cumulative sum for
    top-p."""
    z = np.asarray(x, np.float64) @ np.asarray(R, np.float64).T
    p = expit(z)
    c = p + (0.0 if bias is None else np.asarray(bias, np.float64)[None, :])
    S, E = z.shape
    ids = np.full((S, K), -1, np.int64)
    w = np.zeros((S, K))
    for s in range(S):
        order = sorted(range(E), key=lambda e: (-c[s, e], e))[:K]
        pw = p[s, order]
        keep = K
        if 0.0 < topp < 1.0:
            keep = int(np.argmax(np.cumsum(pw) >= topp * pw.sum())) + 1
        ww = pw[:keep]
        if norm_topk:
            ww = ww / ww.sum()
        ids[s, :keep] = order[:keep]
        w[s, :keep] = ww * scale
    return ids, w, z


def pin_router_bruteforce(orc):
    r = np.random.default_rng(11)
    for (S, D, E, K, topp, norm, scale, bs) in [(3, 40, 10, 4, 0.0, True, 1.0, 0.05),
                                                (5, 17, 33, 8, 0.6, True, 2.5, 0.05),
                                                (2, 64, 8, 8, 0.0, False, 1.0, 0.05),
                                                (4, 9, 16, 3, 0.9, False, 0.5, 0.05),
                                                (8, 20, 24, 6, 0.5, True, 1.0, 0.4)]:
        x = r.standard_normal((S, D)).astype(np.float32)
        R = (r.standard_normal((E, D)) * 0.3).astype(np.float32)
        b = (r.standard_normal(E) * bs).astype(np.float32)
        ids, w, z = orc.moe_router(x, R, b, K, topp, norm, scale)
        ri, rw, rz = ref_router(x, R, b, K, topp, norm, scale)
        A = np.abs(x).astype(np.float64) @ np.abs(R).astype(np.float64).T
        assert np.all(np.abs(z - rz) <= 1e-13 * A), "router logits"
        assert np.array_equal(ids, ri), (ids, ri)
        assert np.allclose(w, rw, rtol=1e-12, atol=0), "router weights"


def pin_router_ties_bias_topp(orc):
    """x = 0: every logit is 0 and every sigmoid 1/2 exactly, so the keys are
    1/2 + bias and the ties are exact."""
    E, K, D = 12, 5, 7
    x = np.zeros((1, D), np.float32)
    R = np.ones((E, D), np.float32)
    # no bias: all keys equal -> picks 0, 1, 2, 3, 4 (smaller index first)
    ids, w, _ = orc.moe_router(x, R, None, K, 0.0, True, 3.0)
    assert ids.tolist() == [[0, 1, 2, 3, 4]] and np.allclose(w, 3.0 / K, rtol=1e-15, atol=0)
    # bias 1 on expert 9, 0.5 on experts 7 and 4 (tied): 9 first, then 4, 7
    b = np.zeros(E, np.float32)
    b[9], b[7], b[4] = 1.0, 0.5, 0.5
    ids, w, _ = orc.moe_router(x, R, b, K, 0.0, False, 1.0)
    assert ids.tolist() == [[9, 4, 7, 0, 1]] and np.all(w == 0.5)  # weights ignore the bias
    # top-p: 4 picks of 1/2 each, total 2; topp = 1/4 -> the first pick alone
    # reaches 1/2 = topp * total exactly and ends the list
    ids, w, _ = orc.moe_router(x, R, None, 4, 0.25, True, 1.0)
    assert ids.tolist() == [[0, -1, -1, -1]] and w.tolist() == [[1.0, 0.0, 0.0, 0.0]]
    ids, w, _ = orc.moe_router(x, R, None, 4, 0.5, False, 2.0)   # 1 = topp * 2 after two picks
    assert ids.tolist() == [[0, 1, -1, -1]] and w.tolist() == [[1.0, 1.0, 0.0, 0.0]]


def pin_router_invariants(orc):
    r = np.random.default_rng(12)
    S, D, E, K = 4, 24, 20, 6
    x = r.standard_normal((S, D)).astype(np.float32)
    R = (r.standard_normal((E, D)) * 0.4).astype(np.float32)
    b = (r.standard_normal(E) * 0.1).astype(np.float32)
    ids, w, z = orc.moe_router(x, R, b, K, 0.0, True, 1.0)
    # relabelling the experts relabels the picks
    perm = r.permutation(E)
    ids2, w2, _ = orc.moe_router(x, R[perm], b[perm], K, 0.0, True, 1.0)
    assert np.array_equal(perm[ids2], ids) and np.allclose(w2, w, rtol=1e-15)
    # norm_topk: weights sum to routed_scale; routed_scale is a plain factor
    ids3, w3, _ = orc.moe_router(x, R, b, K, 0.0, True, 2.75)
    assert np.array_equal(ids3, ids) and np.allclose(w3.sum(axis=1), 2.75, rtol=1e-14)
    assert np.allclose(w3, 2.75 * w, rtol=1e-15)
    # a single-row problem equals the same row inside a batch
    i1, w1, _ = orc.moe_router(x[2:3], R, b, K, 0.0, True, 1.0)
    assert np.array_equal(i1[0], ids[2]) and np.array_equal(w1[0], w[2])
    # without norm_topk the weights are the picks' sigmoids, in pick order
    i4, w4, z4 = orc.moe_router(x, R, b, K, 0.0, False, 1.0)
    assert np.allclose(w4, expit(np.take_along_axis(z4, i4.astype(np.int64), axis=1)), rtol=1e-15)


def pin_rmsnorm_closed_forms(orc):
    """RMSNorm (the post-attention norm of the layer): a hand-worked row,
    constant rows, the weight as a per-feature factor, scale invariance."""
    # x = (3, 4): mean of squares 12.5, so y = (3, 4) / sqrt(12.5)
    y = orc.rmsnorm(np.array([[3.0, 4.0]], np.float32), None, 0.0)
    assert np.allclose(y[0], [0.8485281374238571, 1.1313708498984762], rtol=1e-15, atol=0)
    # constant rows c: y = c / sqrt(c^2 + eps) * w
    D = 96
    r = np.random.default_rng(3)
    w = r.uniform(0.5, 2.0, D).astype(np.float32)
    for c, eps in ((2.0, 1e-6), (-0.5, 0.25), (1e-3, 1e-6)):
        y = orc.rmsnorm(np.full((1, D), c, np.float32), w, eps)
        want = np.float64(np.float32(c)) / np.sqrt(np.float64(np.float32(c)) ** 2 + eps) * w
        assert np.allclose(y[0], want, rtol=1e-14, atol=0), (c, eps)
    # weight = per-feature factor on the unweighted result, rows independent
    x = r.standard_normal((5, D)).astype(np.float32)
    y0 = orc.rmsnorm(x, None, 1e-5)
    yw = orc.rmsnorm(x, w, 1e-5)
    assert np.array_equal(yw, y0 * w.astype(np.float64))
    assert np.array_equal(orc.rmsnorm(x[2:3], None, 1e-5), y0[2:3])
    # eps = 0: mean of squares of the output is 1, and x -> 4x changes nothing
    y1 = orc.rmsnorm(x, None, 0.0)
    assert np.allclose(np.mean(y1 ** 2, axis=1), 1.0, rtol=1e-13)
    assert np.array_equal(orc.rmsnorm(4 * x, None, 0.0), y1)


def pin_moe_layer_zero_norm_weight(orc):
    """The layer with an all-zero norm weight: the normed rows are zero, every
    logit is 0 and every key 1/2 + bias, so the picks are the K largest
    biases (smaller index on ties), the block adds exactly zero and out = h."""
    S, K, E, D, F = 3, 3, 8, 64, 32
    G, U, Dn, x, _, _, sh = _moe_case(41, S, K, E, D, F, shared=True)
    R = np.random.default_rng(5).standard_normal((E, D)).astype(np.float32)
    bias = np.array([0.1, 0.3, 0.3, -0.2, 0.0, 0.3, 0.05, 0.2], np.float32)
    out, st = orc.moe_layer(x, np.zeros(D, np.float32), 1e-6, R, bias, K, 0.0, True, 1.0,
                            G, U, Dn, shared=sh)
    assert np.array_equal(st["xn"], np.zeros((S, D), np.float32))
    assert np.array_equal(st["ids"], np.tile(np.array([1, 2, 5], np.int32), (S, 1)))
    assert np.allclose(st["w"], 1.0 / 3.0, rtol=1e-15)
    assert np.array_equal(out, x.astype(np.float64))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


# ---------------------------------------------------------------------------
# MLA decode attention (colibri-strix commit log, fused decode attention
# commits): RoPE closed forms, the absorbed core against the expanded
# textbook attention, the one-key case, row equivalence, causality.
# ---------------------------------------------------------------------------

def pin_rope_closed_forms(orc):
    # one pair: a rotation of the plane by the position itself
    for pos in (0, 1, 7, 123):
        a, b = 0.3, -1.7
        got = orc.rope(np.array([a, b]), pos, 10000.0)
        c, s = np.cos(pos), np.sin(pos)
        assert np.allclose(got, [a * c - b * s, a * s + b * c], rtol=0, atol=1e-14)
    # second pair of four: frequency theta^(-2/4) = 0.1 for theta = 100
    got = orc.rope(np.array([0.0, 0.0, 1.0, 0.0]), 10, 100.0)
    assert np.allclose(got, [0.0, 0.0, np.cos(1.0), np.sin(1.0)], rtol=0, atol=1e-14)
    # position 0 is the identity, pair norms are kept, rotations compose
    v = np.random.default_rng(5).standard_normal(64)
    assert np.array_equal(orc.rope(v, 0, 10000.0), v)
    r1 = orc.rope(v, 37, 10000.0)
    assert np.allclose(np.hypot(r1[0::2], r1[1::2]), np.hypot(v[0::2], v[1::2]), atol=1e-13)
    assert np.allclose(orc.rope(orc.rope(v, 12, 10000.0), 25, 10000.0), r1, atol=1e-12)


def _mla_case(seed, S, pos_base, D=64, qr=32, L=48, H=3, dn=8, dr=4, dv=6, gs=16, T=None):
    from oracle import MlaWeights
    r = sd.rng(seed)
    T = T or pos_base + S + 3
    mats, shapes, qn, kn, Lc, Rc = sd.gen_mla(r, D, qr, L, H, dn, dr, dv, gs, T, pos_base)
    Q = {k: QMat(4, o, i, gs, *mats[k]) for k, (o, i) in shapes.items()}
    W = MlaWeights(Q["q_a"], qn, Q["q_b"], Q["kv_a"], kn, Q["kv_b"], Q["o_proj"], H, dn, dr, dv,
                   eps=1e-6, theta=50.0)
    x = sd.gen_x(r, S, D)
    return W, x, Lc, Rc


def _naive_mla(W, x, pos_base, Lc0, Rc0):
    """Textbook multi-head attention with K and V expanded from the latent
    cache, every weight from the independent decoder (ref_dense), RoPE and
    RMSNorm written out with numpy."""
    S = x.shape[0]
    H, dn, dr, dv, L = W.H, W.dn, W.dr, W.dv, W.kv_b.I
    Wqa, Wqb, Wkva, Wkvb, Wo = (ref_dense(m) for m in (W.q_a, W.q_b, W.kv_a, W.kv_b, W.o_proj))

    def rms(v, w):
        return v / np.sqrt(np.mean(v * v) + W.eps) * w.astype(np.float64)

    def rot(v, pos):
        f = W.theta ** (-np.arange(0, dr, 2) / dr)
        c, s_ = np.cos(pos * f), np.sin(pos * f)
        o = np.empty_like(v)
        o[0::2] = v[0::2] * c - v[1::2] * s_
        o[1::2] = v[0::2] * s_ + v[1::2] * c
        return o

    xd = x.astype(np.float64)
    Lc, Rc = Lc0.copy(), Rc0.copy()
    for s in range(S):
        ckv = Wkva @ xd[s]
        Lc[pos_base + s] = rms(ckv[:L], W.kv_norm).astype(np.float32)
        Rc[pos_base + s] = rot(ckv[L:], pos_base + s).astype(np.float32)
    blocks = Wkvb.reshape(H, dn + dv, L)
    out, ctx = np.zeros((S, W.o_proj.O)), np.zeros((S, H * dv))
    for s in range(S):
        q = (Wqb @ rms(Wqa @ xd[s], W.q_norm)).reshape(H, dn + dr)
        T = pos_base + s + 1
        Lt, Rt = Lc[:T].astype(np.float64), Rc[:T].astype(np.float64)
        for h in range(H):
            Kh = np.concatenate([Lt @ blocks[h, :dn].T, Rt], axis=1)      # [T][dn+dr]
            Vh = Lt @ blocks[h, dn:].T                                      # [T][dv]
            qh = np.concatenate([q[h, :dn], rot(q[h, dn:], pos_base + s)])
            z = Kh @ qh / np.sqrt(dn + dr)
            p = np.exp(z - z.max())
            p /= p.sum()
            ctx[s, h * dv:(h + 1) * dv] = p @ Vh
        out[s] = Wo @ ctx[s]
    return out, ctx, Lc, Rc


def pin_mla_absorbed_equals_expanded(orc):
    for seed, S, pb in ((1, 1, 0), (2, 3, 5), (3, 4, 9), (4, 2, 1)):
        W, x, Lc, Rc = _mla_case(seed, S, pb)
        out, st, Lc1, Rc1 = orc.mla_decode(W, x, pb, Lc, Rc)
        nout, nctx, nLc, nRc = _naive_mla(W, x, pb, Lc, Rc)
        assert np.array_equal(Lc1[:pb + S], nLc[:pb + S]) or \
            np.allclose(Lc1, nLc, rtol=2 ** -23, atol=0), "latent cache rows"
        assert np.allclose(Rc1, nRc, rtol=2 ** -23, atol=1e-30), "rotary cache rows"
        mag_ctx = np.abs(nctx).max() + 1e-30
        assert np.max(np.abs(st["ctx"] - nctx)) <= 1e-11 * mag_ctx, "ctx"
        mag = np.abs(ref_dense(W.o_proj)) @ np.abs(nctx[0])
        assert np.max(np.abs(out - nout)) <= 1e-11 * (mag.max() + 1e-30), "out"


def pin_mla_one_key(orc):
    """pos_base 0, one row: the single key takes probability 1, so the
    context of head h is its value rows times the new latent row."""
    W, x, Lc, Rc = _mla_case(11, 1, 0)
    out, st, Lc1, _ = orc.mla_decode(W, x, 0, Lc, Rc)
    assert np.all(st["p"][:, :, 0] == 1.0)
    H, dn, dv, L = W.H, W.dn, W.dv, W.kv_b.I
    Wv = ref_dense(W.kv_b).reshape(H, dn + dv, L)[:, dn:]
    want = np.concatenate([Wv[h] @ Lc1[0].astype(np.float64) for h in range(H)])
    assert np.allclose(st["ctx"][0], want, rtol=1e-13, atol=1e-15)


def pin_mla_rows_equal_single_calls(orc):
    """Row s of an S-row call is the single-row call at pos_base + s made
    after the rows before it (the caches carry the earlier rows)."""
    W, x, Lc, Rc = _mla_case(21, 4, 6)
    out, _, Lc4, Rc4 = orc.mla_decode(W, x, 6, Lc, Rc)
    Lcs, Rcs = Lc.copy(), Rc.copy()
    for s in range(4):
        o1, _, Lcs, Rcs = orc.mla_decode(W, x[s:s + 1], 6 + s, Lcs, Rcs)
        assert np.array_equal(o1[0], out[s]), s
    assert np.array_equal(Lcs, Lc4) and np.array_equal(Rcs, Rc4)


def pin_mla_causal(orc):
    """Cache rows past the last position never matter; earlier rows do."""
    W, x, Lc, Rc = _mla_case(31, 3, 4, T=12)
    out, _, _, _ = orc.mla_decode(W, x, 4, Lc, Rc)
    Lf, Rf = Lc.copy(), Rc.copy()
    Lf[7:] = 9.0
    Rf[7:] = -9.0
    out2, _, _, _ = orc.mla_decode(W, x, 4, Lf, Rf)
    assert np.array_equal(out, out2)
    Lp = Lc.copy()
    Lp[2] += 1.0
    out3, _, _, _ = orc.mla_decode(W, x, 4, Lp, Rc)
    assert not np.allclose(out, out3)


ALL_PINS += [pin_rope_closed_forms, pin_mla_absorbed_equals_expanded, pin_mla_one_key,
             pin_mla_rows_equal_single_calls, pin_mla_causal]


# ---------------------------------------------------------------------------
# Full decode layer (colibri-strix commit log, full decode layer commit): the
# composition, checked through cases that reduce it to one half.
# ---------------------------------------------------------------------------

def _layer_case(seed, S, pb, D=64, E=6, F=32, K=2, gs=16):
    W, x, Lc, Rc = _mla_case(seed, S, pb, D=D, gs=gs)
    r = sd.rng(seed + 1000)
    G, U, Dn, _, _, _, sh = _moe_case(seed + 2000, S, K, E, D, F, gs=gs, shared=True)
    R = r.standard_normal((E, D)).astype(np.float32)
    bias = r.uniform(-0.1, 0.1, E).astype(np.float32)
    in_ln = r.uniform(0.5, 1.5, D).astype(np.float32)
    post_ln = r.uniform(0.5, 1.5, D).astype(np.float32)
    return W, x, Lc, Rc, G, U, Dn, sh, R, bias, in_ln, post_ln


def pin_layer_reduces_to_its_halves(orc):
    from oracle import QMat as QM
    W, x, Lc, Rc, G, U, Dn, sh, R, bias, in_ln, post_ln = _layer_case(41, 3, 4)
    args = (R, bias, 2, 0.0, True, 1.0, G, U, Dn)
    # attention output projection zero: h = x, the layer is the expert half on x
    Wz = W.__class__(**{**W.__dict__, "o_proj": QM(4, W.o_proj.O, W.o_proj.I, W.o_proj.gs,
                                                  W.o_proj.q, np.zeros_like(W.o_proj.s))})
    out, it, _, _ = orc.layer_decode(x, in_ln, 1e-6, Wz, 4, Lc, Rc, post_ln, *args, shared=sh)
    assert np.array_equal(it["h"], x)
    ref, _ = orc.moe_layer(x, post_ln, 1e-6, *args, shared=sh)
    assert np.array_equal(out, ref)
    # every down projection zero: the layer is x + attention(in_ln(x))
    Dz = QM(4, Dn.O, Dn.I, Dn.gs, Dn.q, np.zeros_like(Dn.s))
    shz = (sh[0], sh[1], QM(4, sh[2].O, sh[2].I, sh[2].gs, sh[2].q, np.zeros_like(sh[2].s)))
    out, it, Lc1, _ = orc.layer_decode(x, in_ln, 1e-6, W, 4, Lc, Rc, post_ln, R, bias, 2, 0.0,
                                       True, 1.0, G, U, Dz, shared=shz)
    xn = orc.rmsnorm(x, in_ln, 1e-6).astype(np.float32)
    a, _, Lc2, _ = orc.mla_decode(W, xn, 4, Lc, Rc)
    assert np.array_equal(out, (x.astype(np.float64) + a).astype(np.float32).astype(np.float64))
    assert np.array_equal(Lc1, Lc2)


ALL_PINS += [pin_layer_reduces_to_its_halves]
