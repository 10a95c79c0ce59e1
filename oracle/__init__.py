"""CPU oracle for the colibri quantized matmul and MoE block -- TEST INFRASTRUCTURE.

The arithmetic lives in ``coli_oracle.c`` (plain C, f64).  This module only
compiles it with gcc and marshals numpy arrays through ctypes.  It shares no
code with the GPU library; only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it.

Every function here states the passage it follows in the C source; the
readings taken where the pages are silent are listed there as well.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "coli_oracle.c")
LIB = os.path.join(HERE, "libcoli_oracle.so")

CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
          "-ffp-contract=off", "-fopenmp", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc into a shared library; returns its path."""
    cmd = ["gcc", *CFLAGS, *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class OracleQT(C.Structure):
    """Mirror of the oracle's own ``oracle_qt`` record (one expert stack)."""
    _fields_ = [("fmt", C.c_int32), ("O", C.c_int32), ("I", C.c_int32),
                ("gs", C.c_int32), ("ng", C.c_int32), ("pad_", C.c_int32),
                ("q_stride", C.c_int64), ("s_stride", C.c_int64),
                ("q", C.c_void_p), ("s", C.c_void_p)]


def row_bytes(fmt: int, I: int) -> int:
    return {1: I, 2: (I + 1) // 2, 4: (I + 1) // 2, 3: (I + 3) // 4}[fmt]


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


@dataclass
class QMat:
    """A quantized matrix (or stack of n matrices) held in host memory.

    q: uint8 [n][O][row_bytes] (int8 bytes for fmt 1 are stored as uint8)
    s: float32 [n][O][ng] for fmt 4, [n][O] for fmt 1-3.
    """
    fmt: int
    O: int
    I: int
    gs: int
    q: np.ndarray
    s: np.ndarray

    @property
    def ng(self) -> int:
        return -(-self.I // self.gs) if self.fmt == 4 else 1

    @property
    def n(self) -> int:
        return self.q.shape[0] if self.q.ndim == 3 else 1

    def qt(self) -> OracleQT:
        q = np.ascontiguousarray(self.q.view(np.uint8))
        s = np.ascontiguousarray(self.s, dtype=np.float32)
        self._keep = (q, s)
        return OracleQT(self.fmt, self.O, self.I, self.gs if self.fmt == 4 else 0,
                        self.ng, 0, self.O * row_bytes(self.fmt, self.I),
                        self.O * self.ng, q.ctypes.data, s.ctypes.data)

    def expert(self, e: int) -> "QMat":
        if self.q.ndim == 2:
            assert e == 0
            return self
        return QMat(self.fmt, self.O, self.I, self.gs, self.q[e], self.s[e])


class Oracle:
    """ctypes front end of one compiled oracle library."""

    def __init__(self, lib_path: str | None = None, nthreads: int = 1):
        path = lib_path or LIB
        if lib_path is None and (not os.path.exists(path)
                                 or os.path.getmtime(path) < os.path.getmtime(SRC)):
            build()
        self.lib = C.CDLL(path)
        self.nthreads = nthreads
        L = self.lib
        i64, i32, vp, dbl = C.c_int64, C.c_int, C.c_void_p, C.c_double
        L.oracle_row_bytes.restype = i64
        L.oracle_row_bytes.argtypes = [i32, i64]
        L.oracle_shape_ok.restype = i32
        L.oracle_shape_ok.argtypes = [i32, i64, i64, i64, i64]
        L.oracle_decode_codes.argtypes = [i32, i64, i64, vp, vp]
        L.oracle_dequant_f32.argtypes = [i32, i64, i64, i64, i64, vp, vp, vp]
        L.oracle_dequant_f64.argtypes = [i32, i64, i64, i64, i64, vp, vp, vp]
        L.oracle_qmatmul.argtypes = [i32, i64, i64, i64, i64, vp, vp, i64, vp, vp, vp, i32]
        L.oracle_qmatmul_f64in.argtypes = [i32, i64, i64, i64, i64, vp, vp, i64, vp, vp, vp, i32]
        L.oracle_silu.restype = dbl
        L.oracle_silu.argtypes = [dbl]
        L.oracle_moe_route.restype = i64
        L.oracle_moe_route.argtypes = [vp, i64, i64, i64, vp, vp, vp]
        L.oracle_moe_router.argtypes = [vp, i64, i64, vp, vp, i64, i64, dbl, i32, dbl, vp, vp, vp]
        L.oracle_rmsnorm.argtypes = [vp, i64, i64, vp, dbl, vp]
        QP = C.POINTER(OracleQT)
        L.oracle_rope.argtypes = [vp, i64, i64, dbl, vp]
        L.oracle_mla_qabs.argtypes = [QP, i64, i64, i64, i64, vp, i64, vp, vp]
        L.oracle_mla_scores.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, dbl, vp, vp]
        L.oracle_mla_softmax.argtypes = [vp, i64, i64, i64, i64, vp]
        L.oracle_mla_clat.argtypes = [vp, vp, i64, i64, i64, i64, i64, vp, vp]
        L.oracle_mla_ctx.argtypes = [QP, i64, i64, i64, vp, i64, vp, vp]
        L.oracle_mla_decode.argtypes = [QP, vp, QP, QP, vp, QP, QP, i64, i64, i64, i64, dbl, dbl,
                                        vp, i64, i64, vp, vp, vp, C.POINTER(C.c_void_p), i32]
        L.oracle_moe_block.restype = i64
        L.oracle_moe_block.argtypes = [C.POINTER(OracleQT)] * 3 + [
            i64, vp, i64, vp, vp, i64] + [C.POINTER(OracleQT)] * 3 + [
            i64, vp, vp, vp, vp, vp, vp, vp, i32]

    # --- formats -----------------------------------------------------------
    def row_bytes(self, fmt: int, I: int) -> int:
        return int(self.lib.oracle_row_bytes(fmt, I))

    def shape_ok(self, fmt, O, I, gs, ng) -> bool:
        return bool(self.lib.oracle_shape_ok(fmt, O, I, gs, ng))

    def decode_codes(self, W: QMat) -> np.ndarray:
        q = np.ascontiguousarray(W.q.view(np.uint8))
        v = np.zeros((W.O, W.I), dtype=np.int32)
        self.lib.oracle_decode_codes(W.fmt, W.O, W.I, _p(q), _p(v))
        return v

    def dequant_f32(self, W: QMat) -> np.ndarray:
        q = np.ascontiguousarray(W.q.view(np.uint8))
        s = np.ascontiguousarray(W.s, dtype=np.float32)
        w = np.zeros((W.O, W.I), dtype=np.float32)
        self.lib.oracle_dequant_f32(W.fmt, W.O, W.I, W.gs, W.ng, _p(q), _p(s), _p(w))
        return w

    def dequant_f64(self, W: QMat) -> np.ndarray:
        q = np.ascontiguousarray(W.q.view(np.uint8))
        s = np.ascontiguousarray(W.s, dtype=np.float32)
        w = np.zeros((W.O, W.I), dtype=np.float64)
        self.lib.oracle_dequant_f64(W.fmt, W.O, W.I, W.gs, W.ng, _p(q), _p(s), _p(w))
        return w

    # --- matmul --------------------------------------------------------------
    def qmatmul(self, W: QMat, x: np.ndarray):
        """y[s][o] = sum_i w(o,i) x[s][i] in f64; returns (y, A) with A the
        magnitude sum_i |w||x| per output."""
        x = np.ascontiguousarray(np.atleast_2d(x))
        S = x.shape[0]
        q = np.ascontiguousarray(W.q.view(np.uint8))
        s = np.ascontiguousarray(W.s, dtype=np.float32)
        y = np.zeros((S, W.O), dtype=np.float64)
        A = np.zeros((S, W.O), dtype=np.float64)
        if x.dtype == np.float64:
            fn = self.lib.oracle_qmatmul_f64in
        else:
            assert x.dtype == np.float32
            fn = self.lib.oracle_qmatmul
        fn(W.fmt, W.O, W.I, W.gs, W.ng, _p(q), _p(s), S, _p(x), _p(y), _p(A),
           self.nthreads)
        return y, A

    # --- MoE -----------------------------------------------------------------
    def silu(self, z: float) -> float:
        return float(self.lib.oracle_silu(float(z)))

    def moe_route(self, ids: np.ndarray, E: int):
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        S, K = ids.shape
        counts = np.zeros(E, dtype=np.int32)
        offsets = np.zeros(E + 1, dtype=np.int32)
        perm = np.full(S * K, -1, dtype=np.int32)
        bad = self.lib.oracle_moe_route(_p(ids), S, K, E, _p(counts), _p(offsets), _p(perm))
        return counts, offsets, perm, int(bad)

    def moe_router(self, x: np.ndarray, R: np.ndarray, bias, K: int, topp: float = 0.0,
                   norm_topk: bool = True, routed_scale: float = 1.0):
        """Router logits, sigmoid, greedy top-K over sigmoid + bias (ties to the
        smaller index), top-p, norm_topk, routed_scale (coli_oracle.c states
        the readings).  Returns ids [S][K] int32, w [S][K] f64, z [S][E] f64."""
        x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
        R = np.ascontiguousarray(R, dtype=np.float32)
        S, D = x.shape
        E = R.shape[0]
        assert R.shape[1] == D and 1 <= K <= E
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        ids = np.zeros((S, K), dtype=np.int32)
        w = np.zeros((S, K), dtype=np.float64)
        z = np.zeros((S, E), dtype=np.float64)
        self.lib.oracle_moe_router(_p(x), S, D, _p(R), _p(b), E, K, float(topp),
                                   int(bool(norm_topk)), float(routed_scale), _p(ids), _p(w), _p(z))
        return ids, w, z

    def rmsnorm(self, x: np.ndarray, w, eps: float) -> np.ndarray:
        """Per-row RMSNorm with a per-feature weight (coli_oracle.c states the
        reading).  Returns y [S][D] f64."""
        x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
        S, D = x.shape
        wf = None if w is None else np.ascontiguousarray(w, dtype=np.float32)
        assert wf is None or wf.shape == (D,)
        y = np.zeros((S, D), dtype=np.float64)
        self.lib.oracle_rmsnorm(_p(x), S, D, _p(wf), float(eps), _p(y))
        return y

    def moe_layer(self, h: np.ndarray, ln_w, eps: float, R: np.ndarray, bias, K: int,
                  topp: float, norm_topk: bool, routed_scale: float, gate: QMat, up: QMat,
                  down: QMat, shared=None):
        """The expert half of a decode layer (colibri-strix commit log, full decode layer commit): xn = RMSNorm(h), stored as
        f32; router and exact top-K on xn; the expert block on xn with the
        routed weights as f32; out = h + block.  Each step is one of the
        functions above, called in that order.  Returns out [S][D] f64 and a
        dict with xn (f32), ids, w (f64) and the block output y (f64)."""
        h = np.ascontiguousarray(np.atleast_2d(h), dtype=np.float32)
        xn = self.rmsnorm(h, ln_w, eps).astype(np.float32)
        ids, w, _ = self.moe_router(xn, R, bias, K, topp, norm_topk, routed_scale)
        y = self.moe_block(gate, up, down, xn, ids, w.astype(np.float32), shared=shared)
        return h.astype(np.float64) + y, {"xn": xn, "ids": ids, "w": w, "y": y}

    def moe_block(self, gate: QMat, up: QMat, down: QMat, x: np.ndarray,
                  ids: np.ndarray, w: np.ndarray, shared=None, rows=None,
                  intermediates: bool = False):
        """Returns out [S][D or len(rows)] f64 (and a dict of per-pair g, u, h,
        Ag, Au [P][F] when intermediates=True)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        w = np.ascontiguousarray(w, dtype=np.float32)
        S, K = ids.shape
        E = gate.n
        F = gate.O
        qg, qu, qd = gate.qt(), up.qt(), down.qt()
        sh = [None, None, None]
        if shared is not None:
            sh = [C.pointer(m.qt()) for m in shared]
        P = S * K + (S if shared is not None else 0)
        nout = len(rows) if rows is not None else down.O
        rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
        out = np.zeros((S, nout), dtype=np.float64)
        inter = {k: np.zeros((P, F), dtype=np.float64) for k in ("g", "u", "h", "Ag", "Au")} \
            if intermediates else {}
        bad = self.lib.oracle_moe_block(
            C.pointer(qg), C.pointer(qu), C.pointer(qd), E, _p(x), S, _p(ids), _p(w), K,
            sh[0], sh[1], sh[2], nout if rows is not None else 0, _p(rows_arr), _p(out),
            *(_p(inter.get(k)) for k in ("g", "u", "h", "Ag", "Au")), self.nthreads)
        self._keep = (shared,)
        if intermediates:
            inter["bad"] = int(bad)
            return out, inter
        return out


    # --- MLA decode attention (coli_oracle.c states the passages and readings)
    def rope(self, v: np.ndarray, pos: int, theta: float) -> np.ndarray:
        """RoPE of rotary vectors v [..., d_rope] (f64) at one position."""
        v = np.ascontiguousarray(v, dtype=np.float64)
        dr = v.shape[-1]
        flat = v.reshape(-1, dr)
        out = np.zeros_like(flat)
        for i in range(flat.shape[0]):
            self.lib.oracle_rope(_p(flat[i]), dr // 2, int(pos), float(theta), _p(out[i]))
        return out.reshape(v.shape)

    def mla_qabs(self, kv_b: QMat, H, dn, dr, dv, q):
        """(qabs [S][H][L], A) from q [S][H*(dn+dr)] (key absorption)."""
        q = np.ascontiguousarray(np.atleast_2d(q), dtype=np.float64)
        S, L = q.shape[0], kv_b.I
        qa = np.zeros((S, H, L))
        A = np.zeros((S, H, L))
        t = kv_b.qt()
        self.lib.oracle_mla_qabs(C.pointer(t), H, dn, dr, dv, _p(q), S, _p(qa), _p(A))
        return qa, A

    def mla_scores(self, qabs, qpe, Lc, Rc, pos_base, scale):
        """(scores [S][H][pos_base+S], A): scaled q.k over t <= pos_base+s."""
        qabs = np.ascontiguousarray(qabs, dtype=np.float64)
        qpe = np.ascontiguousarray(qpe, dtype=np.float64)
        Lc = np.ascontiguousarray(Lc, dtype=np.float32)
        Rc = np.ascontiguousarray(Rc, dtype=np.float32)
        S, H, L = qabs.shape
        dr = qpe.shape[2]
        Ts = pos_base + S
        sc = np.zeros((S, H, Ts))
        A = np.zeros((S, H, Ts))
        self.lib.oracle_mla_scores(_p(qabs), _p(qpe), _p(Lc), _p(Rc), S, H, L, dr, pos_base, Ts,
                                   float(scale), _p(sc), _p(A))
        return sc, A

    def mla_softmax(self, scores, pos_base):
        scores = np.ascontiguousarray(scores, dtype=np.float64)
        S, H, Ts = scores.shape
        p = np.zeros_like(scores)
        self.lib.oracle_mla_softmax(_p(scores), S, H, pos_base, Ts, _p(p))
        return p

    def mla_clat(self, p, Lc, pos_base):
        p = np.ascontiguousarray(p, dtype=np.float64)
        Lc = np.ascontiguousarray(Lc, dtype=np.float32)
        S, H, Ts = p.shape
        L = Lc.shape[1]
        cl = np.zeros((S, H, L))
        A = np.zeros((S, H, L))
        self.lib.oracle_mla_clat(_p(p), _p(Lc), S, H, L, pos_base, Ts, _p(cl), _p(A))
        return cl, A

    def mla_ctx(self, kv_b: QMat, H, dn, dv, clat):
        clat = np.ascontiguousarray(clat, dtype=np.float64)
        S = clat.shape[0]
        ctx = np.zeros((S, H * dv))
        A = np.zeros((S, H * dv))
        t = kv_b.qt()
        self.lib.oracle_mla_ctx(C.pointer(t), H, dn, dv, _p(clat), S, _p(ctx), _p(A))
        return ctx, A

    def mla_decode(self, W: "MlaWeights", x, pos_base: int, Lc, Rc):
        """The decode attention of S rows at positions pos_base.. (every step
        in order, f64).  Lc [T][L] / Rc [T][dr] f32 are copied; the copies get
        this call's rows.  Returns out [S][D] f64, the stages (dict) and the
        new caches."""
        x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
        S = x.shape[0]
        H, dn, dr, dv = W.H, W.dn, W.dr, W.dv
        L, qr = W.kv_b.I, W.q_a.O
        Lc = np.array(Lc, dtype=np.float32, order="C", copy=True)
        Rc = np.array(Rc, dtype=np.float32, order="C", copy=True)
        assert Lc.shape[0] >= pos_base + S and Rc.shape[0] >= pos_base + S
        Ts = pos_base + S
        shapes = [(S, qr), (S, L + dr), (S, qr), (S, H * (dn + dr)), (S, H, L), (S, H, dr),
                  (S, H, Ts), (S, H, Ts), (S, H, L), (S, H * dv)]
        names = ["cq_raw", "ckv_raw", "cq", "q", "qabs", "qpe", "scores", "p", "clat", "ctx"]
        st = {n: np.zeros(sh) for n, sh in zip(names, shapes)}
        ptrs = (C.c_void_p * 10)(*[st[n].ctypes.data for n in names])
        out = np.zeros((S, W.o_proj.O))
        ts = [m.qt() for m in (W.q_a, W.q_b, W.kv_a, W.kv_b, W.o_proj)]
        qn = None if W.q_norm is None else np.ascontiguousarray(W.q_norm, dtype=np.float32)
        kn = None if W.kv_norm is None else np.ascontiguousarray(W.kv_norm, dtype=np.float32)
        self.lib.oracle_mla_decode(C.pointer(ts[0]), _p(qn), C.pointer(ts[1]), C.pointer(ts[2]),
                                   _p(kn), C.pointer(ts[3]), C.pointer(ts[4]), H, dn, dr, dv,
                                   float(W.eps), float(W.theta), _p(x), S, pos_base, _p(Lc),
                                   _p(Rc), _p(out), ptrs, self.nthreads)
        self._keep = ts
        return out, st, Lc, Rc


def _layer_decode(self, x, in_ln, eps, attn: "MlaWeights", pos_base, Lc, Rc, post_ln, R, bias, K,
                  topp, norm_topk, routed_scale, gate, up, down, shared=None):
    """One decode layer (colibri-strix commit log, full decode layer commit:
    in_ln RMSNorm -> fused attention -> residual add -> post_ln RMSNorm ->
    shared expert, router with the exact top-K, routed experts -> residual
    add), each step one of the functions above, called in that order; the
    values handed from one step to the next are f32 (as stored):
      xn = rmsnorm(x, in_ln);  a = mla_decode(xn);  h = f32(x + a);
      out = moe_layer(h, post_ln)                       (its own residual add)
    Returns out [S][D] f64, a dict of the intermediates, and the new caches."""
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
    xn = self.rmsnorm(x, in_ln, eps).astype(np.float32)
    a, st, Lc1, Rc1 = self.mla_decode(attn, xn, pos_base, Lc, Rc)
    h = (x.astype(np.float64) + a).astype(np.float32)
    out, inter = self.moe_layer(h, post_ln, eps, R, bias, K, topp, norm_topk, routed_scale,
                                gate, up, down, shared=shared)
    inter.update({"xn": xn, "attn": a, "h": h, "attn_stages": st, "xn_moe": inter["xn"]})
    return out, inter, Lc1, Rc1


Oracle.layer_decode = _layer_decode


@dataclass
class MlaWeights:
    """One decode attention layer's weights and hyper-parameters (the
    readings in coli_oracle.c): q_a [qr][D], q_b [H(dn+dr)][qr], kv_a
    [L+dr][D], kv_b [H(dn+dv)][L], o_proj [D][H dv]; q_norm [qr] and
    kv_norm [L] f32 (None: ones)."""
    q_a: QMat
    q_norm: np.ndarray | None
    q_b: QMat
    kv_a: QMat
    kv_norm: np.ndarray | None
    kv_b: QMat
    o_proj: QMat
    H: int
    dn: int
    dr: int
    dv: int
    eps: float = 1e-6
    theta: float = 10000.0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.dn + self.dr))


_default: Oracle | None = None


def get(nthreads: int = 1) -> Oracle:
    """The default oracle instance (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    _default.nthreads = nthreads
    return _default
