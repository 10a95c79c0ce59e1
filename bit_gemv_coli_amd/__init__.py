"""Python binding of libcoli -- the MI355X (gfx950) quantized-weight matmul
and MoE-block library.

Argument marshalling only: every function here forwards to the C entry point
of the same name in ``libcoli.so`` (declared in ``include/coli.h``).  Device
memory and streams come from PyTorch: pass tensors (their ``data_ptr()`` is
used) or raw integer device pointers.  There is no CPU fallback: if the
library is missing, importing a compute function raises.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcoli.so")

COLI_OK, COLI_DECLINED, COLI_HIP_ERROR = 1, 0, -1


class coli_mla_layer(C.Structure):
    """Mirror of ``coli_mla_layer`` in include/coli.h."""
    _fields_ = [("q_a", C.c_void_p), ("q_b", C.c_void_p), ("kv_a", C.c_void_p),
                ("kv_b", C.c_void_p), ("o_proj", C.c_void_p), ("q_norm", C.c_void_p),
                ("kv_norm", C.c_void_p), ("H", C.c_int32), ("d_nope", C.c_int32),
                ("d_rope", C.c_int32), ("d_v", C.c_int32), ("eps", C.c_float),
                ("rope_theta", C.c_float)]


class coli_qtensor(C.Structure):
    """Mirror of ``coli_qtensor`` in include/coli.h."""
    _fields_ = [("fmt", C.c_int32), ("n", C.c_int32), ("O", C.c_int32), ("I", C.c_int32),
                ("gs", C.c_int32), ("ng", C.c_int32), ("row_bytes", C.c_int64),
                ("q_stride", C.c_int64), ("s_stride", C.c_int64), ("q", C.c_void_p),
                ("s", C.c_void_p), ("magic", C.c_uint32), ("flags", C.c_uint32),
                ("pk", C.c_void_p), ("pk_stride", C.c_int64), ("pk_scale_off", C.c_int64)]


_lib = None


class ColiError(RuntimeError):
    pass


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ColiError(f"libcoli.so is not built ({LIB_PATH}); run "
                        "`python -m bit_gemv_coli_amd.build` (hipcc, gfx950)")
    try:  # bind to the HIP runtime torch already loaded (one runtime per process)
        import torch  # noqa: F401
    except ImportError:
        pass
    L = C.CDLL(LIB_PATH)
    vp, i32, i64, sz = C.c_void_p, C.c_int, C.c_int64, C.c_size_t
    QP = C.POINTER(coli_qtensor)
    sig = {
        "coli_tensor_upload": (i32, [QP, i32, i32, i32, i32, i32, i32, vp, vp]),
        "coli_qmatmul": (i32, [QP, vp, vp, i32, vp]),
        "coli_qmatmul_ws": (i32, [QP, vp, vp, i32, vp, sz, vp]),
        "coli_qmatmul_workspace_bytes": (sz, [QP, i32]),
        "coli_qmatmul_group": (i32, [i32, vp, vp, vp, i32, vp]),
        "coli_moe_block_two_phase_workspace_bytes": (sz, [i32, i32, i32, i32, i32, i32]),
        "coli_moe_block_begin": (i32, [QP, QP, QP, vp, i32, vp, vp, i32, vp, QP, QP, QP, vp, vp, sz, vp]),
        "coli_moe_block_end": (i32, [QP, QP, QP, vp, i32, vp, i32, i32, vp, vp, sz, vp]),
        "coli_packed_bytes": (sz, [i32, i32, i32, i32, i32]),
        "coli_tensor_pack": (i32, [QP, vp, sz, vp]),
        "coli_gemv_max_rows": (i32, []),
        "coli_set_gemv_max_rows": (i32, [i32]),
        "coli_set_decode_kernel": (i32, [i32]),
        "coli_dequantize": (i32, [QP, vp, vp]),
        "coli_moe_route": (i32, [vp, i32, i32, i32, vp, vp, vp, vp, vp]),
        "coli_moe_block": (i32, [QP, QP, QP, vp, i32, vp, vp, i32, QP, QP, QP, vp, vp, sz, vp]),
        "coli_moe_hidden": (i32, [QP, QP, vp, i32, vp, i32, QP, QP, vp, vp, sz, vp]),
        "coli_moe_workspace_bytes": (sz, [i32, i32, i32, i32, i32, i32]),
        "coli_moe_block_noalloc": (i32, [QP, QP, QP, vp, i32, vp, vp, i32, QP, QP, QP, vp, vp]),
        "coli_last_reason": (C.c_char_p, []),
        "coli_last_error": (C.c_char_p, []),
        "coli_stats": (None, [vp, vp, vp]),
        "coli_set_fail_after": (None, [i64]),
        "coli_prof_enable": (None, [i32]),
        "coli_prof_reset": (None, []),
        "coli_prof_read": (i64, [C.c_char_p, vp]),
        "coli_prof_tag": (C.c_char_p, [i32]),
        "coli_version": (C.c_char_p, []),
        "coli_moe_router_workspace_bytes": (sz, [i32, i32]),
        "coli_moe_router": (i32, [vp, i32, i32, vp, vp, i32, i32, C.c_float, i32, C.c_float, vp, vp,
                                  vp, sz, vp]),
        "coli_rmsnorm": (i32, [vp, i32, i32, vp, C.c_float, vp, vp]),
        "coli_moe_layer_workspace_bytes": (sz, [i32, i32, i32, i32, i32, i32]),
        "coli_moe_layer": (i32, [QP, QP, QP, vp, i32, vp, C.c_float, vp, vp, i32, C.c_float, i32,
                                 C.c_float, QP, QP, QP, vp, vp, sz, vp]),
        "coli_probe_read": (i32, [vp, sz, vp, vp]),
        "coli_probe_mfma": (i32, [i32, i32, vp, vp]),
        "coli_probe_launch": (i32, [i32, vp, vp]),
        "coli_mla_workspace_bytes": (sz, [C.POINTER(coli_mla_layer), i32, i32]),
        "coli_mla_workspace_layout": (sz, [C.POINTER(coli_mla_layer), i32, i32,
                                           C.POINTER(C.c_size_t)]),
        "coli_mla_decode": (i32, [C.POINTER(coli_mla_layer), vp, i32, i32, vp, vp, i32, vp, vp, sz,
                                  vp]),
        "coli_layer_decode_workspace_bytes": (sz, [C.POINTER(coli_mla_layer), QP, i32, i32, i32,
                                                   i32]),
        "coli_layer_decode_workspace_layout": (sz, [C.POINTER(coli_mla_layer), QP, i32, i32, i32,
                                                    i32, C.POINTER(C.c_size_t)]),
        "coli_layer_decode": (i32, [C.POINTER(coli_mla_layer), vp, QP, QP, QP, vp, vp, vp, i32,
                                    C.c_float, i32, C.c_float, QP, QP, QP, C.c_float, vp, i32, i32,
                                    vp, vp, i32, vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def exported_symbols():
    """Names the binding expects libcoli to export."""
    return ["coli_tensor_upload", "coli_packed_bytes", "coli_tensor_pack", "coli_qmatmul",
            "coli_qmatmul_ws", "coli_qmatmul_workspace_bytes",
            "coli_qmatmul_group", "coli_gemv_max_rows", "coli_set_gemv_max_rows",
            "coli_moe_block_two_phase_workspace_bytes", "coli_moe_block_begin",
            "coli_moe_block_end",
            "coli_set_decode_kernel",
            "coli_dequantize", "coli_moe_route", "coli_moe_block", "coli_moe_hidden",
            "coli_moe_workspace_bytes", "coli_moe_block_noalloc", "coli_last_reason", "coli_last_error", "coli_stats",
            "coli_set_fail_after", "coli_prof_enable", "coli_prof_reset", "coli_prof_read",
            "coli_prof_tag", "coli_version", "coli_probe_read", "coli_probe_mfma", "coli_probe_launch",
            "coli_moe_router_workspace_bytes", "coli_moe_router", "coli_rmsnorm",
            "coli_moe_layer_workspace_bytes", "coli_moe_layer", "coli_mla_workspace_bytes",
            "coli_mla_workspace_layout", "coli_mla_decode", "coli_layer_decode_workspace_bytes",
            "coli_layer_decode_workspace_layout", "coli_layer_decode"]


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _qp(t):
    if t is None:
        return None
    return C.byref(t.desc if isinstance(t, QTensor) else t)


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def coli_tensor_upload(desc: coli_qtensor, fmt, n, O, I, gs, ng, q, s) -> int:
    return _load().coli_tensor_upload(C.byref(desc), fmt, n, O, I, gs, ng, _ptr(q), _ptr(s))


def coli_packed_bytes(fmt, n, O, I, gs) -> int:
    return _load().coli_packed_bytes(fmt, n, O, I, gs)


def coli_tensor_pack(W, packed, nbytes, stream=None) -> int:
    return _load().coli_tensor_pack(_qp(W), _ptr(packed), nbytes, _stream(stream))


def coli_qmatmul(W, x, y, S, stream=None) -> int:
    return _load().coli_qmatmul(_qp(W), _ptr(x), _ptr(y), S, _stream(stream))


def coli_qmatmul_ws(W, x, y, S, workspace, ws_bytes, stream=None) -> int:
    return _load().coli_qmatmul_ws(_qp(W), _ptr(x), _ptr(y), S, _ptr(workspace), ws_bytes,
                                   _stream(stream))


def coli_qmatmul_workspace_bytes(W, S) -> int:
    return _load().coli_qmatmul_workspace_bytes(_qp(W), S)


COLI_GROUP_MAX = 8


def coli_moe_block_two_phase_workspace_bytes(E, S, K, F, D, has_shared) -> int:
    return _load().coli_moe_block_two_phase_workspace_bytes(E, S, K, F, D, int(bool(has_shared)))


def coli_moe_block_begin(gate, up, down, x, S, ids, w, K, late, sh_gate, sh_up, sh_down, out,
                         workspace, ws_bytes, stream=None) -> int:
    return _load().coli_moe_block_begin(_qp(gate), _qp(up), _qp(down), _ptr(x), S, _ptr(ids),
                                        _ptr(w), K, _ptr(late), _qp(sh_gate), _qp(sh_up),
                                        _qp(sh_down), _ptr(out), _ptr(workspace), ws_bytes,
                                        _stream(stream))


def coli_moe_block_end(gate, up, down, x, S, w, K, has_shared, out, workspace, ws_bytes,
                       stream=None) -> int:
    return _load().coli_moe_block_end(_qp(gate), _qp(up), _qp(down), _ptr(x), S, _ptr(w), K,
                                      int(bool(has_shared)), _ptr(out), _ptr(workspace), ws_bytes,
                                      _stream(stream))


def coli_qmatmul_group(Ws, xs, ys, S, stream=None) -> int:
    """y[g] = W[g] x[g] for the members of one group (lists of equal length)."""
    n = len(Ws)
    if not (len(xs) == n and len(ys) == n):
        raise ValueError("coli_qmatmul_group: W, x and y lists differ in length")
    descs = (C.POINTER(coli_qtensor) * max(n, 1))(
        *[C.pointer(w.desc if isinstance(w, QTensor) else w) for w in Ws])
    xp = (C.c_void_p * max(n, 1))(*[_ptr(x) for x in xs])
    yp = (C.c_void_p * max(n, 1))(*[_ptr(y) for y in ys])
    return _load().coli_qmatmul_group(n, descs, xp, yp, S, _stream(stream))


def coli_gemv_max_rows() -> int:
    return _load().coli_gemv_max_rows()


def coli_set_gemv_max_rows(s: int) -> int:
    return _load().coli_set_gemv_max_rows(s)


def coli_set_decode_kernel(mode: int) -> int:
    return _load().coli_set_decode_kernel(mode)


def coli_dequantize(W, w_out, stream=None) -> int:
    return _load().coli_dequantize(_qp(W), _ptr(w_out), _stream(stream))


def coli_moe_route(ids, S, K, E, counts, offsets, perm, n_bad, stream=None) -> int:
    return _load().coli_moe_route(_ptr(ids), S, K, E, _ptr(counts), _ptr(offsets), _ptr(perm),
                                  _ptr(n_bad), _stream(stream))


def coli_moe_block(gate, up, down, x, S, ids, w, K, sh_gate, sh_up, sh_down, out, workspace,
                   ws_bytes, stream=None) -> int:
    return _load().coli_moe_block(_qp(gate), _qp(up), _qp(down), _ptr(x), S, _ptr(ids), _ptr(w),
                                  K, _qp(sh_gate), _qp(sh_up), _qp(sh_down), _ptr(out),
                                  _ptr(workspace), ws_bytes, _stream(stream))


COLI_NOALLOC_SCRATCH_BYTES = 8 << 20


def coli_moe_block_noalloc(gate, up, down, x, S, ids, w, K, sh_gate, sh_up, sh_down, out,
                           stream=None) -> int:
    return _load().coli_moe_block_noalloc(_qp(gate), _qp(up), _qp(down), _ptr(x), S, _ptr(ids),
                                          _ptr(w), K, _qp(sh_gate), _qp(sh_up), _qp(sh_down),
                                          _ptr(out), _stream(stream))


def coli_moe_hidden(gate, up, x, S, ids, K, sh_gate, sh_up, h_out, workspace, ws_bytes,
                    stream=None) -> int:
    return _load().coli_moe_hidden(_qp(gate), _qp(up), _ptr(x), S, _ptr(ids), K, _qp(sh_gate),
                                   _qp(sh_up), _ptr(h_out), _ptr(workspace), ws_bytes,
                                   _stream(stream))


def coli_moe_workspace_bytes(E, S, K, F, Dm, has_shared) -> int:
    return _load().coli_moe_workspace_bytes(E, S, K, F, Dm, int(bool(has_shared)))


def coli_last_reason() -> str:
    return _load().coli_last_reason().decode()


def coli_last_error() -> str:
    return _load().coli_last_error().decode()


def coli_stats():
    a, b, c = C.c_uint64(), C.c_uint64(), C.c_uint64()
    _load().coli_stats(C.addressof(a), C.addressof(b), C.addressof(c))
    return a.value, b.value, c.value


def coli_set_fail_after(n: int) -> None:
    _load().coli_set_fail_after(n)


def coli_moe_router_workspace_bytes(S: int, E: int) -> int:
    return _load().coli_moe_router_workspace_bytes(S, E)


def coli_moe_router(x, S, D, R, bias, E, K, topp, norm_topk, routed_scale, ids, w, workspace,
                    ws_bytes, stream=None) -> int:
    return _load().coli_moe_router(_ptr(x), S, D, _ptr(R), _ptr(bias), E, K, float(topp),
                                   int(bool(norm_topk)), float(routed_scale), _ptr(ids), _ptr(w),
                                   _ptr(workspace), ws_bytes, _stream(stream))


def coli_rmsnorm(x, S, D, w, eps, y, stream=None) -> int:
    return _load().coli_rmsnorm(_ptr(x), S, D, _ptr(w), float(eps), _ptr(y), _stream(stream))


def coli_moe_layer_workspace_bytes(E, S, K, F, D, has_shared) -> int:
    return _load().coli_moe_layer_workspace_bytes(E, S, K, F, D, int(bool(has_shared)))


def coli_moe_layer(gate, up, down, h, S, ln_w, eps, R, bias, K, topp, norm_topk, routed_scale,
                   sh_gate, sh_up, sh_down, out, workspace, ws_bytes, stream=None) -> int:
    return _load().coli_moe_layer(_qp(gate), _qp(up), _qp(down), _ptr(h), S, _ptr(ln_w),
                                  float(eps), _ptr(R), _ptr(bias), K, float(topp),
                                  int(bool(norm_topk)), float(routed_scale), _qp(sh_gate),
                                  _qp(sh_up), _qp(sh_down), _ptr(out), _ptr(workspace), ws_bytes,
                                  _stream(stream))


def coli_probe_read(buf, sink, stream=None) -> int:
    """Stream the bytes of device tensor `buf` once (HBM read probe)."""
    return _load().coli_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                   _stream(stream))


def coli_probe_mfma(workgroups: int, iters: int, sink, stream=None) -> int:
    """workgroups x 4 wavefronts x 8 x iters bf16 32x32x16 products."""
    return _load().coli_probe_mfma(int(workgroups), int(iters), _ptr(sink), _stream(stream))


COLI_MLA_MAX_ROWS = 4096  # include/coli.h
MLA_STAGES = ["cq_raw", "ckv_raw", "cq", "q", "qabs", "qpe", "scores", "p", "clat", "ctx"]


class MlaLayer:
    """A coli_mla_layer record plus the QTensors and norm weights it refers to
    (kept alive)."""

    def __init__(self, q_a, q_b, kv_a, kv_b, o_proj, q_norm, kv_norm, H, d_nope, d_rope, d_v,
                 eps=1e-6, rope_theta=10000.0):
        self.mats = (q_a, q_b, kv_a, kv_b, o_proj)
        self.norms = (q_norm, kv_norm)
        self.desc = coli_mla_layer(
            *[C.addressof(m.desc) for m in self.mats], _ptr(q_norm), _ptr(kv_norm), H, d_nope,
            d_rope, d_v, float(eps), float(rope_theta))


def coli_mla_workspace_bytes(layer, S, T_cap) -> int:
    return _load().coli_mla_workspace_bytes(C.byref(layer.desc), S, T_cap)


def coli_mla_workspace_layout(layer, S, T_cap):
    """(total bytes, {stage name: byte offset})."""
    off = (C.c_size_t * len(MLA_STAGES))()
    tot = _load().coli_mla_workspace_layout(C.byref(layer.desc), S, T_cap, off)
    return tot, dict(zip(MLA_STAGES, list(off)))


def coli_mla_decode(layer, x, S, pos_base, Lc, Rc, T_cap, out, workspace, ws_bytes,
                    stream=None) -> int:
    return _load().coli_mla_decode(C.byref(layer.desc), _ptr(x), S, pos_base, _ptr(Lc), _ptr(Rc),
                                   T_cap, _ptr(out), _ptr(workspace), ws_bytes, _stream(stream))


LAYER_STAGES = ["xn", "attn", "h", "attn_ws", "moe_ws"]


def coli_layer_decode_workspace_bytes(attn, gate, S, K, T_cap, has_shared) -> int:
    return _load().coli_layer_decode_workspace_bytes(C.byref(attn.desc), _qp(gate), S, K, T_cap,
                                                     int(bool(has_shared)))


def coli_layer_decode_workspace_layout(attn, gate, S, K, T_cap, has_shared):
    """(total bytes, {stage name: byte offset})."""
    off = (C.c_size_t * len(LAYER_STAGES))()
    tot = _load().coli_layer_decode_workspace_layout(C.byref(attn.desc), _qp(gate), S, K, T_cap,
                                                     int(bool(has_shared)), off)
    return tot, dict(zip(LAYER_STAGES, list(off)))


def coli_layer_decode(attn, in_ln, gate, up, down, post_ln, R, bias, K, topp, norm_topk,
                      routed_scale, sh_gate, sh_up, sh_down, eps, x, S, pos_base, Lc, Rc, T_cap,
                      out, workspace, ws_bytes, stream=None) -> int:
    return _load().coli_layer_decode(
        C.byref(attn.desc), _ptr(in_ln), _qp(gate), _qp(up), _qp(down), _ptr(post_ln), _ptr(R),
        _ptr(bias), K, float(topp), int(bool(norm_topk)), float(routed_scale), _qp(sh_gate),
        _qp(sh_up), _qp(sh_down), float(eps), _ptr(x), S, pos_base, _ptr(Lc), _ptr(Rc), T_cap,
        _ptr(out), _ptr(workspace), ws_bytes, _stream(stream))


def coli_probe_launch(workgroups: int, sink, stream=None) -> int:
    """One launch of an empty kernel (the launch floor)."""
    return _load().coli_probe_launch(int(workgroups), _ptr(sink), _stream(stream))


PROBE_MFMA_FLOPS_PER_WG_ITER = 4 * 8 * 2 * 32 * 32 * 16


def coli_prof_enable(on: bool) -> None:
    _load().coli_prof_enable(int(bool(on)))


def coli_prof_reset() -> None:
    _load().coli_prof_reset()


def coli_prof_read(tag: str):
    ms = C.c_double()
    n = _load().coli_prof_read(tag.encode(), C.addressof(ms))
    return int(n), ms.value


def coli_prof_tags():
    out, i = [], 0
    while True:
        t = _load().coli_prof_tag(i)
        if t is None:
            return out
        out.append(t.decode())
        i += 1


def coli_version() -> str:
    return _load().coli_version().decode()


# ---------------------------------------------------------------------------
# Small conveniences (still marshalling only)
# ---------------------------------------------------------------------------

class QTensor:
    """A coli_qtensor record plus the device tensors it refers to (kept alive)."""

    def __init__(self, fmt, q, s, O, I, gs=0, n=None):
        self.q, self.s = q, s
        n = n if n is not None else (q.shape[0] if q.dim() == 3 else 1)
        ng = -(-I // gs) if fmt == 4 else 1
        self.desc = coli_qtensor()
        rc = coli_tensor_upload(self.desc, fmt, n, O, I, gs if fmt == 4 else 0, ng, q, s)
        if rc != COLI_OK:
            raise ColiError(f"coli_tensor_upload declined: {coli_last_reason()}")

    @property
    def fmt(self):
        return self.desc.fmt

    def pack(self, stream=None) -> bool:
        """Attach a packed copy (allocated here with torch) when the format has
        one; returns whether it did."""
        import torch
        d = self.desc
        nb = coli_packed_bytes(d.fmt, d.n, d.O, d.I, d.gs)
        if nb == 0:
            return False
        self.packed = torch.empty(nb, dtype=torch.uint8, device=self.q.device)
        check(coli_tensor_pack(self, self.packed, nb, stream), "coli_tensor_pack")
        return True


def check(rc: int, what: str = "call") -> None:
    """Raise unless rc == COLI_OK, naming the library's reason."""
    if rc == COLI_OK:
        return
    if rc == COLI_DECLINED:
        raise ColiError(f"{what} declined: {coli_last_reason()}")
    raise ColiError(f"{what} failed: {coli_last_error()}")
