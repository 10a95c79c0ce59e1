"""Host-side checks of the C ABI (no GPU): the library loads, exports every
symbol include/coli.h declares, and its validation declines bad input before
touching the device (colibri PR #298: an entry that cannot honour its input
returns 0 -- a declined call is a fallback, not a wrong result)."""
import ctypes as C
import os
import re
import subprocess

import pytest

import bit_gemv_coli_amd as coli

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coli.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(coli_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(coli.LIB_PATH):
        pytest.fail("libcoli.so is not built: run `python -m bit_gemv_coli_amd.build`")
    return coli._load()


def test_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", coli.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    declared = declared_functions()
    assert declared, "no declarations parsed from coli.h"
    missing = [n for n in declared if n not in exported]
    assert not missing, missing
    assert sorted(coli.exported_symbols()) == declared


def test_version(lib):
    assert "gfx950" in coli.coli_version()


FAKE_Q = 0x7f0000000000  # never dereferenced: validation only
FAKE_S = 0x7f0000100000


def upload(fmt, n, O, I, gs, ng, q=FAKE_Q, s=FAKE_S):
    d = coli.coli_qtensor()
    rc = coli.coli_tensor_upload(d, fmt, n, O, I, gs, ng, q, s)
    return rc, d


@pytest.mark.parametrize("args,frag", [
    ((0, 1, 4, 64, 0, 1), "unknown fmt"),
    ((5, 1, 4, 64, 0, 1), "unknown fmt"),
    ((7, 1, 4, 64, 0, 1), "unknown fmt"),
    ((4, 1, 4, 64, 0, 1), "gs >= 1"),
    ((4, 1, 4, 130, 64, 2), "ceil(I/gs)=3"),
    ((4, 1, 4, 130, 64, 4), "ceil(I/gs)=3"),
    ((2, 1, 4, 64, 64, 1), "gs must be 0"),
    ((1, 1, 4, 64, 0, 2), "ng must be 1"),
    ((4, 0, 4, 64, 64, 1), "bad shape"),
    ((4, 1, 0, 64, 64, 1), "bad shape"),
    ((4, 1, 4, 0, 64, 0), "bad shape"),
])
def test_upload_declines(lib, args, frag):
    rc, d = upload(*args)
    assert rc == coli.COLI_DECLINED
    assert frag in coli.coli_last_reason(), coli.coli_last_reason()
    assert d.magic == 0  # nothing written


def test_upload_null_pointers(lib):
    rc, _ = upload(4, 1, 4, 64, 64, 1, q=None)
    assert rc == coli.COLI_DECLINED and "NULL" in coli.coli_last_reason()


@pytest.mark.parametrize("fmt,I,gs,rb,fast,g32,g16", [
    (4, 6144, 64, 3072, True, True, False),
    (4, 6144, 128, 3072, True, True, False),
    (4, 96, 16, 48, True, False, True),
    (4, 130, 64, 65, False, True, False),
    (4, 129, 64, 65, False, True, False),
    (4, 96, 48, 48, True, False, True),
    (4, 96, 24, 48, True, False, False),
    (2, 6144, 0, 3072, True, False, False),
    (3, 6144, 0, 1536, True, False, False),
    (3, 7, 0, 2, False, False, False),
    (1, 6144, 0, 6144, True, False, False),
    (1, 40, 0, 40, False, False, False),
])
def test_upload_layout(lib, fmt, I, gs, rb, fast, g32, g16):
    ng = -(-I // gs) if fmt == 4 else 1
    rc, d = upload(fmt, 3, 5, I, gs, ng)
    assert rc == coli.COLI_OK, coli.coli_last_reason()
    assert d.row_bytes == rb and d.q_stride == 5 * rb and d.s_stride == 5 * ng
    assert bool(d.flags & 1) == fast and bool(d.flags & 2) == g32 and bool(d.flags & 4) == g16


def test_upload_misaligned_codes_not_fast(lib):
    rc, d = upload(4, 1, 4, 64, 64, 1, q=FAKE_Q + 8)
    assert rc == coli.COLI_OK and not (d.flags & 1)


def test_compute_entries_decline_before_device(lib):
    rc, W = upload(4, 1, 4, 64, 64, 1)
    assert rc == coli.COLI_OK
    calls0, dec0, launch0 = coli.coli_stats()
    assert coli.coli_qmatmul(W, None, FAKE_S, 1, 0) == coli.COLI_DECLINED
    assert coli.coli_qmatmul(W, FAKE_S, FAKE_S, 0, 0) == coli.COLI_DECLINED
    assert coli.coli_qmatmul(W, FAKE_S + 2, FAKE_S, 1, 0) == coli.COLI_DECLINED
    bogus = coli.coli_qtensor()
    assert coli.coli_qmatmul(bogus, FAKE_S, FAKE_S, 1, 0) == coli.COLI_DECLINED
    assert "coli_tensor_upload" in coli.coli_last_reason()
    assert coli.coli_dequantize(bogus, FAKE_S, 0) == coli.COLI_DECLINED
    assert coli.coli_moe_route(None, 1, 8, 256, FAKE_S, FAKE_S, FAKE_S, FAKE_S, 0) == 0
    assert coli.coli_moe_route(FAKE_S, 1, 8, 5000, FAKE_S, FAKE_S, FAKE_S, FAKE_S, 0) == 0
    _, _, launch1 = coli.coli_stats()
    assert launch1 == launch0  # nothing was launched


def test_two_phase_block_declines_before_device(lib):
    """begin / end validate like coli_moe_block, need the late flags, and size
    their workspace for both calls; nothing is launched on a decline."""
    g, u, d = _moe_tensors()
    _, _, launch0 = coli.coli_stats()
    need = coli.coli_moe_block_two_phase_workspace_bytes(4, 2, 2, 64, 128, False)
    assert need > coli.coli_moe_workspace_bytes(4, 2, 2, 64, 128, False)
    assert coli.coli_moe_block_two_phase_workspace_bytes(0, 2, 2, 64, 128, False) == 0
    ws = FAKE_Q // 256 * 256 + 256
    b = coli.coli_moe_block_begin
    assert b(g, u, d, FAKE_S, 2, FAKE_S, FAKE_S, 2, None, None, None, None, FAKE_S, ws, need, 0) == 0
    assert "late" in coli.coli_last_reason()
    assert b(g, u, d, FAKE_S, 2, FAKE_S, FAKE_S, 2, FAKE_S, None, None, None, FAKE_S, ws, need - 1,
             0) == 0
    assert b(g, u, d, FAKE_S, 2, FAKE_S, FAKE_S, 2, FAKE_S, None, None, None, FAKE_S, ws + 8, need,
             0) == 0
    e = coli.coli_moe_block_end
    assert e(g, u, d, FAKE_S, 2, FAKE_S, 2, False, FAKE_S, None, need, 0) == 0
    assert e(g, u, d, FAKE_S, 2, FAKE_S, 2, False, None, ws, need, 0) == 0
    assert e(coli.coli_qtensor(), u, d, FAKE_S, 2, FAKE_S, 2, False, FAKE_S, ws, need, 0) == 0
    _, _, launch1 = coli.coli_stats()
    assert launch1 == launch0


def test_qmatmul_group_declines_before_device(lib):
    """Every member is validated before anything is enqueued: bad counts,
    NULL arrays or members, S < 1, misaligned pointers and tensors never
    uploaded all decline with no launch."""
    rc, W = upload(4, 1, 4, 64, 64, 1)
    assert rc == coli.COLI_OK
    _, _, launch0 = coli.coli_stats()
    g = coli.coli_qmatmul_group
    assert g([], [], [], 1, 0) == coli.COLI_DECLINED
    assert g([W] * 9, [FAKE_S] * 9, [FAKE_S] * 9, 1, 0) == coli.COLI_DECLINED
    assert "1..8" in coli.coli_last_reason()
    assert g([W, W], [FAKE_S, None], [FAKE_S, FAKE_S], 1, 0) == coli.COLI_DECLINED
    assert "member 1" in coli.coli_last_reason()
    assert g([W], [FAKE_S], [FAKE_S], 0, 0) == coli.COLI_DECLINED
    assert g([W, W], [FAKE_S, FAKE_S], [FAKE_S, FAKE_S + 2], 1, 0) == coli.COLI_DECLINED
    assert g([W, coli.coli_qtensor()], [FAKE_S] * 2, [FAKE_S] * 2, 1, 0) == coli.COLI_DECLINED
    assert "coli_tensor_upload" in coli.coli_last_reason()
    L = coli._load()
    assert L.coli_qmatmul_group(1, None, None, None, 1, None) == coli.COLI_DECLINED
    with pytest.raises(ValueError):
        g([W], [FAKE_S, FAKE_S], [FAKE_S], 1, 0)
    _, _, launch1 = coli.coli_stats()
    assert launch1 == launch0


def _moe_tensors(fmt=4, E=4, F=64, D=128, gs=64):
    ng_g = -(-D // gs) if fmt == 4 else 1
    ng_d = -(-F // gs) if fmt == 4 else 1
    g = upload(fmt, E, F, D, gs if fmt == 4 else 0, ng_g)[1]
    u = upload(fmt, E, F, D, gs if fmt == 4 else 0, ng_g)[1]
    d = upload(fmt, E, D, F, gs if fmt == 4 else 0, ng_d)[1]
    return g, u, d


def test_moe_block_declines(lib):
    g, u, d = _moe_tensors()
    ws = coli.coli_moe_workspace_bytes(4, 1, 2, 64, 128, 0)
    assert ws > 0
    base = dict(x=FAKE_S, S=1, ids=FAKE_S, w=FAKE_S, K=2, out=FAKE_S, workspace=FAKE_Q, ws=ws)

    def call(gate=g, up=u, down=d, sh=(None, None, None), **kw):
        a = dict(base, **kw)
        return coli.coli_moe_block(gate, up, down, a["x"], a["S"], a["ids"], a["w"], a["K"],
                                   sh[0], sh[1], sh[2], a["out"], a["workspace"], a["ws"], 0)

    assert call(ws=ws - 1) == 0 and "workspace" in coli.coli_last_reason()
    assert call(workspace=FAKE_Q + 64) == 0 and "aligned" in coli.coli_last_reason()
    assert call(K=0) == 0
    assert call(K=65) == 0
    assert call(x=FAKE_S + 4) == 0 and "16-byte" in coli.coli_last_reason()
    assert call(down=u) == 0 and "down" in coli.coli_last_reason()
    # a shared expert whose group size differs from the routed experts is declined
    sg, su, sd = _moe_tensors(E=1, gs=32)
    assert call(sh=(sg, su, sd)) == 0 and "group sizes" in coli.coli_last_reason()
    sg, su, sd = _moe_tensors(E=1)
    assert call(sh=(sg, su, None)) == 0 and "shared" in coli.coli_last_reason()
    # a format mix is declined
    g1, u1, d1 = _moe_tensors(fmt=2)
    assert call(gate=g1) == 0 and "fmt" in coli.coli_last_reason()
    # an expert stack whose rows are not whole packets is declined, loudly
    g2, u2, d2 = _moe_tensors(D=130)
    assert call(gate=g2, up=u2, down=d2) == 0


def test_workspace_sizes(lib):
    assert coli.coli_moe_workspace_bytes(0, 1, 8, 2048, 6144, 0) == 0
    a = coli.coli_moe_workspace_bytes(256, 1, 8, 2048, 6144, 0)
    b = coli.coli_moe_workspace_bytes(256, 1, 8, 2048, 6144, 1)
    assert a >= 8 * 2048 * 4 and b >= 9 * 2048 * 4 and a % 256 == 0


def test_gemv_threshold(lib):
    old = coli.coli_gemv_max_rows()
    assert 1 <= old <= 4
    assert coli.coli_set_gemv_max_rows(9) == 0
    assert coli.coli_set_gemv_max_rows(2) == old
    assert coli.coli_gemv_max_rows() == 2
    coli.coli_set_gemv_max_rows(old)


def test_fault_injection_declines(lib):
    rc, W = upload(4, 1, 4, 64, 64, 1)
    coli.coli_set_fail_after(0)
    try:
        # valid arguments, but injection trips before any launch
        _, _, l0 = coli.coli_stats()
        assert coli.coli_qmatmul(W, FAKE_S, FAKE_S + 4096, 1, 0) == coli.COLI_DECLINED
        assert "fault injection" in coli.coli_last_reason()
        _, _, l1 = coli.coli_stats()
        assert l1 == l0
    finally:
        coli.coli_set_fail_after(-1)


def test_moe_hidden_validation(lib):
    g, u, d = _moe_tensors()
    ws = coli.coli_moe_workspace_bytes(4, 1, 2, 64, 128, 0)
    # no shared expert: validation reaches the output check
    assert coli.coli_moe_hidden(g, u, FAKE_S, 1, FAKE_S, 2, None, None, None, FAKE_Q, ws, 0) == 0
    assert "h_out" in coli.coli_last_reason(), coli.coli_last_reason()
    sg, su, _ = _moe_tensors(E=1)
    assert coli.coli_moe_hidden(g, u, FAKE_S, 1, FAKE_S, 2, sg, None, FAKE_S, FAKE_Q, ws, 0) == 0
    assert "shared" in coli.coli_last_reason()
    assert coli.coli_moe_hidden(g, u, FAKE_S, 1, FAKE_S, 2, sg, su, None, FAKE_Q, ws, 0) == 0
    assert "h_out" in coli.coli_last_reason(), coli.coli_last_reason()


@pytest.mark.parametrize("fmt,O,I,gs,expect", [
    (4, 2048, 6144, 64, 2048 // 16 * 48 * (1024 + 2 * 64)),
    (4, 6144, 2048, 128, 6144 // 16 * 16 * (1024 + 64)),
    (4, 33, 4160, 32, 3 * 33 * 1024 + 3 * 9 * 16 * 4 * 4 * 4),  # scales in whole quads
    (2, 100, 256, 0, ((7 * 2 * 1024 + 255) // 256) * 256),
    (1, 16, 128, 0, 2048), (1, 40, 4096 + 32, 0, 3 * 33 * 2048),   # int8: 2 KiB tile blocks
    (3, 16, 128, 0, 512), (3, 40, 4096 + 32, 0, 3 * 33 * 512),     # int2: 512-byte tile blocks
    (4, 16, 96, 48, 0), (4, 16, 96, 16, 0), (1, 16, 100, 0, 0), (3, 16, 66, 0, 0),
    (4, 16, 100, 64, 0),
])
def test_packed_bytes(lib, fmt, O, I, gs, expect):
    assert coli.coli_packed_bytes(fmt, 1, O, I, gs) == expect
    assert coli.coli_packed_bytes(fmt, 3, O, I, gs) == 3 * expect


def test_pack_declines_before_device(lib):
    _, _, l0 = coli.coli_stats()
    rc, W = upload(4, 1, 64, 96, 48, 2)
    assert coli.coli_tensor_pack(W, FAKE_Q, 1 << 20, 0) == 0 and "packed form" in coli.coli_last_reason()
    rc, W = upload(4, 1, 64, 256, 64, 4)
    need = coli.coli_packed_bytes(4, 1, 64, 256, 64)
    assert coli.coli_tensor_pack(W, FAKE_Q, need - 1, 0) == 0 and "bytes" in coli.coli_last_reason()
    assert coli.coli_tensor_pack(W, FAKE_Q + 64, need, 0) == 0 and "aligned" in coli.coli_last_reason()
    rc, W = upload(4, 1, 64, 256, 64, 4, q=FAKE_Q + 8)
    assert coli.coli_tensor_pack(W, FAKE_Q, need, 0) == 0 and "aligned" in coli.coli_last_reason()
    _, _, l1 = coli.coli_stats()
    assert l1 == l0
