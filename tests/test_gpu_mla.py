"""GPU parity of the MLA decode attention (coli_mla_decode) against the oracle
(colibri-strix commit log: fused decode attention commit (Phase 2) and its
S <= 4 commit -- row s attends keys [0, pos_base + s]; the regression test
commit checks S = 1/3/4 at pos_base 0/12/37 including the cache rows).

Every step is checked against the oracle's step evaluated on the GPU's own
input to that step (the stage arrays the call leaves in its workspace):
  projections (q_a, kv_a, q_b, o_proj)  decode GEMV bound tau*A (+ the
                                        matrix-core term 2^-29*Ahat)
  RMSNorm, RoPE                         one f32 rounding of an f64 result:
                                        2^-22 * |y| / 2^-22 * (|a| + |b|)
  qabs, scores, clat, ctx               fp32 sums: tau * sum |terms| (ctx of
                                        more than 4 rows with a packed kv_b
                                        whose head blocks are whole 16-row
                                        tiles: the bf16 matrix cores, 4e-3)
  softmax                               (8 + n + 2 |z - max|) * 2^-24 * p
                                        (the f32 rounding of exp's argument z - max
                                        and exp itself, the n-term sum, one division)
then the output end to end against the oracle's f64 chain."""
import numpy as np
import pytest
import torch

import bit_gemv_coli_amd as coli
import synthdata as sd
from gpu_util import TOL_BF16, TOL_FP32, assert_within, decode_kernels, need_gpu, qtensor, rep_allowance, to_dev
from oracle import MlaWeights, QMat

pytestmark = pytest.mark.gpu

FULL = dict(D=6144, qr=1536, L=512, H=64, dn=192, dr=64, dv=256, gs=64)
SMALL = dict(D=256, qr=64, L=96, H=3, dn=16, dr=8, dv=24, gs=32)


def _setup(seed, S, pb, dims, T=None, pack=True, kvb_fmt=4, theta=10000.0, kva=None):
    d = dict(dims)
    T = T or pb + S + 5
    r = sd.rng(seed)
    mats, shapes, qn, kn, Lc, Rc = sd.gen_mla(r, d["D"], d["qr"], d["L"], d["H"], d["dn"], d["dr"],
                                              d["dv"], d["gs"], T, pb)
    Q = {k: QMat(4, o, i, d["gs"], *mats[k]) for k, (o, i) in shapes.items()}
    if kva is not None:  # kv_a drawn again (its own stream) as (fmt, gs)
        fmt, gs = kva
        q, s_ = sd.gen_matrix(sd.rng(seed + 7919), fmt, *shapes["kv_a"], gs)
        Q["kv_a"] = QMat(fmt, *shapes["kv_a"], gs, q, s_)
    if kvb_fmt == 2:  # kv_b with one scale per row: the first group's scale
        q, s = mats["kv_b"]
        Q["kv_b"] = QMat(2, *shapes["kv_b"], 0, q, np.ascontiguousarray(s[:, 0]))
    W = MlaWeights(Q["q_a"], qn, Q["q_b"], Q["kv_a"], kn, Q["kv_b"], Q["o_proj"], d["H"], d["dn"],
                   d["dr"], d["dv"], eps=1e-6, theta=theta)
    x = sd.gen_x(r, S, d["D"])
    dev = {k: qtensor(Q[k], pack=pack) for k in Q}
    qn_d, kn_d = to_dev(qn), to_dev(kn)
    layer = coli.MlaLayer(dev["q_a"], dev["q_b"], dev["kv_a"], dev["kv_b"], dev["o_proj"], qn_d,
                          kn_d, d["H"], d["dn"], d["dr"], d["dv"], 1e-6, theta)
    layer._keep = (dev, qn_d, kn_d)
    return W, layer, x, Lc, Rc, T


def _run(layer, x, pb, Lc, Rc, T):
    S = x.shape[0]
    total, off = coli.coli_mla_workspace_layout(layer, S, T)
    assert total > 0, coli.coli_last_reason()
    ws = torch.full((total,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN fill
    Lc_d, Rc_d = to_dev(Lc), to_dev(Rc)
    out = torch.full((S, layer.mats[4].desc.O), float("nan"), device="cuda")
    coli.check(coli.coli_mla_decode(layer, to_dev(x), S, pb, Lc_d, Rc_d, T, out, ws, total),
               "coli_mla_decode")
    torch.cuda.synchronize()
    wsh = ws.cpu().numpy()

    def stage(name, shape):
        n = int(np.prod(shape))
        return wsh[off[name]:off[name] + 4 * n].view(np.float32).reshape(shape).copy()
    return out.cpu().numpy(), Lc_d.cpu().numpy(), Rc_d.cpu().numpy(), stage


def _check(orc, W, x, pb, Lc, Rc, T, out, Lc1, Rc1, stage, packed=True):
    S = x.shape[0]
    H, dn, dr, dv, L, qr = W.H, W.dn, W.dr, W.dv, W.kv_b.I, W.q_a.O
    # more than 4 rows: the projections run the bf16 prefill kernels
    tol = TOL_FP32 if S <= 4 else TOL_BF16
    rep = ((lambda M, inp: rep_allowance(orc, M, inp)) if packed and S <= 4
           else (lambda M, inp: None))
    cq_raw = stage("cq_raw", (S, qr))
    ckv = stage("ckv_raw", (S, L + dr))
    cq = stage("cq", (S, qr))
    q = stage("q", (S, H * (dn + dr)))
    qabs = stage("qabs", (S, H, L))
    qpe = stage("qpe", (S, H, dr))
    sc = stage("scores", (S, H, T))
    p = stage("p", (S, H, T))
    clat = stage("clat", (S, H, L))
    ctx = stage("ctx", (S, H * dv))
    # projections from x
    for M, y, nm in ((W.q_a, cq_raw, "q_a"), (W.kv_a, ckv, "kv_a")):
        yr, A = orc.qmatmul(M, x)
        assert_within(y, yr, A, tol, nm, rep(M, x))
    # norms, rotary key, cache rows
    ref = orc.rmsnorm(cq_raw, W.q_norm, W.eps)
    assert np.all(np.abs(cq - ref) <= 2.0 ** -22 * np.abs(ref) + 1e-30), "q latent norm"
    ref = orc.rmsnorm(np.ascontiguousarray(ckv[:, :L]), W.kv_norm, W.eps)
    assert np.all(np.abs(Lc1[pb:pb + S] - ref) <= 2.0 ** -22 * np.abs(ref) + 1e-30), "Lc rows"

    def rope_check(got, src, pos, what):
        ref = orc.rope(src.astype(np.float64), pos, W.theta)
        pair = np.abs(src[..., 0::2]).astype(np.float64) + np.abs(src[..., 1::2])
        bound = 2.0 ** -22 * np.repeat(pair, 2, axis=-1) + 1e-30
        assert np.all(np.abs(got - ref) <= bound), what
    for s in range(S):
        rope_check(Rc1[pb + s], ckv[s, L:], pb + s, f"Rc row {pb + s}")
    keep = np.ones(T, bool)
    keep[pb:pb + S] = False
    assert np.array_equal(Lc1[keep], Lc[keep]) and np.array_equal(Rc1[keep], Rc[keep]), \
        "cache rows outside this call's positions changed"
    # q_b
    yr, A = orc.qmatmul(W.q_b, cq)
    assert_within(q, yr, A, tol, "q_b", rep(W.q_b, cq))
    # rotary part of the query
    qh = q.reshape(S, H, dn + dr)
    for s in range(S):
        rope_check(qpe[s], qh[s, :, dn:], pb + s, f"qpe row {s}")
    # key absorption
    ref, A = orc.mla_qabs(W.kv_b, H, dn, dr, dv, q)
    assert_within(qabs, ref, A, TOL_FP32, "qabs")
    # scores over keys 0 .. pb + s
    ref, A = orc.mla_scores(qabs, qpe, Lc1, Rc1, pb, W.scale)
    for s in range(S):
        n = pb + s + 1
        assert_within(sc[s, :, :n], ref[s, :, :n], A[s, :, :n], TOL_FP32, f"scores row {s}")
    # softmax from the GPU's scores
    scd = np.zeros((S, H, pb + S))
    for s in range(S):
        scd[s, :, :pb + s + 1] = sc[s, :, :pb + s + 1]
    ref = orc.mla_softmax(scd, pb)
    for s in range(S):
        n = pb + s + 1
        z = scd[s, :, :n]
        gap = z.max(axis=1, keepdims=True) - z   # exp's argument; its f32 rounding
        err = np.abs(p[s, :, :n] - ref[s, :, :n])  # becomes a relative error of p
        bound = (8 + n + 2 * gap) * 2.0 ** -24 * ref[s, :, :n] + 1e-30
        assert np.all(err <= bound), f"softmax row {s}: max err/bound {np.max(err / bound):.3e}"
    # latent context from the GPU's probabilities
    pd = np.zeros((S, H, pb + S))
    for s in range(S):
        pd[s, :, :pb + s + 1] = p[s, :, :pb + s + 1]
    ref, A = orc.mla_clat(pd, Lc1, pb)
    assert_within(clat, ref, A, TOL_FP32, "clat")
    # value absorption (more than 4 rows, packed kv_b with head blocks of
    # whole 16-row tiles: per-head products on the bf16 matrix cores), o_proj
    ref, A = orc.mla_ctx(W.kv_b, H, dn, dv, clat)
    ctx_mc = S > 4 and packed and dn % 16 == 0 and (dn + dv) % 16 == 0 and W.kv_b.fmt in (2, 4)
    assert_within(ctx, ref, A, TOL_BF16 if ctx_mc else TOL_FP32, "ctx")
    yr, A = orc.qmatmul(W.o_proj, ctx)
    assert_within(out, yr, A, tol, "o_proj", rep(W.o_proj, ctx))
    # end to end against the oracle's f64 chain: within 1e-4 (fp32
    # projections) or 5e-2 (bf16 projections, S > 4) of the output
    # projection's magnitude -- the sum of the steps' bounds, carried through
    # the softmax, stays inside it for these inputs
    o_ref, st, Lc_ref, Rc_ref = orc.mla_decode(W, x, pb, Lc, Rc)
    _, A_o = orc.qmatmul(W.o_proj, np.abs(st["ctx"]).astype(np.float32))
    err = np.abs(out - o_ref)
    e2e = 1e-4 if S <= 4 else 5e-2
    assert np.all(err <= e2e * A_o + 1e-30), f"end to end: max err/A {np.max(err / A_o):.3e}"
    return float(np.max(err / A_o))


CASES = [(S, pb) for S in (1, 3, 4) for pb in (0, 12, 37)]


@pytest.mark.parametrize("S,pb", CASES, ids=[f"S{S}-pos{pb}" for S, pb in CASES])
def test_mla_decode_full_dims(orc, S, pb):
    """The pages' matrix: S = 1/3/4 x pos_base 0/12/37 at the layer's real
    dimensions (hidden 6144, q_a 1536, latent 512 + rotary 64, 64 heads of
    192 + 64 query and 256 value components), fmt 4 g64, packed projections."""
    need_gpu()
    W, layer, x, Lc, Rc, T = _setup(40 + 7 * S + pb, S, pb, FULL)
    out, Lc1, Rc1, stage = _run(layer, x, pb, Lc, Rc, T)
    _check(orc, W, x, pb, Lc, Rc, T, out, Lc1, Rc1, stage)


@pytest.mark.parametrize("S,pb,T", [(1, 0, 1), (2, 63, 70), (4, 300, 304), (3, 600, 700)])
def test_mla_decode_small_dims_long_context(orc, S, pb, T):
    """Odd dimensions (3 heads, latent 96, gs 32), a cache exactly as long as
    the call needs, and contexts across several 64-key and 256-key chunks."""
    need_gpu()
    W, layer, x, Lc, Rc, T = _setup(90 + S + pb, S, pb, SMALL, T=T)
    out, Lc1, Rc1, stage = _run(layer, x, pb, Lc, Rc, T)
    _check(orc, W, x, pb, Lc, Rc, T, out, Lc1, Rc1, stage)


PREFILL = [(5, 0, None), (9, 7, None), (13, 3, 20), (40, 0, 48), (27, 61, 100),
           (66, 0, None), (70, 3, 80), (130, 10, 150), (200, 3, 210), (389, 7, 400)]


@pytest.mark.parametrize("S,pb,T", PREFILL, ids=[f"S{S}-pos{pb}-T{T}" for S, pb, T in PREFILL])
def test_mla_prefill_small_dims(orc, S, pb, T):
    """More than 4 rows (prefill): the projections on the bf16 prefill
    kernels, the core in groups of up to 192 rows (64-row tiles inside a
    group; 200 and 389 rows make two and three groups), row s attending keys
    up to pos_base + s -- including groups whose keys are the earlier groups'
    new cache rows."""
    need_gpu()
    W, layer, x, Lc, Rc, T = _setup(300 + S + pb, S, pb, SMALL, T=T)
    out, Lc1, Rc1, stage = _run(layer, x, pb, Lc, Rc, T)
    _check(orc, W, x, pb, Lc, Rc, T, out, Lc1, Rc1, stage)


@pytest.mark.parametrize("S,pb", [(24, 37), (68, 5), (200, 5)], ids=["S24-pos37", "S68-pos5", "S200-pos5"])
def test_mla_prefill_full_dims(orc, S, pb):
    """Prefill rows at the layer's real dimensions: one group of 24 rows, one
    of 68 (two 64-row tiles), and two groups of 100 rows whose latent
    contexts feed one value absorption of all rows on the bf16 matrix cores."""
    need_gpu()
    W, layer, x, Lc, Rc, T = _setup(330 + S, S, pb, FULL)
    out, Lc1, Rc1, stage = _run(layer, x, pb, Lc, Rc, T)
    _check(orc, W, x, pb, Lc, Rc, T, out, Lc1, Rc1, stage)


@pytest.mark.parametrize("kva", [(4, 128), (2, 0)], ids=["kva-g128", "kva-fmt2"])
def test_mla_prefill_kva_other_layout(orc, kva):
    """Prefill with kv_a in another layout than q_a (fmt 4 gs 64): gs 128
    (q_a and kv_a still share one launch of the split-K GEMM, each with its
    own group geometry) and per-row fmt 2 (two launches)."""
    need_gpu()
    W, layer, x, Lc, Rc, T = _setup(360 + kva[1], 24, 37, FULL, kva=kva)
    out, Lc1, Rc1, stage = _run(layer, x, 37, Lc, Rc, T)
    _check(orc, W, x, 37, Lc, Rc, T, out, Lc1, Rc1, stage)


@pytest.mark.parametrize("kmode", [0, 1], ids=["mfma", "valu"])
def test_mla_decode_kvb_per_row_and_plain_projections(orc, kmode):
    """kv_b with one scale per row (fmt 2), projections without packed copies
    (vector-ALU GEMVs) and with them under the vector-ALU mode."""
    need_gpu()
    W, layer, x, Lc, Rc, T = _setup(120 + kmode, 3, 9, SMALL, pack=(kmode == 0), kvb_fmt=2,
                                    theta=500.0)
    with decode_kernels(kmode):
        out, Lc1, Rc1, stage = _run(layer, x, 9, Lc, Rc, T)
    _check(orc, W, x, 9, Lc, Rc, T, out, Lc1, Rc1, stage, packed=(kmode == 0))


def test_mla_decode_rows_match_single_row_calls(orc):
    """An S = 4 call equals four S = 1 calls at consecutive positions (the
    cache carrying the earlier rows) within the per-row bounds, and the S = 1
    calls are bit-identical to rerunning them."""
    need_gpu()
    W, layer, x, Lc, Rc, T = _setup(140, 4, 20, SMALL)
    out4, Lc4, Rc4, _ = _run(layer, x, 20, Lc, Rc, T)
    Lcs, Rcs = Lc, Rc
    for s in range(4):
        o1, Lcs, Rcs, _ = _run(layer, x[s:s + 1], 20 + s, Lcs, Rcs, T)
        o1b, _, _, _ = _run(layer, x[s:s + 1], 20 + s, Lcs, Rcs, T)
        assert np.array_equal(o1.view(np.uint32), o1b.view(np.uint32))
        ref, _, _, _ = orc.mla_decode(W, x[s:s + 1], 20 + s, Lcs, Rcs)
        scale = np.max(np.abs(ref)) + 1e-30
        assert np.max(np.abs(out4[s] - o1[0])) <= 1e-4 * scale, s


def test_mla_decode_declines():
    """Host-side refusals: positions past the cache, more rows than the
    workspace was sized for or than COLI_MLA_MAX_ROWS, a too-small workspace;
    nothing is launched."""
    need_gpu()
    W, layer, x, Lc, Rc, T = _setup(150, 2, 3, SMALL)
    total = coli.coli_mla_workspace_bytes(layer, 2, T)
    ws = torch.empty(total, dtype=torch.uint8, device="cuda")
    xd, Lc_d, Rc_d = to_dev(x), to_dev(Lc), to_dev(Rc)
    out = torch.zeros((2, 256), device="cuda")
    n0 = coli.coli_stats()[2]
    assert coli.coli_mla_decode(layer, xd, 2, T - 1, Lc_d, Rc_d, T, out, ws, total) == 0
    assert coli.coli_mla_decode(layer, xd, 5, 0, Lc_d, Rc_d, T, out, ws, total) == 0
    assert coli.coli_mla_decode(layer, xd, 2, 0, Lc_d, Rc_d, T, out, ws, total - 256) == 0
    assert coli.coli_mla_workspace_bytes(layer, coli.COLI_MLA_MAX_ROWS + 1, 1 << 14) == 0
    assert coli.coli_stats()[2] == n0
