"""GPU parity of the whole decode layer in one submission (coli_layer_decode;
colibri-strix commit log, full decode layer commit: in_ln RMSNorm -> fused
attention -> residual add -> post_ln RMSNorm -> shared expert, router with the
exact top-K, routed experts -> residual add) against the oracle, step by step
from the GPU's own input to each step (the workspace keeps them):
  xn      one f32 rounding of the oracle's f64 norm of x
  a       the attention's staged checks on the GPU's xn (test_gpu_mla)
  h       x + a in f32, bit-exact
  experts picks bit-exact against the oracle's router on the GPU's h; the
          block within its staged bound (test_gpu_moe)."""
import numpy as np
import pytest
import torch

import bit_gemv_coli_amd as coli
import synthdata as sd
from gpu_util import TOL_BF16, TOL_FP32, decode_kernels, need_gpu, qtensor, to_dev
from test_gpu_mla import FULL, SMALL, _check as check_attention, _setup as setup_attention
from test_gpu_moe import _check_moe, _moe_inputs

pytestmark = pytest.mark.gpu

CASES = [  # (S, pos_base, attention dims, E, F, K, shared, topp, decode kernels)
    (1, 0, FULL, 16, 1024, 8, True, 0.0, 0),
    (4, 37, FULL, 16, 1024, 8, True, 0.8, 0),
    (3, 12, SMALL, 12, 96, 4, True, 0.0, 0),
    (2, 70, SMALL, 9, 64, 3, False, 0.9, 0),
    # the vector-ALU decode kernels: every norm and residual add a launch of its own
    (2, 33, SMALL, 10, 64, 4, True, 0.0, 1),
    # prefill rows: the bf16 prefill kernels, norms and residual adds on their own
    (9, 20, SMALL, 12, 96, 4, True, 0.0, 0),
]


def _al256(n):
    return (n + 255) // 256 * 256


@pytest.mark.parametrize("case", CASES, ids=["S{}-pos{}-D{}-E{}-F{}-K{}-sh{}-p{}-k{}".format(
    c[0], c[1], c[2]["D"], *c[3:]) for c in CASES])
def test_layer_decode_matches_oracle(orc, case):
    need_gpu()
    S, pb, dims, E, F, K, shared, topp, kmode = case
    D, eps, norm, scale = dims["D"], 1e-6, True, 2.5
    W, layer, x, Lc, Rc, T = setup_attention(500 + S + pb + D, S, pb, dims)
    G, U, Dn, sh, _, _, _ = _moe_inputs(600 + S + E, 4, S, K, E, D, F, 64 if D > 256 else 32,
                                        shared)
    r = sd.rng(700 + S)
    R = (r.standard_normal((E, D)) / np.sqrt(D)).astype(np.float32)
    bias = (r.standard_normal(E) * 0.05).astype(np.float32)
    in_ln = r.uniform(0.5, 1.5, D).astype(np.float32)
    post_ln = r.uniform(0.5, 1.5, D).astype(np.float32)
    x = (x * 2.0).astype(np.float32)
    tg, tu, td = qtensor(G, True), qtensor(U, True), qtensor(Dn, True)
    ts = [qtensor(m, True) for m in sh] if sh is not None else [None, None, None]
    total, off = coli.coli_layer_decode_workspace_layout(layer, tg, S, K, T, sh is not None)
    assert total > 0, coli.coli_last_reason()
    ws = torch.full((total,), 0xFF, dtype=torch.uint8, device="cuda")
    Lc_d, Rc_d = to_dev(Lc), to_dev(Rc)
    out = torch.full((S, D), float("nan"), device="cuda")
    with decode_kernels(kmode):
        coli.check(coli.coli_layer_decode(layer, to_dev(in_ln), tg, tu, td, to_dev(post_ln),
                                          to_dev(R), to_dev(bias), K, topp, norm, scale, ts[0],
                                          ts[1], ts[2], eps, to_dev(x), S, pb, Lc_d, Rc_d, T, out,
                                          ws, total), "coli_layer_decode")
        torch.cuda.synchronize()
    wsh = ws.cpu().numpy()

    def arr(at, shape, dtype=np.float32):
        n = int(np.prod(shape)) * np.dtype(dtype).itemsize
        return wsh[at:at + n].view(dtype).reshape(shape).copy()
    xn = arr(off["xn"], (S, D))
    a = arr(off["attn"], (S, D))
    h = arr(off["h"], (S, D))
    out = out.cpu().numpy()
    # 1. input norm
    ref = orc.rmsnorm(x, in_ln, eps)
    assert np.all(np.abs(xn - ref) <= 2.0 ** -24 * np.abs(ref) * 1.0001), "in_ln"
    # 2. attention on the GPU's xn, from the attention's own workspace
    _, moff = coli.coli_mla_workspace_layout(layer, S, T)

    def stage(name, shape):
        return arr(off["attn_ws"] + moff[name], shape)
    check_attention(orc, W, xn, pb, Lc, Rc, T, a, Lc_d.cpu().numpy(), Rc_d.cpu().numpy(), stage,
                    packed=(kmode == 0))
    # 3. residual
    assert np.array_equal(h, (x + a).astype(np.float32)), "h = x + a"
    # 4. the expert half on the GPU's h: picks, then the block
    out_ref, st = orc.moe_layer(h, post_ln, eps, R, bias, K, topp, norm, scale, G, U, Dn,
                                shared=sh)
    ids = arr(off["moe_ws"] + _al256(S * D * 4), (S, K), np.int32)
    assert np.array_equal(ids, st["ids"]), (ids, st["ids"])
    xn2 = arr(off["moe_ws"], (S, D))
    assert np.all(np.abs(xn2 - st["xn"]) <= 2.0 ** -24 * np.abs(st["xn"]) * 1.0001), "post_ln"
    y_est = out.astype(np.float64) - h.astype(np.float64)
    _check_moe(orc, G, U, Dn, sh, st["xn"], st["ids"], st["w"].astype(np.float32), y_est, None,
               TOL_FP32 if S <= 4 else TOL_BF16)


def test_layer_decode_in_place_and_declines(orc):
    """out = x in place gives the same bits as a separate output; a K the
    router cannot take and a position past the cache are declined."""
    need_gpu()
    S, pb, E, F, K = 2, 5, 8, 64, 4
    W, layer, x, Lc, Rc, T = setup_attention(800, S, pb, SMALL)
    D = SMALL["D"]
    G, U, Dn, sh, _, _, _ = _moe_inputs(801, 4, S, K, E, D, F, 32, True)
    R = (sd.rng(802).standard_normal((E, D)) / np.sqrt(D)).astype(np.float32)
    tg, tu, td = qtensor(G, True), qtensor(U, True), qtensor(Dn, True)
    ts = [qtensor(m, True) for m in sh]
    total = coli.coli_layer_decode_workspace_bytes(layer, tg, S, K, T, True)
    ws = torch.empty(total, dtype=torch.uint8, device="cuda")
    Rd = to_dev(R)

    def run(xd, out, k=K, pos=pb):
        Lc_d, Rc_d = to_dev(Lc), to_dev(Rc)
        return coli.coli_layer_decode(layer, None, tg, tu, td, None, Rd, None, k, 0.0, 1, 1.0,
                                      ts[0], ts[1], ts[2], 1e-6, xd, S, pos, Lc_d, Rc_d, T, out,
                                      ws, total)
    xd = to_dev(x)
    sep = torch.empty_like(xd)
    coli.check(run(xd, sep), "separate output")
    inplace = to_dev(x)
    coli.check(run(inplace, inplace), "in place")
    torch.cuda.synchronize()
    assert np.array_equal(sep.cpu().numpy().view(np.uint32), inplace.cpu().numpy().view(np.uint32))
    n0 = coli.coli_stats()[2]
    assert run(xd, sep, k=17) == coli.COLI_DECLINED
    assert run(xd, sep, pos=T - 1) == coli.COLI_DECLINED
    assert coli.coli_stats()[2] == n0
