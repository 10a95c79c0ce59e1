"""Seeded synthetic inputs shaped like the colibri workloads.

This module only draws random numbers and lays them out in the storage
formats; it holds none of the matmul / MoE arithmetic, so both the GPU tests
and the CPU oracle can consume what it produces.

Draw order inside one case is fixed: x -> weight codes -> scales -> routing.
Everything uses numpy's PCG64 (``np.random.default_rng(seed)``).  The
multi-GB expert pools of the benchmark are drawn on the GPU with a seeded
torch generator instead (``pool_on_device``); the oracle then receives the
few experts it needs copied back to the host.

Value distributions (the workloads of the pages' decode and prefill runs):
  x        ~ N(0,1) float32
  fmt 1    int8 uniform in [-127, 127]
  fmt 2/4  uniform random bytes (two independent uniform nibbles 0..15)
  fmt 3    uniform random bytes (four independent uniform 2-bit codes)
  scales   uniform in [0.001, 0.02] float32
  decode routing  K distinct experts uniform without replacement per token,
                  weights = softmax of K N(0,1) logits
  prefill routing expert popularity Zipf(s) over ranks 1..E mapped to ids by
                  a seeded permutation, K distinct experts per token drawn by
                  Gumbel-top-K on log p (sampling without replacement), weights
                  = softmax of K N(0,1) logits
"""
from __future__ import annotations

import numpy as np

SCALE_LO, SCALE_HI = 0.001, 0.02


def row_bytes(fmt: int, I: int) -> int:
    """Storage bytes of one row (layout only: fmt 1 byte/input, fmt 2/4 two
    nibbles per byte, fmt 3 four 2-bit codes per byte)."""
    return {1: I, 2: (I + 1) // 2, 4: (I + 1) // 2, 3: (I + 3) // 4}[fmt]


def n_groups(fmt: int, I: int, gs: int) -> int:
    return -(-I // gs) if fmt == 4 else 1


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def gen_x(r: np.random.Generator, S: int, I: int) -> np.ndarray:
    return r.standard_normal((S, I), dtype=np.float32)


def gen_codes(r: np.random.Generator, fmt: int, O: int, I: int, n: int | None = None) -> np.ndarray:
    """uint8 [(n,) O, row_bytes]; fmt 1 bytes are int8 values viewed as uint8."""
    shape = (O, row_bytes(fmt, I)) if n is None else (n, O, row_bytes(fmt, I))
    if fmt == 1:
        return r.integers(-127, 128, size=shape, dtype=np.int8).view(np.uint8)
    return r.integers(0, 256, size=shape, dtype=np.uint8)


def gen_scales(r: np.random.Generator, fmt: int, O: int, I: int, gs: int,
               n: int | None = None) -> np.ndarray:
    ng = n_groups(fmt, I, gs)
    shape = (O, ng) if fmt == 4 else (O,)
    if n is not None:
        shape = (n,) + shape
    return r.uniform(SCALE_LO, SCALE_HI, size=shape).astype(np.float32)


def gen_matrix(r: np.random.Generator, fmt: int, O: int, I: int, gs: int = 64,
               n: int | None = None):
    """(codes, scales) for one matrix or a stack of n."""
    q = gen_codes(r, fmt, O, I, n)
    s = gen_scales(r, fmt, O, I, gs, n)
    return q, s


def _softmax_rows(z: np.ndarray) -> np.ndarray:
    # plain normalisation of the drawn logits into routing weights
    z = z.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def gen_routing_uniform(r: np.random.Generator, S: int, K: int, E: int):
    """ids int32 [S][K] (distinct per token), w float32 [S][K]."""
    ids = np.stack([r.choice(E, size=K, replace=False) for _ in range(S)]).astype(np.int32)
    w = _softmax_rows(r.standard_normal((S, K)))
    return ids, w


def zipf_popularity(r: np.random.Generator, E: int, s: float) -> np.ndarray:
    """p[e]: Zipf(s) over ranks 1..E, ranks assigned to ids by a permutation."""
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p_rank = ranks ** (-s)
    p_rank /= p_rank.sum()
    perm = r.permutation(E)
    p = np.empty(E)
    p[perm] = p_rank
    return p


def gen_routing_zipf(r: np.random.Generator, S: int, K: int, E: int, s: float = 1.1):
    """ids int32 [S][K] by Gumbel-top-K on log p, w float32 [S][K]."""
    logp = np.log(zipf_popularity(r, E, s))
    g = r.gumbel(size=(S, E))
    ids = np.argsort(-(logp[None, :] + g), axis=1, kind="stable")[:, :K].astype(np.int32)
    w = _softmax_rows(r.standard_normal((S, K)))
    return ids, w


# ---------------------------------------------------------------------------
# Large pools drawn on the GPU (benchmark only)
# ---------------------------------------------------------------------------

def pool_on_device(seed: int, fmt: int, n: int, O: int, I: int, gs: int, device="cuda"):
    """Stack of n matrices drawn on the device with a seeded torch generator:
    codes uint8 [n][O][row_bytes], scales float32 [n][O][ng] (or [n][O])."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    rb = row_bytes(fmt, I)
    if fmt == 1:
        q = torch.randint(-127, 128, (n, O, rb), generator=g, device=device,
                          dtype=torch.int16).to(torch.int8).view(torch.uint8)
    else:
        q = torch.randint(0, 256, (n, O, rb), generator=g, device=device, dtype=torch.uint8)
    ng = n_groups(fmt, I, gs)
    shape = (n, O, ng) if fmt == 4 else (n, O)
    s = torch.empty(shape, device=device, dtype=torch.float32)
    s.uniform_(SCALE_LO, SCALE_HI, generator=g)
    return q, s


# ---------------------------------------------------------------------------
# Decode attention layer (MLA): weights, norm weights and prior cache rows
# ---------------------------------------------------------------------------

def gen_mla(r: np.random.Generator, D: int, qr: int, L: int, H: int, dn: int, dr: int, dv: int,
            gs: int = 64, T: int = 64, pos_base: int = 0):
    """Weights of one decode attention layer, all fmt 4 with group size gs:
    q_a [qr][D], q_b [H(dn+dr)][qr], kv_a [L+dr][D], kv_b [H(dn+dv)][L],
    o_proj [D][H dv] as (codes, scales); norm weights q_norm [qr], kv_norm [L]
    uniform in [0.5, 1.5]; caches Lc [T][L], Rc [T][dr] whose rows below
    pos_base hold N(0,1) draws (earlier tokens) and the rest zeros."""
    shapes = {"q_a": (qr, D), "q_b": (H * (dn + dr), qr), "kv_a": (L + dr, D),
              "kv_b": (H * (dn + dv), L), "o_proj": (D, H * dv)}
    mats = {k: gen_matrix(r, 4, o, i, gs) for k, (o, i) in shapes.items()}
    q_norm = r.uniform(0.5, 1.5, size=qr).astype(np.float32)
    kv_norm = r.uniform(0.5, 1.5, size=L).astype(np.float32)
    Lc = np.zeros((T, L), np.float32)
    Rc = np.zeros((T, dr), np.float32)
    Lc[:pos_base] = r.standard_normal((pos_base, L), dtype=np.float32)
    Rc[:pos_base] = r.standard_normal((pos_base, dr), dtype=np.float32)
    return mats, shapes, q_norm, kv_norm, Lc, Rc
