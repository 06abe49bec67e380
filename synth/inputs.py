"""Seeded Q/K/V draws.

Recipe (per tensor t in {Q=0, K=1, V=2}, batch b, head h):

1. ``x = N(0, 1)`` float32 draws of shape ``[L, d]`` from PCG64 seeded with
   ``SeedSequence([seed, t, b, h])``.  Each (tensor, batch, head) slab has its
   own stream, so any subset of heads can be regenerated alone and the slabs
   can be drawn in parallel threads.
2. For workloads with a token grid (frames F, rows Y, cols X), add a 3-D
   sinusoidal term: token n < S sits at frame ``n // (Y*X)``, row
   ``(n % (Y*X)) // X`` and column ``n % X``.  The channels split into three
   groups (frame | row | col) of sizes ``d - 2g | g | g`` with ``g`` = d//3
   rounded down to even (44 | 42 | 42 at d=128).  In a group of size G starting
   at channel o, channel ``o+2j`` holds ``sin(pos * w_j)`` and ``o+2j+1``
   holds ``cos(pos * w_j)`` with ``w_j = 10000 ** (-2j/G)``; amplitude 1.
   The same term is added to Q, K and V.
3. bfloat16 workloads round to nearest-even bfloat16.
4. Tokens n >= S are set to zero (padding).

Arrays are returned as float32 (bfloat16-exact for bfloat16 workloads).
"""

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

from .bf16 import round_bf16

_THREADS = max(1, min(16, os.cpu_count() or 1))


def positional_term(L, S, d, grid):
    """[L, d] float32 3-D sinusoidal term; zero for tokens >= S or without a grid."""
    pe = np.zeros((L, d), dtype=np.float64)
    if grid is None:
        return pe.astype(np.float32)
    F, Y, X = grid
    n = np.arange(min(S, F * Y * X))
    pos = [n // (Y * X), (n % (Y * X)) // X, n % X]
    g = (d // 3) // 2 * 2
    sizes = [d - 2 * g, g, g]
    off = 0
    for p, G in zip(pos, sizes):
        j = np.arange(G // 2)
        w = 10000.0 ** (-2.0 * j / G)
        ang = p[:, None].astype(np.float64) * w[None, :]
        pe[: len(n), off + 2 * j] = np.sin(ang)
        pe[: len(n), off + 2 * j + 1] = np.cos(ang)
        off += G
    return pe.astype(np.float32)


def _draw(seed, tid, b, h, L, d, out):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, b, h])))
    rng.standard_normal((L, d), dtype=np.float32, out=out)


def _gen(cfg, seed, tids, heads, B=None):
    B = cfg.B if B is None else B
    heads = list(range(cfg.H)) if heads is None else list(heads)
    pe = positional_term(cfg.L, cfg.S, cfg.d, cfg.grid)
    outs = [np.empty((B, len(heads), cfg.L, cfg.d), dtype=np.float32) for _ in tids]

    def work(item):
        i, b, j = item
        x = outs[i][b, j]
        _draw(seed, tids[i], b, heads[j], cfg.L, cfg.d, x)
        if cfg.grid is not None:
            x += pe
        if cfg.dtype == "bf16":
            x[...] = round_bf16(x)
        x[cfg.S:] = 0.0

    items = [(i, b, j) for i in range(len(tids)) for b in range(B) for j in range(len(heads))]
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(work, items))
    return outs


def gen_qkv(cfg, seed=None, heads=None, B=None):
    """Q, K, V float32 arrays [B, len(heads), L, d] for workload ``cfg``."""
    seed = cfg.data_seed if seed is None else seed
    q, k, v = _gen(cfg, seed, (0, 1, 2), heads, B)
    return q, k, v


def repeat_rows(x, grid, S, heads, mix, bf16=True):
    """Spatially repetitive heads: for the listed heads (indices into axis 1),
    token (f, y, x) becomes (1 - mix) * token (f, 0, x) + mix * itself, so its
    rows repeat down each frame up to a fraction ``mix`` of fresh draw.  In
    place; rounded back to bfloat16 when ``bf16``; tokens >= S untouched."""
    F, Y, X = grid
    for h in heads:
        v = x[:, h, :F * Y * X].reshape(x.shape[0], F, Y, X, x.shape[3])
        v[...] = (1.0 - mix) * v[:, :, :1] + mix * v
        if bf16:
            v[...] = round_bf16(v)
    return x


def gen_qk(cfg, seed, heads=None, B=None):
    """Q, K only (calibration prompts need no V)."""
    q, k = _gen(cfg, seed, (0, 1), heads, B)
    return q, k
