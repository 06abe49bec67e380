"""Offline calibration: pooled mass, top key blocks, agreement, CSR (test infrastructure only).

Pages (CalibAtt, arXiv 2603.05503):
* Fig. 2 caption: post-softmax attention maps viewed at block granularity;
  Table S5 caption: "block energies" computed on the calibration prompts.
  Reading: the energy of tile (qb, kb) is the sum of the dense post-softmax
  probabilities over the tile's valid (query, key) pairs; the softmax runs
  over all valid keys (calibration sees the full map).
* Fig. 5(a) caption: the top key blocks of each query block are kept, per
  prompt, then the per-prompt masks are aggregated across prompts.
  Reading: a fixed count K per row; order by mass descending, ties broken by
  the smaller key-block index (any tie-break is valid for the method; this
  one makes the result unique).  NaN sorts last.  The decision is taken on
  float32 values, the precision in which the kernel stores the mass.
* Fig. 3(b) caption: each block's keep frequency across prompts, from 0
  (skipped for every prompt) to 1 (always kept), with an agreement
  threshold; Fig. 7 caption: agreement threshold rho.
  Reading: keep iff count >= ceil(rho * P), computed in exact rationals.
* Abstract: the kept patterns are compiled per layer, head and timestep.
  Encoding: CSR rows r = h * nqb + qb with ascending key-block indices.
* Fig. S8 caption: an energy threshold epsilon, scheduled over the
  normalised timestep, is the pages' own per-row rule; no formula or value
  survives in the text.  Reading: keep the shortest prefix of the row's
  (mass descending, index ascending, NaN last) order whose mass reaches
  (1 - epsilon) of the row's mass, i.e. block b is kept when the mass of the
  blocks before it is still short of that target.  Decided exactly: masses
  become integers in units of 2^-40 (round half to even, NaN and negative
  values 0, each capped at 128, the most a pooled 128-query row can hold)
  and epsilon is read as a decimal fraction.  The schedule over timesteps is
  the caller's: one epsilon per compile.
"""

from fractions import Fraction
import math

import numpy as np


def block_mass_rows(q_bh, k_bh, block, scale, seq_len, qb):
    """Pooled mass of one query block against every key block: [nkb] float64."""
    q_bh = np.asarray(q_bh, dtype=np.float64)
    k_bh = np.asarray(k_bh, dtype=np.float64)
    L = k_bh.shape[0]
    nkb = L // block
    mass = np.zeros(nkb, dtype=np.float64)
    lo, hi = qb * block, min((qb + 1) * block, seq_len)
    if hi <= lo:
        return mass
    s = scale * (q_bh[lo:hi] @ k_bh[:seq_len].T)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)               # dense post-softmax rows
    for kb in range(nkb):
        a, z = kb * block, min((kb + 1) * block, seq_len)
        if z > a:
            mass[kb] = p[:, a:z].sum()
    return mass


def block_mass(q, k, block, scale, seq_len):
    """[B, H, L, d] queries/keys -> mass [B, H, nqb, nkb] float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, L, d = q.shape
    nqb = L // block
    out = np.zeros((B, H, nqb, nqb), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for qb in range(nqb):
                out[b, h, qb] = block_mass_rows(q[b, h], k[b, h], block, scale, seq_len, qb)
    return out


def topk_keep(mass, K, nkb_valid=None):
    """Keep the K top key blocks of every row (last axis) by (mass desc, index asc).

    Only the first ``nkb_valid`` key blocks compete; later ones are never kept."""
    mass = np.asarray(mass, dtype=np.float32)
    nkb = mass.shape[-1]
    nv = nkb if nkb_valid is None else nkb_valid
    m = mass[..., :nv].astype(np.float64)              # exact widening of float32
    idx = np.broadcast_to(np.arange(nv), m.shape)
    order = np.lexsort((idx, -np.nan_to_num(m, nan=0.0), np.isnan(m)), axis=-1)
    rank = np.empty(m.shape, dtype=np.int64)
    np.put_along_axis(rank, order, np.broadcast_to(np.arange(nv), m.shape), axis=-1)
    keep = np.zeros(mass.shape, dtype=bool)
    keep[..., :nv] = rank < K
    return keep


MASS_UNIT_BITS = 40          # fixed point of block mass: 2^-40
MASS_CAP = 128.0             # a pooled row of 128 queries holds at most 128


def mass_fixed(mass):
    """float32 block mass -> integer multiples of 2^-40 (int64 array).

    NaN and negative values count 0; values are capped at MASS_CAP; rounding
    is to the nearest integer, halves to even.  m * 2^40 is exact in
    float64, and so is its rounding (below 2^53)."""
    m = np.asarray(mass, dtype=np.float32).astype(np.float64)
    m = np.where(np.isnan(m), 0.0, m)
    m = np.clip(m, 0.0, MASS_CAP)
    return np.rint(np.ldexp(m, MASS_UNIT_BITS)).astype(np.int64)


def as_fraction(x):
    """A threshold as an exact fraction; a float is read as the decimal it prints as."""
    if isinstance(x, float):
        x = str(x)
    return Fraction(x)


def energy_keep(mass, eps, nkb_valid=None):
    """Keep, per row (last axis), the shortest prefix of the (mass desc, index
    asc, NaN last) order whose mass reaches (1 - eps) of the row's mass.

    Block b is kept when the fixed-point mass of the blocks before it in that
    order, times the denominator of eps, is below (den - num) times the
    row's total: exact integer arithmetic.  Only the first ``nkb_valid``
    blocks take part."""
    e = as_fraction(eps)
    if not (0 <= e <= 1):
        raise ValueError("eps must lie in [0, 1]")
    num, den = e.numerator, e.denominator
    mass = np.asarray(mass, dtype=np.float32)
    nkb = mass.shape[-1]
    nv = nkb if nkb_valid is None else nkb_valid
    flat = mass.reshape(-1, nkb)
    keep = np.zeros(flat.shape, dtype=bool)
    fx_all = mass_fixed(flat[:, :nv])
    for r in range(flat.shape[0]):
        row = flat[r, :nv].astype(np.float64)
        order = sorted(range(nv), key=lambda i: (bool(np.isnan(row[i])),
                                                 -(0.0 if np.isnan(row[i]) else row[i]), i))
        fx = [int(v) for v in fx_all[r]]
        total = sum(fx)
        before = 0
        for i in order:
            if before * den < (den - num) * total:
                keep[r, i] = True
            before += fx[i]
    return keep.reshape(mass.shape)


def compile_masks_energy(mass, eps, min_agree, nkb_valid=None):
    """mass [P, H, nqb, nkb] -> CSR of the blocks that >= min_agree prompts keep
    under the energy rule with threshold eps (one epsilon per compile, the
    caller's schedule)."""
    keep = energy_keep(mass, eps, nkb_valid)
    agreed = agreement(keep, min_agree)
    if nkb_valid is not None:
        agreed[..., nkb_valid:] = False
    return to_csr(agreed)


def min_agree_count(rho, P):
    """Smallest prompt count meeting agreement fraction rho over P prompts: ceil(rho * P).

    A float rho is read as the decimal it prints as (0.1 -> 1/10), not as the
    binary value nearest to it."""
    if isinstance(rho, float):
        rho = str(rho)
    return math.ceil(Fraction(rho) * P)


def agreement(keep, min_agree):
    """keep [P, ...] bool -> blocks kept by at least min_agree prompts."""
    return np.asarray(keep, dtype=bool).sum(axis=0) >= min_agree


def to_csr(mask):
    """[H, nqb, nkb] bool -> (row_ptr, col_idx) int32; rows h*nqb+qb, columns ascending."""
    mask = np.asarray(mask, dtype=bool)
    H, nqb, nkb = mask.shape
    row_ptr = [0]
    cols = []
    for h in range(H):
        for qb in range(nqb):
            c = [kb for kb in range(nkb) if mask[h, qb, kb]]
            cols.extend(c)
            row_ptr.append(row_ptr[-1] + len(c))
    return np.array(row_ptr, dtype=np.int32), np.array(cols, dtype=np.int32)


def compile_masks(mass, keep_topk, min_agree, nkb_valid=None):
    """mass [P, H, nqb, nkb] -> CSR of the blocks that >= min_agree prompts keep in their top K.

    Key blocks at or past nkb_valid hold no valid key: they are never kept,
    whatever the agreement threshold (also when min_agree is 0)."""
    keep = topk_keep(mass, keep_topk, nkb_valid)
    agreed = agreement(keep, min_agree)
    if nkb_valid is not None:
        agreed[..., nkb_valid:] = False
    return to_csr(agreed)
