"""Kept key-block lists (CSR) for the synthetic workloads.

A mask set is ``(row_ptr, col_idx)``: int32 arrays, row ``r = h * nqb + qb``
keeps the key blocks ``col_idx[row_ptr[r]:row_ptr[r+1]]`` (ascending, unique,
each below ceil(S / block)).  These are inputs to the attention calls; the
generators never derive them from attention scores.

Recipes (each per head h, random draws from PCG64 seeded with
``SeedSequence([mask_seed, set, h])``):

* tiny: the diagonal blocks plus exactly half of the off-diagonal blocks,
  chosen without replacement (one draw for the single head).
* wan: union of (i) a band |qb - kb| <= w_h, (ii) intra-frame blocks (the two
  blocks hold tokens of a common frame), (iii) same spatial position across
  frames (kb holds a token n' with n' = n mod frame_tokens for a token n of qb),
  (iv) Bernoulli(0.05) blocks.  w_h is the smallest width giving head density
  >= 0.30.  These are the diagonal, intra-frame and repeated spatial
  structures that the pages' attention-map figures show (Fig. 2, Fig. 4).
* mochi: band |qb - kb| <= 2 plus uniformly random blocks so that every row
  keeps exactly 26 of 128 blocks (20.3%).
* drifting timestep sets (drifting_sets): the Wan mask, then per step a
  shrinking fraction of each row's kept blocks swapped for others.
* imbalance: per head a density rho_h ~ U(0.05, 0.90); row r gets weight
  1 / (1 + pi(r)) for a random permutation pi (Zipf, s = 1); counts are
  rho_h * nqb * nkb split by weight, capped at nkb with the excess
  re-spread over the uncapped rows, rounded and clipped to [1, nkb]; each row
  keeps its diagonal block plus (count - 1) uniformly random other blocks.
"""

import numpy as np


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _pack_rows(rows):
    """List of per-row ascending block lists -> (row_ptr, col_idx) int32."""
    lens = np.array([len(r) for r in rows], dtype=np.int64)
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(lens)
    col_idx = (np.concatenate(rows) if rows else np.zeros(0)).astype(np.int32)
    return row_ptr.astype(np.int32), col_idx


def _lists(mask):
    """[H, nqb, nkb] bool generator output -> per-row lists of its set blocks."""
    H, nqb, nkb = mask.shape
    return [np.flatnonzero(row) for row in mask.reshape(H * nqb, nkb)]


def tiny_csr(cfg, set_index=0):
    nqb = cfg.nqb
    rng = _rng(cfg.mask_seed, set_index, 0)
    off = [(i, j) for i in range(nqb) for j in range(nqb) if i != j]
    pick = rng.choice(len(off), len(off) // 2, replace=False)
    m = np.eye(nqb, dtype=bool)
    for p in pick:
        m[off[p]] = True
    return _pack_rows(_lists(m[None].repeat(cfg.H, axis=0)))


def _block_token_ranges(cfg):
    lo = np.arange(cfg.nqb) * cfg.block
    hi = np.minimum(lo + cfg.block, cfg.S)
    return lo, hi


def _structure(cfg):
    """Intra-frame and same-spatial-position block masks [nqb, nkb] (head independent)."""
    F, Y, X = cfg.grid
    ft = Y * X
    lo, hi = _block_token_ranges(cfg)
    nb = cfg.nqb
    # frames touched by each block (valid tokens only)
    fr = np.zeros((nb, F), dtype=bool)
    pos = np.zeros((nb, ft), dtype=bool)
    for b in range(nb):
        if hi[b] <= lo[b]:
            continue
        t = np.arange(lo[b], hi[b])
        fr[b, np.unique(t // ft)] = True
        pos[b, t % ft] = True
    intra = (fr.astype(np.int32) @ fr.T.astype(np.int32)) > 0
    spatial = (pos.astype(np.int32) @ pos.T.astype(np.int32)) > 0
    return intra, spatial


def wan_csr(cfg, set_index=0, target=0.30):
    nqb, nkb = cfg.nqb, cfg.nkb
    intra, spatial = _structure(cfg)
    qb = np.arange(nqb)[:, None]
    kb = np.arange(nkb)[None, :]
    valid_k = kb < cfg.nkb_valid
    masks = np.zeros((cfg.H, nqb, nkb), dtype=bool)
    for h in range(cfg.H):
        rng = _rng(cfg.mask_seed, set_index, h)
        rand = rng.random((nqb, nkb)) < 0.05
        base = intra | spatial | rand
        for w in range(nkb):
            m = (base | (np.abs(qb - kb) <= w)) & valid_k
            if m.mean() >= target:
                break
        masks[h] = m
    return _pack_rows(_lists(masks))


def mochi_csr(cfg, set_index=0, per_row=26, band=2):
    nqb, nkb = cfg.nqb, cfg.nkb
    masks = np.zeros((cfg.H, nqb, nkb), dtype=bool)
    for h in range(cfg.H):
        rng = _rng(cfg.mask_seed, set_index, h)
        for q in range(nqb):
            row = np.zeros(nkb, dtype=bool)
            row[max(0, q - band): min(nkb, q + band + 1)] = True
            free = np.flatnonzero(~row)
            row[rng.choice(free, per_row - row.sum(), replace=False)] = True
            masks[h, q] = row
    return _pack_rows(_lists(masks))


def _zipf_counts(rng, rho, nqb, nkb):
    perm = rng.permutation(nqb)
    w = 1.0 / (1.0 + perm)
    c = rho * nqb * nkb * w / w.sum()
    capped = np.zeros(nqb, dtype=bool)
    for _ in range(nqb):
        over = (c > nkb) & ~capped
        if not over.any():
            break
        excess = float((c[over] - nkb).sum())
        c[over] = nkb
        capped |= over
        free = ~capped
        if not free.any():
            break
        c[free] += excess * w[free] / w[free].sum()
    return np.clip(np.rint(c), 1, nkb).astype(np.int64)


def imbalance_csr(cfg, set_index=0):
    nqb, nkb = cfg.nqb, cfg.nkb
    rows = []
    for h in range(cfg.H):
        rng = _rng(cfg.mask_seed, set_index, h)
        rho = rng.uniform(0.05, 0.90)
        counts = _zipf_counts(rng, rho, nqb, nkb)
        keys = rng.random((nqb, nkb))
        keys[np.arange(nqb), np.arange(nqb)] = -1.0      # the diagonal block always comes first
        order = np.argsort(keys, axis=1, kind="stable")
        for q in range(nqb):
            rows.append(np.sort(order[q, : counts[q]]))
    return _pack_rows(rows)


def random_csr(rng, H, nqb, nkb_valid, density, empty_rows=0, full_rows=0):
    """Bernoulli(density) kept blocks over kb < nkb_valid, for tests.

    ``empty_rows`` rows (chosen at random) keep nothing; ``full_rows`` keep all."""
    m = rng.random((H, nqb, nkb_valid)) < density
    flat = m.reshape(H * nqb, nkb_valid)
    if empty_rows or full_rows:
        pick = rng.choice(H * nqb, empty_rows + full_rows, replace=False)
        flat[pick[:empty_rows]] = False
        flat[pick[empty_rows:]] = True
    return _pack_rows(_lists(m))


def drifting_sets(cfg, T, drift=0.10):
    """T timestep mask sets at the Wan shape whose later steps are more alike.

    Set 0 is the Wan mask of ``cfg``.  Set t (t >= 1) takes set t-1 and, in
    every row, swaps round(f_t * n_row) kept non-diagonal blocks for as many
    blocks not kept, f_t = drift * (1 - t / T)^2 (row counts stay fixed): the
    structure of Fig. S11, where late denoising steps differ least.  Draws per
    (set, head) from PCG64 seeded with SeedSequence([mask_seed, 7000 + t, h])."""
    nqb, nkv = cfg.nqb, cfg.nkb_valid
    rp, ci = wan_csr(cfg, 0)
    kept = np.zeros((cfg.H, nqb, nkv), dtype=bool)
    for r in range(cfg.H * nqb):
        kept[r // nqb, r % nqb, ci[rp[r]:rp[r + 1]]] = True
    diag = np.zeros((nqb, nkv), dtype=bool)
    idx = np.arange(min(nqb, nkv))
    diag[idx, idx] = True
    sets = [(rp, ci)]
    for t in range(1, T):
        f = drift * (1.0 - t / T) ** 2
        nxt = kept.copy()
        for h in range(cfg.H):
            rng = _rng(cfg.mask_seed, 7000 + t, h)
            k = kept[h]
            n_swap = np.rint(f * k.sum(axis=1)).astype(np.int64)
            n_swap = np.minimum(n_swap, np.minimum((k & ~diag).sum(axis=1), (~k).sum(axis=1)))
            pri = np.where(k & ~diag, rng.random(k.shape), np.inf)
            rank = np.argsort(np.argsort(pri, axis=1), axis=1)
            drop = rank < n_swap[:, None]
            pri2 = np.where(~k, rng.random(k.shape), np.inf)
            rank2 = np.argsort(np.argsort(pri2, axis=1), axis=1)
            add = rank2 < n_swap[:, None]
            nxt[h] = (k & ~drop) | add
        kept = nxt
        sets.append(_pack_rows(_lists(kept)))
    return sets


def csr_for_config(cfg, set_index=0):
    if cfg.name == "tiny":
        return tiny_csr(cfg, set_index)
    if cfg.name == "wan":
        return wan_csr(cfg, set_index)
    if cfg.name == "wan720":
        return wan_csr(cfg, set_index, target=0.375)
    if cfg.name == "mochi":
        return mochi_csr(cfg, set_index)
    if cfg.name == "imbalance":
        return imbalance_csr(cfg, set_index)
    raise ValueError(f"workload {cfg.name!r} has no generated mask (calibration produces it)")
