"""Planted mistakes in copies of the oracle must each trip at least one pin.

This shows the pins are sharp enough to catch the plausible slips (a dropped
term, a wrong index, a transposed operand, an off-by-one rule) in the oracle.
Everything here runs on the CPU."""

import functools
import math

import numpy as np
import pytest

import oracle
from oracle import attention as oa
from tests import pins


def _gather_with(row_fn):
    def impl(q, k, v, row_ptr, col_idx, block, scale, seq_len):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, H, L, d = q.shape
        nqb = L // block
        O = np.zeros((B, H, L, d))
        for b in range(B):
            for h in range(H):
                for qb in range(nqb):
                    r = h * nqb + qb
                    O[b, h, qb * block:(qb + 1) * block] = row_fn(
                        q[b, h], k[b, h], v[b, h], col_idx[row_ptr[r]:row_ptr[r + 1]], qb, block, scale, seq_len)
        return O
    return impl


def _row_generic(qs, ks, vs, kbs, qb, block, scale, seq_len, *, key_limit=None, norm=True,
                 scale_pow=1, zero_pad_rows=True):
    d = vs.shape[1]
    out = np.zeros((block, d))
    lo = qb * block
    hi = min(lo + block, seq_len) if zero_pad_rows else lo + block
    if hi <= lo:
        return out
    lim = seq_len if key_limit is None else key_limit
    J = [j for kb in kbs for j in range(kb * block, min((kb + 1) * block, lim))]
    if not J:
        return out
    s = (scale ** scale_pow) * (qs[lo:hi] @ ks[J].T)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    num = e @ vs[J]
    out[: hi - lo] = num / e.sum(axis=1, keepdims=True) if norm else num
    return out


ATTN_MUTANTS = {
    "padded_keys_in_softmax": _gather_with(lambda *a: _row_generic(*a, key_limit=10 ** 9)),
    "missing_denominator": _gather_with(lambda *a: _row_generic(*a, norm=False)),
    "scale_squared": _gather_with(lambda *a: _row_generic(*a, scale_pow=2)),
    "padded_rows_not_zero": _gather_with(lambda *a: _row_generic(*a, zero_pad_rows=False)),
}


def _transposed_mask(q, k, v, row_ptr, col_idx, block, scale, seq_len):
    B, H, L, d = np.shape(q)
    nqb = L // block
    bm = oracle.csr_to_block_mask(row_ptr, col_idx, H, nqb, nqb).transpose(0, 2, 1)
    return oracle.sparse_attention_masked_dense(q, k, v, bm, block, scale, seq_len)


ATTN_MUTANTS["transposed_block_mask"] = _transposed_mask

ATTN_PINS = [pins.pin_sparse_all_kept_is_sdpa, pins.pin_sparse_is_masked_sdpa, pins.pin_lone_valid_key,
             pins.pin_zero_query_is_mean, pins.pin_golden_attention]


def _trips(fn, pin_list):
    tripped = []
    for p in pin_list:
        try:
            p(fn)
        except (AssertionError, IndexError, ValueError):
            tripped.append(p.__name__)
    return tripped


@pytest.mark.parametrize("name", sorted(ATTN_MUTANTS))
def test_attention_mutant_is_caught(name):
    assert _trips(ATTN_MUTANTS[name], ATTN_PINS), f"no pin caught mutant {name}"


def _mass_generic(q, k, block, scale, seq_len, *, q_limit=None, transpose=False, normalise=True):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, L, d = q.shape
    nb = L // block
    out = np.zeros((B, H, nb, nb))
    ql = seq_len if q_limit is None else q_limit
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h, :ql] @ k[b, h, :seq_len].T)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True) if normalise else e
            for i in range(p.shape[0]):
                for j in range(p.shape[1]):
                    a, c = (j // block, i // block) if transpose else (i // block, j // block)
                    out[b, h, a, c] += p[i, j]
    return out


MASS_MUTANTS = {
    "padded_queries_pooled": lambda *a: _mass_generic(*a, q_limit=np.shape(a[0])[2]),
    "transposed_tile": lambda *a: _mass_generic(*a, transpose=True),
    "unnormalised_exp": lambda *a: _mass_generic(*a, normalise=False),
}
MASS_PINS = [pins.pin_mass_row_sums, pins.pin_mass_zero_query, pins.pin_mass_brute_force, pins.pin_mass_golden]


@pytest.mark.parametrize("name", sorted(MASS_MUTANTS))
def test_mass_mutant_is_caught(name):
    assert _trips(MASS_MUTANTS[name], MASS_PINS), f"no pin caught mutant {name}"


def _topk_generic(mass, K, nkb_valid=None, *, desc_index=False, ascending=False):
    mass = np.asarray(mass, dtype=np.float32)
    nv = mass.shape[-1] if nkb_valid is None else nkb_valid
    m = mass[..., :nv].astype(np.float64)
    idx = np.broadcast_to(np.arange(nv), m.shape)
    key = m if ascending else -m
    order = np.lexsort(((-idx if desc_index else idx), np.nan_to_num(key), np.isnan(m)), axis=-1)
    rank = np.empty(m.shape, dtype=np.int64)
    np.put_along_axis(rank, order, np.broadcast_to(np.arange(nv), m.shape), axis=-1)
    keep = np.zeros(mass.shape, dtype=bool)
    keep[..., :nv] = rank < K
    return keep


TOPK_MUTANTS = {
    "ties_by_larger_index": lambda *a: _topk_generic(*a, desc_index=True),
    "keeps_smallest": lambda *a: _topk_generic(*a, ascending=True),
}


@pytest.mark.parametrize("name", sorted(TOPK_MUTANTS))
def test_topk_mutant_is_caught(name):
    assert _trips(TOPK_MUTANTS[name], [pins.pin_topk_subsets, pins.pin_topk_counts])


def test_agreement_mutants_are_caught():
    strict = lambda keep, t: np.asarray(keep).sum(0) > t
    assert _trips(strict, [pins.pin_agreement_brute])
    floor = lambda rho, P: math.floor(float(rho) * P)
    assert _trips(floor, [pins.pin_min_agree])
    binary = lambda rho, P: math.ceil(__import__("fractions").Fraction(rho) * P)
    assert _trips(binary, [pins.pin_min_agree]), "binary reading of 0.1 must be caught"


def test_csr_and_schedule_mutants_are_caught():
    def desc_cols(mask):
        rp, ci = oracle.to_csr(mask)
        ci = ci.copy()
        for r in range(len(rp) - 1):
            ci[rp[r]:rp[r + 1]] = ci[rp[r]:rp[r + 1]][::-1]
        return rp, ci
    assert _trips(desc_cols, [pins.pin_csr])

    def shortest_first(row_ptr, H, nqb):
        o = oracle.lpt_work_order(row_ptr, H, nqb).copy()
        for i in range(0, H * nqb, nqb):
            o[i:i + nqb] = o[i:i + nqb][::-1]
        return o
    assert _trips(shortest_first, [pins.pin_lpt])

    def heads_in_index_order(row_ptr, H, nqb):
        from oracle import schedule as sc
        orig = sc.head_partitions
        sc.head_partitions = lambda rp, H_, n: [list(range(p, H_, 8)) for p in range(8)]
        try:
            return sc.lpt_work_order(row_ptr, H, nqb)
        finally:
            sc.head_partitions = orig
    assert _trips(heads_in_index_order, [pins.pin_lpt])


def _energy_generic(mass, eps, nkb_valid=None, *, mode="ok"):
    """Energy rule with a planted mistake (see ENERGY_MUTANTS)."""
    e = oracle.calibration.as_fraction(eps)
    num, den = e.numerator, e.denominator
    mass = np.asarray(mass, dtype=np.float32)
    nkb = mass.shape[-1]
    nv = nkb if nkb_valid is None else nkb_valid
    flat = mass.reshape(-1, nkb)
    keep = np.zeros(flat.shape, dtype=bool)
    fx_all = oracle.mass_fixed(flat[:, :nv])
    for r in range(flat.shape[0]):
        row = np.nan_to_num(flat[r, :nv].astype(np.float64), nan=-1.0)
        sign = 1.0 if mode == "ascending" else -1.0
        order = sorted(range(nv), key=lambda i: (sign * row[i], i))
        fx = [int(v) for v in fx_all[r]]
        total = sum(fx)
        before = 0
        for i in order:
            if mode == "excludes_crossing":
                ok = (before + fx[i]) * den <= (den - num) * total and fx[i] > 0
            elif mode == "le":
                ok = before * den <= (den - num) * total
            elif mode == "eps_is_kept_fraction":
                ok = before * den < num * total
            else:
                ok = before * den < (den - num) * total
            keep[r, i] = ok
            before += fx[i]
    return keep.reshape(mass.shape)


ENERGY_MUTANTS = {
    "excludes_crossing_block": lambda *a: _energy_generic(*a, mode="excludes_crossing"),
    "keeps_at_equality": lambda *a: _energy_generic(*a, mode="le"),
    "eps_is_kept_fraction": lambda *a: _energy_generic(*a, mode="eps_is_kept_fraction"),
    "ascending_order": lambda *a: _energy_generic(*a, mode="ascending"),
}


@pytest.mark.parametrize("name", sorted(ENERGY_MUTANTS))
def test_energy_mutant_is_caught(name):
    assert _trips(ENERGY_MUTANTS[name], [pins.pin_energy_golden, pins.pin_energy_brute, pins.pin_energy_special])


def test_energy_reference_passes_its_pins():
    """The mutant harness itself, run without a mistake, passes (so a trip means the mistake)."""
    ok = lambda *a: _energy_generic(*a, mode="ok")
    assert not _trips(ok, [pins.pin_energy_golden, pins.pin_energy_brute])


def _iou_kept_sets(kept, nkb_valid):
    """Mistake: IoU of the kept sets instead of the skipped sets."""
    valid = np.arange(np.asarray(kept).shape[-1]) < nkb_valid
    return oracle.iou_matrix(~np.asarray(kept, dtype=bool) & valid, nkb_valid)


def _iou_pooled(kept, nkb_valid):
    """Mistake: IoU pooled over heads instead of averaged."""
    s = oracle.skipped_sets(kept, nkb_valid)
    T = s.shape[0]
    out = np.ones((T, T))
    for a in range(T):
        for b in range(T):
            u = np.count_nonzero(s[a] | s[b])
            out[a, b] = 1.0 if u == 0 else np.count_nonzero(s[a] & s[b]) / u
    return out


def _cluster_chain(iou, tau):
    """Mistake: compare a timestep only with the one before it."""
    T = iou.shape[0]
    cl = np.zeros(T, dtype=np.int32)
    for t in range(1, T):
        cl[t] = cl[t - 1] + (0 if iou[t - 1, t] >= tau else 1)
    return cl


def _share_intersection(kept, tau, nkb_valid):
    """Mistake: a cluster keeps only what all members keep."""
    cl, shared, iou = oracle.share_timesteps(kept, tau, nkb_valid)
    kept = np.asarray(kept, dtype=bool)
    out = np.ones_like(shared)
    for t in range(len(cl)):
        out[cl[t]] &= kept[t]
    out[..., nkb_valid:] = False
    return cl, out, iou


def test_sharing_mutants_are_caught():
    assert _trips(_iou_kept_sets, [pins.pin_iou_brute])
    assert _trips(_iou_pooled, [pins.pin_iou_brute])
    assert _trips(_cluster_chain, [pins.pin_cluster_props])
    assert _trips(_share_intersection, [pins.pin_shared_union, pins.pin_sharing_golden])


def _merge_largest(iv, w):
    """Mistake: fill the largest gaps."""
    n = len(iv)
    if n <= w:
        return list(iv)
    gaps = [(-(iv[i + 1][0] - iv[i][1]), i) for i in range(n - 1)]
    fill = {i for _, i in sorted(gaps)[: n - w]}
    out = [list(iv[0])]
    for i in range(1, n):
        if i - 1 in fill:
            out[-1][1] = iv[i][1]
        else:
            out.append(list(iv[i]))
    return [tuple(x) for x in out]


def _merge_rightmost(iv, w):
    """Mistake: ties go to the rightmost gap."""
    n = len(iv)
    if n <= w:
        return list(iv)
    gaps = [(iv[i + 1][0] - iv[i][1], -i) for i in range(n - 1)]
    fill = {-j for _, j in sorted(gaps)[: n - w]}
    out = [list(iv[0])]
    for i in range(1, n):
        if i - 1 in fill:
            out[-1][1] = iv[i][1]
        else:
            out.append(list(iv[i]))
    return [tuple(x) for x in out]


def _pct_floor(widths, pct):
    """Mistake: floor instead of ceil for the rank."""
    w = sorted(int(x) for x in widths)
    k = max(1, math.floor(float(pct) * len(w) / 100))
    return w[k - 1]


def _intervals_inclusive(cols):
    """Mistake: closed runs [start, end]."""
    return [(a, b - 1) for a, b in oracle.row_intervals(cols)]


def test_interval_mutants_are_caught():
    g = lambda r=oracle.row_intervals, m=oracle.merge_row, p=oracle.width_percentile: (r, m, p)
    assert _trips(_merge_largest, [pins.pin_merge_props])
    assert _trips(_merge_rightmost, [pins.pin_merge_props])
    assert _trips(_pct_floor, [pins.pin_percentile_numpy])
    golden = lambda impls: pins.pin_intervals_golden(*impls)
    assert _trips((_intervals_inclusive, oracle.merge_row, oracle.width_percentile), [golden])
    assert _trips((oracle.row_intervals, _merge_rightmost, oracle.width_percentile), [golden])


# ---------------------------------------------------------------- spatial repetition

def _sim_generic(q, k, scale, seq_len, grid, *, lag=None, normalise=True, skip_last_frame=False):
    """Adjacent-row cosine with one planted mistake at a time."""
    q, k = (np.asarray(x, dtype=np.float64) for x in (q, k))
    B, H = q.shape[:2]
    F, R, C = grid
    lag = C if lag is None else lag
    top = [(f * R + y) * C + x for f in range(F - int(skip_last_frame)) for y in range(R - 1) for x in range(C)]
    top = np.array(top or [0])
    out = np.zeros((B, H))
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h, :seq_len] @ k[b, h, :seq_len].T)
            P = np.exp(s - s.max(1, keepdims=True))
            P /= P.sum(1, keepdims=True)
            a, c = P[top], P[np.minimum(top + lag, seq_len - 1)]
            num = (a * c).sum(1)
            out[b, h] = (num / np.sqrt((a * a).sum(1) * (c * c).sum(1)) if normalise else num).mean()
    return out


def _groups_first_row(rows, k):
    """Mistake: the first row of each group is its anchor."""
    return [(lo, hi, lo) for lo, hi, _ in oracle.row_groups(rows, k)]


def _groups_ceil(rows, k):
    """Mistake: equal groups of ceil(rows/k) rows, the last one short."""
    w = -(-rows // k)
    out = []
    for g in range(k):
        lo, hi = min(g * w, rows), min((g + 1) * w, rows)
        out.append((lo, hi, (lo + max(hi, lo + 1) - 1) // 2))
    return out


def _anchor_of_row_from(groups):
    def f(rows, k):
        a = np.zeros(rows, dtype=np.int64)
        for lo, hi, anc in groups(rows, k):
            a[lo:hi] = anc
        return a
    return f


def _anchor_attention_generic(q, k, v, scale, seq_len, grid, k_anchor, heads, *, keys_anchor_only=False,
                              ignore_frame=False):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, L, _ = q.shape
    F, R, C = grid
    arow = oracle.anchor_of_row(R, k_anchor)
    n = np.arange(seq_len)
    f, y, x = n // (R * C), (n // C) % R, n % C
    src = ((0 if ignore_frame else f) * R + arow[y]) * C + x
    anchors = oracle.anchor_tokens(grid, k_anchor)
    keys = anchors if keys_anchor_only else np.arange(seq_len)
    O = np.zeros((B, len(heads), L, v.shape[3]))
    for b in range(B):
        for i, h in enumerate(heads):
            s = scale * (q[b, h, anchors] @ k[b, h, keys].T)
            P = np.exp(s - s.max(1, keepdims=True))
            P /= P.sum(1, keepdims=True)
            out = np.zeros((L, v.shape[3]))
            out[anchors] = P @ v[b, h, keys]
            O[b, i, :seq_len] = out[src]
    return O


def _select_ge(sim, tau):
    """Mistake: a score equal to tau also selects."""
    return np.nonzero(np.asarray(sim, dtype=np.float64).mean(0) >= tau)[0]


def test_repetition_mutants_are_caught():
    sim_pins = [pins.pin_similarity_golden, pins.pin_similarity_special]
    assert _trips(functools.partial(_sim_generic, lag=1), sim_pins)
    assert _trips(functools.partial(_sim_generic, normalise=False), sim_pins)
    assert _trips(functools.partial(_sim_generic, skip_last_frame=True), sim_pins)
    for groups in (_groups_first_row, _groups_ceil):
        assert _trips(groups, [lambda g: pins.pin_row_groups(g, _anchor_of_row_from(g))])
    attn_pins = [pins.pin_anchor_broadcast, pins.pin_anchor_special]
    assert _trips(functools.partial(_anchor_attention_generic, keys_anchor_only=True), attn_pins)
    assert _trips(functools.partial(_anchor_attention_generic, ignore_frame=True), attn_pins)
    assert _trips(_select_ge, [pins.pin_select_golden])
