"""Property tests of the oracle (hypothesis, CPU only).

Random block masks (empty rows, single kept blocks, full rows), random
valid-length tails, and masses drawn from a handful of values (forced ties,
NaN) are checked against invariants that the pages and the mathematics fix,
never against a second copy of the same formula:

* attention over kept blocks (CalibAtt abstract, Fig. 5(b) caption): the
  gather and masked-dense forms agree; each output row is a convex
  combination of the kept valid values; it is linear in V; permuting the keys
  inside a kept block changes nothing; keeping every valid block is dense
  attention; rows with no kept valid key and padded rows are zero;
* pooled block mass (Fig. 2 and Table S5 captions): non-negative, every
  query block's row sums to its count of valid queries, padded key blocks
  hold nothing, equal keys spread mass in proportion to key counts;
* top-K (Fig. 5(a) caption) and the energy rule (Fig. S8 caption) under
  ties: the kept set is a prefix of the (mass desc, index asc, NaN last)
  order, of the right length or the shortest one reaching the target;
* agreement (Fig. 3(b) caption), CSR compile, skip lists (Fig. S10 caption),
  timestep sharing (Fig. S11, Table S3 captions), the work order and the
  repetition helpers (Fig. 5(b) caption): structural invariants.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle

SETTINGS = dict(deadline=None, derandomize=True, database=None, suppress_health_check=[HealthCheck.too_slow])


# --------------------------------------------------------------------------
# strategies
# --------------------------------------------------------------------------

@st.composite
def attn_case(draw):
    """Tiny attention problem: shapes, seeded values, a CSR mask with rows of
    every kind (empty, one block, full, random)."""
    block = draw(st.sampled_from([2, 4, 8]))
    nqb = draw(st.integers(1, 5))
    L = nqb * block
    S = draw(st.integers(1, L))
    H = draw(st.integers(1, 3))
    B = draw(st.integers(1, 2))
    d = draw(st.sampled_from([1, 3, 4]))
    seed = draw(st.integers(0, 2**31 - 1))
    nkb_valid = -(-S // block)
    rows = []
    for _ in range(H * nqb):
        kind = draw(st.sampled_from(["empty", "one", "full", "random", "beyond"]))
        if kind == "empty":
            rows.append([])
        elif kind == "one":
            rows.append([draw(st.integers(0, nqb - 1))])
        elif kind == "full":
            rows.append(list(range(nqb)))
        elif kind == "beyond":
            # only blocks at or past the valid length: no valid key unless S = L
            rows.append(list(range(nkb_valid, nqb)))
        else:
            rows.append(sorted(draw(st.sets(st.integers(0, nqb - 1), max_size=nqb))))
    rp = np.zeros(H * nqb + 1, dtype=np.int32)
    for r, c in enumerate(rows):
        rp[r + 1] = rp[r] + len(c)
    ci = np.array([c for row in rows for c in row], dtype=np.int32)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, L, d)) * 1.5
    k = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    scale = draw(st.sampled_from([0.25, 1.0, 2.0]))
    return dict(q=q, k=k, v=v, rp=rp, ci=ci, block=block, S=S, H=H, nqb=nqb, scale=scale, rows=rows)


def tie_masses(draw, shape, nan=True):
    """float32 masses drawn from a few values so that ties are common."""
    vals = [0.0, 0.25, 0.5, 1.0, 2.0, 3.0] + ([float("nan")] if nan else [])
    n = int(np.prod(shape))
    flat = draw(st.lists(st.sampled_from(vals), min_size=n, max_size=n))
    return np.array(flat, dtype=np.float32).reshape(shape)


def order_key(m, i):
    """The pages' reading of block order: NaN last, then mass descending, then index."""
    x = float(m[i])
    return (math.isnan(x), -(0.0 if math.isnan(x) else x), i)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

@settings(max_examples=60, **SETTINGS)
@given(attn_case())
def test_gather_equals_masked_dense(c):
    g = oracle.sparse_attention_gather(c["q"], c["k"], c["v"], c["rp"], c["ci"], c["block"], c["scale"], c["S"])
    bm = oracle.csr_to_block_mask(c["rp"], c["ci"], c["H"], c["nqb"], c["nqb"])
    m = oracle.sparse_attention_masked_dense(c["q"], c["k"], c["v"], bm, c["block"], c["scale"], c["S"])
    assert np.max(np.abs(g - m), initial=0.0) <= 1e-12


@settings(max_examples=60, **SETTINGS)
@given(attn_case())
def test_output_is_convex_combination_or_zero(c):
    q, k, v, block, S = c["q"], c["k"], c["v"], c["block"], c["S"]
    O = oracle.sparse_attention_gather(q, k, v, c["rp"], c["ci"], block, c["scale"], S)
    B, H, L, _ = q.shape
    nqb = c["nqb"]
    for h in range(H):
        for qb in range(nqb):
            J = [j for kb in c["rows"][h * nqb + qb] for j in range(kb * block, (kb + 1) * block) if j < S]
            for i in range(qb * block, (qb + 1) * block):
                for b in range(B):
                    if i >= S or not J:
                        assert np.all(O[b, h, i] == 0.0)
                    else:
                        lo, hi = v[b, h, J].min(axis=0), v[b, h, J].max(axis=0)
                        assert np.all(O[b, h, i] >= lo - 1e-12) and np.all(O[b, h, i] <= hi + 1e-12)


@settings(max_examples=40, **SETTINGS)
@given(attn_case(), st.floats(-3, 3, allow_nan=False), st.integers(0, 2**31 - 1))
def test_linear_in_values(c, a, seed):
    v2 = np.random.default_rng(seed).standard_normal(c["v"].shape)
    f = lambda vv: oracle.sparse_attention_gather(c["q"], c["k"], vv, c["rp"], c["ci"], c["block"], c["scale"], c["S"])
    lhs = f(c["v"] + a * v2)
    rhs = f(c["v"]) + a * f(v2)
    assert np.max(np.abs(lhs - rhs), initial=0.0) <= 1e-10


@settings(max_examples=40, **SETTINGS)
@given(attn_case(), st.integers(0, 2**31 - 1))
def test_key_permutation_inside_blocks(c, seed):
    """Softmax is a set function of the kept keys: permuting keys (with their
    values) inside each block leaves every output unchanged."""
    rng = np.random.default_rng(seed)
    block, L = c["block"], c["q"].shape[2]
    perm = np.concatenate([kb * block + rng.permutation(block) for kb in range(L // block)])
    # the block holding the valid-length boundary and those after it stay in place
    valid_tail = (c["S"] // block) * block
    for kb in range(valid_tail // block, L // block):
        perm[kb * block:(kb + 1) * block] = np.arange(kb * block, (kb + 1) * block)
    a = oracle.sparse_attention_gather(c["q"], c["k"], c["v"], c["rp"], c["ci"], block, c["scale"], c["S"])
    b = oracle.sparse_attention_gather(c["q"], c["k"][:, :, perm], c["v"][:, :, perm], c["rp"], c["ci"],
                                       block, c["scale"], c["S"])
    assert np.max(np.abs(a - b), initial=0.0) <= 1e-12


@settings(max_examples=40, **SETTINGS)
@given(attn_case())
def test_all_valid_blocks_is_dense(c):
    H, nqb, block, S = c["H"], c["nqb"], c["block"], c["S"]
    nv = -(-S // block)
    rp = (np.arange(H * nqb + 1) * nv).astype(np.int32)
    ci = np.tile(np.arange(nv), H * nqb).astype(np.int32)
    g = oracle.sparse_attention_gather(c["q"], c["k"], c["v"], rp, ci, block, c["scale"], S)
    d = oracle.dense_attention(c["q"], c["k"], c["v"], c["scale"], S)
    assert np.max(np.abs(g - d), initial=0.0) <= 1e-12


@settings(max_examples=40, **SETTINGS)
@given(attn_case(), st.data())
def test_rows_subset_matches_full(c, data):
    B, H, nqb = c["q"].shape[0], c["H"], c["nqb"]
    items = data.draw(st.lists(st.tuples(st.integers(0, B - 1), st.integers(0, H - 1),
                                         st.integers(0, nqb - 1)), min_size=1, max_size=6))
    full = oracle.sparse_attention_gather(c["q"], c["k"], c["v"], c["rp"], c["ci"], c["block"], c["scale"], c["S"])
    part = oracle.sparse_attention_rows(c["q"], c["k"], c["v"], c["rp"], c["ci"], c["block"], c["scale"], c["S"], items)
    blk = c["block"]
    for n, (b, h, qb) in enumerate(items):
        assert np.array_equal(part[n], full[b, h, qb * blk:(qb + 1) * blk])


# --------------------------------------------------------------------------
# pooled block mass
# --------------------------------------------------------------------------

@st.composite
def mass_case(draw):
    block = draw(st.sampled_from([2, 4, 8]))
    nb = draw(st.integers(1, 5))
    L = nb * block
    S = draw(st.integers(1, L))
    d = draw(st.sampled_from([1, 4]))
    seed = draw(st.integers(0, 2**31 - 1))
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 2, L, d)) * 2
    k = rng.standard_normal((1, 2, L, d))
    return q, k, block, S


@settings(max_examples=60, **SETTINGS)
@given(mass_case(), st.sampled_from([0.5, 1.0, 3.0]))
def test_mass_rows_sum_to_valid_queries(c, scale):
    q, k, block, S = c
    m = oracle.block_mass(q, k, block, scale, S)
    nb = q.shape[2] // block
    assert np.all(m >= 0.0)
    nv = -(-S // block)
    assert np.all(m[..., nv:] == 0.0)                     # padded key blocks hold no mass
    for qb in range(nb):
        valid_q = max(0, min((qb + 1) * block, S) - qb * block)
        assert np.allclose(m[:, :, qb].sum(axis=-1), valid_q, rtol=0, atol=1e-12)


@settings(max_examples=40, **SETTINGS)
@given(mass_case())
def test_mass_equal_keys_is_uniform(c):
    """All keys equal: every valid query spreads its probability evenly over the S keys."""
    q, k, block, S = c
    k = np.broadcast_to(k[:, :, :1], k.shape).copy()
    m = oracle.block_mass(q, k, block, 1.0, S)
    nb = q.shape[2] // block
    for qb in range(nb):
        vq = max(0, min((qb + 1) * block, S) - qb * block)
        for kb in range(nb):
            vk = max(0, min((kb + 1) * block, S) - kb * block)
            assert abs(m[0, 0, qb, kb] - vq * vk / S) <= 1e-12


# --------------------------------------------------------------------------
# top-K and energy rule under ties
# --------------------------------------------------------------------------

@st.composite
def tie_rows(draw, nan=True):
    nkb = draw(st.integers(1, 12))
    nv = draw(st.integers(1, nkb))
    rows = draw(st.integers(1, 4))
    return tie_masses(draw, (rows, nkb), nan), nv


@settings(max_examples=150, **SETTINGS)
@given(tie_rows(), st.integers(0, 14))
def test_topk_under_ties(c, K):
    mass, nv = c
    keep = oracle.topk_keep(mass, K, nv)
    for r in range(mass.shape[0]):
        assert not keep[r, nv:].any()
        kept = [i for i in range(nv) if keep[r, i]]
        dropped = [i for i in range(nv) if not keep[r, i]]
        assert len(kept) == min(K, nv)
        # every kept block precedes every dropped one in the total order
        if kept and dropped:
            assert max(order_key(mass[r], i) for i in kept) < min(order_key(mass[r], i) for i in dropped)


@settings(max_examples=150, **SETTINGS)
@given(tie_rows(), st.sampled_from(["0", "1/20", "1/10", "1/4", "1/3", "1/2", "9/10", "1"]))
def test_energy_prefix_under_ties(c, eps):
    mass, nv = c
    keep = oracle.energy_keep(mass, eps, nv)
    e = Fraction(eps)
    for r in range(mass.shape[0]):
        assert not keep[r, nv:].any()
        order = sorted(range(nv), key=lambda i: order_key(mass[r], i))
        flags = [bool(keep[r, i]) for i in order]
        n = sum(flags)
        assert flags == [True] * n + [False] * (nv - n)          # a prefix of the order
        fx = [Fraction(int(x), 2**40) for x in oracle.mass_fixed(mass[r, :nv])]
        total = sum(fx)
        target = (1 - e) * total
        got = sum(fx[i] for i in order[:n])
        if n < nv:
            assert got >= target                                  # the prefix reaches the target ...
        if n > 0:
            assert sum(fx[i] for i in order[:n - 1]) < target     # ... and is the shortest that does
        if total == 0:
            assert n == 0


@settings(max_examples=100, **SETTINGS)
@given(tie_rows(nan=False), st.sampled_from([("1/20", "1/10"), ("1/10", "1/4"), ("0", "1/2"), ("1/4", "1")]))
def test_energy_monotone_in_eps(c, pair):
    mass, nv = c
    small, large = pair
    a = oracle.energy_keep(mass, small, nv)
    b = oracle.energy_keep(mass, large, nv)
    assert np.all(b <= a)                       # a larger epsilon keeps a subset


@settings(max_examples=80, **SETTINGS)
@given(st.data())
def test_mass_fixed_exact_and_monotone(data):
    vals = data.draw(st.lists(st.floats(0, 200, allow_nan=False, width=32), min_size=2, max_size=8))
    x = np.sort(np.array(vals, dtype=np.float32))
    f = oracle.mass_fixed(x)
    assert np.all(np.diff(f) >= 0)
    for xi, fi in zip(x, f):
        exact = Fraction(float(min(xi, 128.0))) * 2**40
        assert abs(Fraction(int(fi)) - exact) <= Fraction(1, 2)


# --------------------------------------------------------------------------
# agreement and CSR
# --------------------------------------------------------------------------

@st.composite
def keep_stack(draw):
    P = draw(st.integers(1, 6))
    H = draw(st.integers(1, 3))
    nqb = draw(st.integers(1, 4))
    nkb = draw(st.integers(1, 6))
    bits = draw(st.lists(st.booleans(), min_size=P * H * nqb * nkb, max_size=P * H * nqb * nkb))
    return np.array(bits).reshape(P, H, nqb, nkb)


@settings(max_examples=100, **SETTINGS)
@given(keep_stack())
def test_agreement_monotone_and_bounds(keep):
    P = keep.shape[0]
    prev = None
    for t in range(P + 2):
        a = oracle.agreement(keep, t)
        if t == 0:
            assert a.all()
        if t == 1:
            assert np.array_equal(a, keep.any(axis=0))
        if t == P:
            assert np.array_equal(a, keep.all(axis=0))
        if t > P:
            assert not a.any()
        if prev is not None:
            assert np.all(a <= prev)
        prev = a


@settings(max_examples=100, **SETTINGS)
@given(keep_stack())
def test_csr_round_trip(keep):
    m = keep[0]
    H, nqb, nkb = m.shape
    rp, ci = oracle.to_csr(m)
    assert rp[0] == 0 and rp[-1] == len(ci) == m.sum()
    for r in range(H * nqb):
        row = ci[rp[r]:rp[r + 1]]
        assert np.all(np.diff(row) > 0)
    assert np.array_equal(oracle.csr_to_block_mask(rp, ci, H, nqb, nkb), m)


@settings(max_examples=100, **SETTINGS)
@given(st.fractions(0, 1), st.integers(1, 40))
def test_min_agree_count_is_ceiling(rho, P):
    m = oracle.min_agree_count(rho, P)
    assert 0 <= m <= P
    assert Fraction(m) >= rho * P > m - 1


@settings(max_examples=80, **SETTINGS)
@given(st.data())
def test_compile_masks_never_keeps_padding(data):
    P, H, nqb = data.draw(st.integers(1, 4)), data.draw(st.integers(1, 2)), data.draw(st.integers(1, 4))
    nkb = data.draw(st.integers(1, 8))
    nv = data.draw(st.integers(1, nkb))
    mass = tie_masses(data.draw, (P, H, nqb, nkb))
    for rp, ci in (oracle.compile_masks(mass, data.draw(st.integers(0, nkb)), 0, nv),
                   oracle.compile_masks_energy(mass, "1/10", 0, nv)):
        assert np.all(ci < nv)
        assert rp[-1] == H * nqb * nv                 # min_agree 0 keeps every valid block


# --------------------------------------------------------------------------
# skip lists
# --------------------------------------------------------------------------

@st.composite
def csr_sets(draw):
    T = draw(st.integers(1, 3))
    rows = draw(st.integers(1, 5))
    nkb = draw(st.integers(1, 16))
    sets = []
    for _ in range(T):
        rp, cols = [0], []
        for _ in range(rows):
            c = sorted(draw(st.sets(st.integers(0, nkb - 1), max_size=nkb)))
            cols.extend(c)
            rp.append(len(cols))
        sets.append((np.array(rp, dtype=np.int32), np.array(cols, dtype=np.int32)))
    return sets, rows, nkb


@settings(max_examples=120, **SETTINGS)
@given(csr_sets(), st.sampled_from([100, 99, 95, 90, 50, 25, 1]))
def test_skip_lists_merge_only_fills_gaps(c, pct):
    sets, rows, nkb = c
    T = len(sets)
    w, counts, pairs = oracle.encode_skip_lists(sets, rows, pct)
    dec = oracle.decode_skip_lists(counts, pairs, T, rows)
    for t in range(T):
        rp, ci = sets[t]
        drp, dci = dec[t]
        for r in range(rows):
            orig = set(ci[rp[r]:rp[r + 1]].tolist())
            got = dci[drp[r]:drp[r + 1]].tolist()
            e = t * rows + r
            assert got == sorted(set(got))                     # ascending, unique
            assert orig <= set(got)                             # merging only adds blocks
            assert counts[e] <= w
            n_orig = len(oracle.row_intervals(sorted(orig)))
            assert counts[e] == min(n_orig, max(w, 1)) or (n_orig == 0 and counts[e] == 0)
            if orig:
                assert min(got) == min(orig) and max(got) == max(orig)   # no block outside the row's span
            if pct == 100:
                assert set(got) == orig                          # plain trimming is lossless
            assert np.all(pairs[e, counts[e]:] == -1)


@settings(max_examples=100, **SETTINGS)
@given(st.integers(1, 64), st.data())
def test_interval_count_bound(nkb, data):
    """A row of nkb blocks holds at most ceil(nkb/2) maximal runs, reached by alternation."""
    cols = sorted(data.draw(st.sets(st.integers(0, nkb - 1), max_size=nkb)))
    iv = oracle.row_intervals(cols)
    assert len(iv) <= -(-nkb // 2)
    assert sum(b - a for a, b in iv) == len(cols)
    alt = list(range(0, nkb, 2))
    assert len(oracle.row_intervals(alt)) == -(-nkb // 2)


def test_fig_s9_maximum_within_the_bound():
    """Fig. S9 caption: the widest skip-list row at N = 75,600 has 295 intervals.
    With 128-token blocks that length spans ceil(75600/128) = 591 key blocks,
    whose most fragmented row has 296 runs, so 295 is attainable and a width
    of 295 needs at least 589 of the 591 blocks' positions."""
    nkb = -(-75600 // 128)
    assert nkb == 591
    assert len(oracle.row_intervals(list(range(0, nkb, 2)))) == 296
    cols = list(range(0, 2 * 295, 2))                      # 295 single-block runs
    assert len(oracle.row_intervals(cols)) == 295 and cols[-1] == 588


# --------------------------------------------------------------------------
# timestep sharing and the work order
# --------------------------------------------------------------------------

@settings(max_examples=80, **SETTINGS)
@given(keep_stack(), st.sampled_from([0.0, 0.3, 0.5, 0.8, 1.0]))
def test_sharing_invariants(kept, tau):
    nkb = kept.shape[-1]
    nv = max(1, nkb - 1)
    cluster, shared, iou = oracle.share_timesteps(kept, tau, nv)
    T = kept.shape[0]
    assert np.allclose(iou, iou.T) and np.all(np.diag(iou) == 1.0)
    assert np.all((iou >= 0) & (iou <= 1))
    assert cluster[0] == 0 and np.all(np.diff(cluster) >= 0) and np.all(np.diff(cluster) <= 1)
    for t in range(T):
        # every timestep computes at least its own valid kept blocks, never a padded one
        assert np.all(shared[cluster[t]][..., :nv] >= kept[t][..., :nv])
        assert not shared[cluster[t]][..., nv:].any()
    for c in range(int(cluster.max()) + 1):
        members = np.nonzero(cluster == c)[0]
        for a in members:
            for b in members:
                assert iou[a, b] >= tau
    if tau == 0.0:
        assert np.all(cluster == 0)


@settings(max_examples=80, **SETTINGS)
@given(st.integers(1, 20), st.integers(1, 6), st.data())
def test_work_order_is_balanced_permutation(H, nqb, data):
    counts = data.draw(st.lists(st.integers(0, 9), min_size=H * nqb, max_size=H * nqb))
    rp = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    wo = oracle.lpt_work_order(rp, H, nqb)
    rows = H * nqb
    order, offs = wo[:rows], wo[rows:]
    assert sorted(order.tolist()) == list(range(rows))
    assert len(offs) == 9 and offs[0] == 0 and offs[-1] == rows and np.all(np.diff(offs) >= 0)
    head_cost = [sum(counts[h * nqb:(h + 1) * nqb]) for h in range(H)]
    loads = []
    for p in range(8):
        seg = order[offs[p]:offs[p + 1]]
        heads = sorted({int(r) // nqb for r in seg})
        assert sum(len([r for r in seg if r // nqb == h]) for h in heads) == len(seg)
        for h in heads:                     # a head lives in one partition, whole
            assert np.count_nonzero(seg // nqb == h) == nqb
        loads.append(sum(head_cost[h] for h in heads))
    # greedy longest-first: the busiest partition exceeds the mean by at most one head
    assert max(loads) <= sum(head_cost) / 8 + max(head_cost)


# --------------------------------------------------------------------------
# spatial repetition
# --------------------------------------------------------------------------

@settings(max_examples=100, **SETTINGS)
@given(st.integers(1, 40), st.data())
def test_row_groups_partition(rows, data):
    k = data.draw(st.integers(1, rows))
    g = oracle.row_groups(rows, k)
    assert g[0][0] == 0 and g[-1][1] == rows
    for (lo, hi, a), nxt in zip(g, g[1:] + [(rows, None, None)]):
        assert lo < hi and lo <= a < hi and hi == nxt[0]
        assert (hi - lo) in (rows // k, -(-rows // k))
    a = oracle.anchor_of_row(rows, k)
    assert len(set(a.tolist())) == k
    assert all(a[y] == y for y in set(a.tolist()))           # an anchor row takes its own output


@settings(max_examples=30, **SETTINGS)
@given(st.integers(1, 3), st.integers(2, 5), st.integers(1, 4), st.integers(0, 2**31 - 1), st.data())
def test_anchor_attention_copies_anchor_rows(F, R, C, seed, data):
    k_anchor = data.draw(st.integers(1, R))
    S = F * R * C
    L = S + data.draw(st.integers(0, 3))
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((1, 2, L, 3)) for _ in range(3))
    O = oracle.anchor_attention(q, k, v, 0.7, S, (F, R, C), k_anchor, [1])
    D = oracle.dense_attention(q, k, v, 0.7, S)
    anc = oracle.anchor_of_row(R, k_anchor)
    for f in range(F):
        for y in range(R):
            for x in range(C):
                n, src = (f * R + y) * C + x, (f * R + anc[y]) * C + x
                assert np.max(np.abs(O[0, 0, n] - D[0, 1, src])) <= 1e-12
    assert np.all(O[0, 0, S:] == 0.0)


@settings(max_examples=30, **SETTINGS)
@given(st.integers(1, 2), st.integers(2, 4), st.integers(1, 4), st.integers(0, 2**31 - 1))
def test_similarity_range_and_repeated_rows(F, R, C, seed):
    S = F * R * C
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 2, S, 3))
    k = rng.standard_normal((1, 2, S, 3))
    # head 1: queries repeat down each column, so vertically adjacent rows are equal
    f, x = np.arange(S) // (R * C), np.arange(S) % C
    q[0, 1] = q[0, 1, f * R * C + x]
    sim = oracle.spatial_similarity(q, k, 1.0, S, (F, R, C))
    assert 0.0 < sim[0, 0] <= 1.0 + 1e-12
    assert abs(sim[0, 1] - 1.0) <= 1e-12


@settings(max_examples=100, **SETTINGS)
@given(st.integers(1, 5), st.integers(1, 6), st.data())
def test_select_heads_threshold(P, H, data):
    sim = np.array(data.draw(st.lists(st.sampled_from([0.5, 0.87, 0.875, 0.9, 1.0]),
                                      min_size=P * H, max_size=P * H))).reshape(P, H)
    tau = data.draw(st.sampled_from([0.5, 0.87, 0.9]))
    sel = oracle.select_repetitive_heads(sim, tau)
    assert np.all(np.diff(sel) > 0)
    mean = [sum(Fraction(float(sim[p, h])) for p in range(P)) / P for h in range(H)]
    for h in range(H):
        # the float64 mean rounds within 1 ulp per add; away from tau the decision is fixed
        if abs(mean[h] - Fraction(tau)) > Fraction(1, 10**9):
            assert (h in sel) == (mean[h] > Fraction(tau))
