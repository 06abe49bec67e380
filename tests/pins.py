"""Pins for the CPU oracle: checks whose expected values do not come from the oracle.

Each ``pin_*`` takes the implementation under test (the oracle's function, or
a deliberately broken copy of it in ``test_oracle_mutants.py``) and raises
AssertionError when it disagrees with the fact the pin encodes:

* library routines on the special cases they cover (torch's
  scaled_dot_product_attention in float64 on the CPU; NumPy sorting),
* closed forms (Q = 0, a lone valid key, row sums of a softmax),
* brute-force enumeration on tiny inputs (all K-subsets, per-prompt counts),
* hand-worked values under ``tests/golden/``.
"""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_csr(rng, H, nqb, nkv, density, force_empty=1, force_full=1):
    m = rng.random((H, nqb, nkv)) < density
    flat = m.reshape(H * nqb, nkv)
    pick = rng.choice(H * nqb, force_empty + force_full, replace=False)
    flat[pick[:force_empty]] = False
    flat[pick[force_empty:]] = True
    row_ptr = np.concatenate([[0], np.cumsum(flat.sum(1))]).astype(np.int32)
    col_idx = np.nonzero(flat)[1].astype(np.int32)
    return m, row_ptr, col_idx


def _sdpa(q, k, v, scale, attn_mask=None):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    m = None if attn_mask is None else torch.from_numpy(attn_mask)
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=m, scale=scale).numpy()


# ---------------------------------------------------------------- attention

def pin_sparse_all_kept_is_sdpa(sparse_impl, seed=0):
    """Every block kept: sparse attention is ordinary attention over the valid keys."""
    rng = _rng(seed)
    B, H, L, S, d, blk = 2, 2, 96, 90, 8, 16
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    nqb = L // blk
    nkv = -(-S // blk)
    row_ptr = (np.arange(H * nqb + 1) * nkv).astype(np.int32)
    col_idx = np.tile(np.arange(nkv), H * nqb).astype(np.int32)
    scale = 0.37
    O = sparse_impl(q, k, v, row_ptr, col_idx, blk, scale, S)
    ref = _sdpa(q[:, :, :S], k[:, :, :S], v[:, :, :S], scale)
    assert np.max(np.abs(O[:, :, :S] - ref)) < 1e-12, "all-kept != SDPA"
    assert np.all(O[:, :, S:] == 0.0), "padded query rows must be zero"


def pin_sparse_is_masked_sdpa(sparse_impl, seed=1):
    """Skipping a block == giving its scores -inf (SDPA boolean mask), rows with keys."""
    rng = _rng(seed)
    B, H, L, S, d, blk = 1, 3, 128, 119, 8, 16
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    nqb = L // blk
    nkv = -(-S // blk)
    bm, row_ptr, col_idx = _rand_csr(rng, H, nqb, nkv, 0.4)
    O = sparse_impl(q, k, v, row_ptr, col_idx, blk, 0.5, S)
    for h in range(H):
        tok = np.zeros((L, L), dtype=bool)
        for qb in range(nqb):
            for kb in range(nkv):
                if bm[h, qb, kb]:
                    tok[qb * blk:(qb + 1) * blk, kb * blk:(kb + 1) * blk] = True
        tok[:, S:] = False
        tok = tok[:S, :S]
        has = tok.any(axis=1)
        ref = _sdpa(q[:, h:h + 1, :S][:, :, has], k[:, h:h + 1, :S], v[:, h:h + 1, :S], 0.5,
                    attn_mask=tok[has])
        got = O[:, h:h + 1, :S][:, :, has]
        assert np.max(np.abs(got - ref)) < 1e-12, "masked attention != SDPA with -inf mask"
        assert np.all(O[:, h, :S][:, ~has] == 0.0), "rows with no kept key must be zero"
        assert np.all(O[:, h, S:] == 0.0), "padded query rows must be zero"


def pin_lone_valid_key(sparse_impl):
    """S=449, block 64: the last block holds one valid token, so a row keeping only it
    returns that token's value row exactly."""
    rng = _rng(2)
    B, H, L, S, d, blk = 1, 1, 512, 449, 8, 64
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    nqb = L // blk
    row_ptr = np.arange(nqb + 1).astype(np.int32)
    col_idx = np.full(nqb, 7, dtype=np.int32)
    O = sparse_impl(q, k, v, row_ptr, col_idx, blk, 0.125, S)
    assert np.array_equal(O[0, 0, :S], np.broadcast_to(v[0, 0, 448], (S, d))), "lone key"


def pin_zero_query_is_mean(sparse_impl):
    """Q = 0: every kept valid key gets the same weight, O is the mean of those V rows."""
    rng = _rng(3)
    B, H, L, S, d, blk = 1, 2, 64, 60, 4, 16
    k, v = (rng.standard_normal((B, H, L, d)) for _ in range(2))
    q = np.zeros((B, H, L, d))
    nqb = L // blk
    bm, row_ptr, col_idx = _rand_csr(rng, H, nqb, nqb, 0.5, force_empty=0)
    O = sparse_impl(q, k, v, row_ptr, col_idx, blk, 1.0, S)
    for h in range(H):
        for qb in range(nqb):
            toks = [j for kb in range(nqb) if bm[h, qb, kb] for j in range(kb * blk, (kb + 1) * blk) if j < S]
            lo, hi = qb * blk, min((qb + 1) * blk, S)
            if not toks or hi <= lo:
                continue
            mean = v[0, h, toks].mean(axis=0)
            assert np.max(np.abs(O[0, h, lo:hi] - mean)) < 1e-13, "Q=0 must give the kept mean"


def pin_golden_attention(sparse_impl):
    """Hand-worked 4-token example (tests/golden/hand_attention.json)."""
    g = json.load(open(os.path.join(GOLDEN, "hand_attention.json")))
    q = np.array(g["q"], dtype=np.float64)[None, None]
    k = np.array(g["k"], dtype=np.float64)[None, None]
    v = np.array(g["v"], dtype=np.float64)[None, None]
    for case in g["cases"]:
        O = sparse_impl(q, k, v, np.array(case["row_ptr"], np.int32), np.array(case["col_idx"], np.int32),
                        g["block"], g["scale"], g["seq_len"])
        exp = np.array([[float(Fraction(x)) for x in row] for row in case["O"]])
        assert np.max(np.abs(O[0, 0] - exp)) < 1e-14, f"golden case {case['name']}"


def pin_dense_is_sdpa(dense_impl, seed=4):
    rng = _rng(seed)
    B, H, L, S, d = 1, 2, 40, 37, 6
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    O = dense_impl(q, k, v, 0.3, S)
    ref = _sdpa(q[:, :, :S], k[:, :, :S], v[:, :, :S], 0.3)
    assert np.max(np.abs(O[:, :, :S] - ref)) < 1e-12, "dense != SDPA"
    assert np.all(O[:, :, S:] == 0.0)


# ---------------------------------------------------------------- calibration

def pin_mass_row_sums(mass_impl, seed=5):
    """Each valid query's softmax row sums to 1: row sums = valid queries, total = S."""
    rng = _rng(seed)
    B, H, L, S, d, blk = 1, 2, 96, 83, 8, 16
    q, k = (rng.standard_normal((B, H, L, d)) for _ in range(2))
    m = mass_impl(q, k, blk, 0.4, S)
    nqb = L // blk
    for qb in range(nqb):
        nvalid = max(0, min((qb + 1) * blk, S) - qb * blk)
        assert np.max(np.abs(m[:, :, qb].sum(-1) - nvalid)) < 1e-11, "row sum != valid queries"
    assert np.max(np.abs(m.sum(axis=(-1, -2)) - S)) < 1e-10, "total mass != S"
    assert np.all(m >= 0.0)


def pin_mass_zero_query(mass_impl):
    """Q = 0: uniform softmax over S keys, tile mass = nq_valid * nk_valid / S."""
    rng = _rng(6)
    B, H, L, S, d, blk = 1, 1, 80, 75, 4, 16
    k = rng.standard_normal((B, H, L, d))
    q = np.zeros_like(k)
    m = mass_impl(q, k, blk, 1.0, S)
    nb = L // blk
    nv = [max(0, min((b + 1) * blk, S) - b * blk) for b in range(nb)]
    exp = np.array([[nv[a] * nv[b] / S for b in range(nb)] for a in range(nb)])
    assert np.max(np.abs(m[0, 0] - exp)) < 1e-13, "Q=0 closed form"


def pin_mass_brute_force(mass_impl):
    """Per-token softmax with math.exp loops on a tiny input."""
    rng = _rng(7)
    B, H, L, S, d, blk = 1, 1, 12, 11, 3, 4
    q, k = (rng.standard_normal((B, H, L, d)) for _ in range(2))
    sc = 0.9
    m = mass_impl(q, k, blk, sc, S)
    nb = L // blk
    exp = [[0.0] * nb for _ in range(nb)]
    for i in range(S):
        w = [math.exp(sc * sum(q[0, 0, i, c] * k[0, 0, j, c] for c in range(d))) for j in range(S)]
        z = sum(w)
        for j in range(S):
            exp[i // blk][j // blk] += w[j] / z
    assert np.max(np.abs(m[0, 0] - np.array(exp))) < 1e-13, "brute-force mass"


def pin_mass_golden(mass_impl):
    g = json.load(open(os.path.join(GOLDEN, "hand_attention.json")))
    q = np.array(g["q"], dtype=np.float64)[None, None]
    k = np.array(g["k"], dtype=np.float64)[None, None]
    m = mass_impl(q, k, g["block"], g["scale"], g["seq_len"])
    exp = np.array([[float(Fraction(x)) for x in row] for row in g["mass"]])
    assert np.max(np.abs(m[0, 0] - exp)) < 1e-14, "golden mass"


def pin_topk_subsets(topk_impl, seed=8):
    """nkb = 8, K = 2: the kept pair is the lexicographically first of the max-sum pairs."""
    rng = _rng(seed)
    rows = rng.integers(0, 4, size=(300, 8)).astype(np.float32)   # many ties
    rows[::7] = rng.random((len(rows[::7]), 8)).astype(np.float32)
    keep = topk_impl(rows, 2)
    for r, row in enumerate(rows):
        best = max(itertools.combinations(range(8), 2),
                   key=lambda s: (float(row[s[0]]) + float(row[s[1]]), [-i for i in s]))
        want = np.zeros(8, dtype=bool)
        want[list(best)] = True
        assert np.array_equal(keep[r], want), f"top-2 row {r}: {row} -> {keep[r]}, want {best}"


def pin_topk_counts(topk_impl, seed=9):
    """Exactly min(K, nkb_valid) kept per row; nothing at or beyond nkb_valid; NaN last."""
    rng = _rng(seed)
    m = rng.random((5, 7, 20)).astype(np.float32)
    m[0, 0, 3] = np.nan
    for K in (0, 1, 5, 17, 20, 25):
        keep = topk_impl(m, K, 17)
        assert np.all(keep.sum(-1) == min(K, 17)), "count per row"
        assert not keep[..., 17:].any(), "blocks past the valid range"
    keep = topk_impl(m, 16, 17)
    assert not keep[0, 0, 3], "NaN must sort last"
    # order-statistic check against a full NumPy sort on distinct values
    x = rng.permutation(1000).astype(np.float32).reshape(10, 100)
    keep = topk_impl(x, 10)
    thr = np.sort(x, axis=1)[:, -10][:, None]
    assert np.array_equal(keep, x >= thr), "top-K != sort threshold"


def pin_agreement_brute(agree_impl, seed=10):
    rng = _rng(seed)
    keep = rng.random((5, 3, 4, 6)) < 0.5
    for t in range(0, 7):
        got = agree_impl(keep, t)
        for idx in itertools.product(range(3), range(4), range(6)):
            cnt = sum(int(keep[(p,) + idx]) for p in range(5))
            assert bool(got[idx]) == (cnt >= t), "agreement count"
    assert np.array_equal(agree_impl(keep[:1], 1), keep[0]), "P = 1 is the identity"
    assert np.array_equal(agree_impl(keep, 5), keep.all(0)), "min_agree = P is the intersection"
    assert np.array_equal(agree_impl(keep, 1), keep.any(0)), "min_agree = 1 is the union"


def pin_min_agree(min_agree_impl):
    assert min_agree_impl(0.5, 8) == 4
    assert min_agree_impl(Fraction(1, 2), 7) == 4
    assert min_agree_impl(Fraction(1, 3), 3) == 1
    assert min_agree_impl(0.1, 10) == 1
    assert min_agree_impl(1.0, 8) == 8
    assert min_agree_impl(0.0, 8) == 0
    for P in range(1, 65):
        for num in range(0, P + 1):
            rho = Fraction(num, P)
            assert min_agree_impl(rho, P) == num, "exact fractions"


def pin_csr(to_csr_impl, seed=11):
    rng = _rng(seed)
    m = rng.random((3, 5, 7)) < 0.4
    m[1, 2] = False
    row_ptr, col_idx = to_csr_impl(m)
    assert row_ptr.dtype == np.int32 and col_idx.dtype == np.int32
    assert row_ptr[0] == 0 and row_ptr[-1] == m.sum() and len(row_ptr) == 16
    assert np.all(np.diff(row_ptr) >= 0)
    back = np.zeros_like(m)
    for r in range(15):
        c = col_idx[row_ptr[r]:row_ptr[r + 1]]
        assert np.all(np.diff(c) > 0), "ascending, unique"
        back[r // 5, r % 5, c] = True
    assert np.array_equal(back, m), "round trip"


def pin_compile_brute(compile_impl, seed=12):
    """Whole compile on a tiny bank of prompts, every step done by enumeration.

    Covers a key range shorter than the mass (nkb_valid < nkb) and the
    thresholds 0 (every eligible block), 1 (union) and P (intersection)."""
    rng = _rng(seed)
    P, H, nqb, nkb, K = 4, 2, 3, 6, 2
    mass = rng.integers(0, 3, size=(P, H, nqb, nkb)).astype(np.float32)
    for nv in (6, 5):
        for t in (0, 1, 2, 4):
            row_ptr, col_idx = compile_impl(mass, K, t, nv)
            want_rows = []
            for h in range(H):
                for qb in range(nqb):
                    cnt = [0] * nkb
                    for p in range(P):
                        row = mass[p, h, qb]
                        best = max(itertools.combinations(range(nv), K),
                                   key=lambda s: (sum(float(row[i]) for i in s), [-i for i in s]))
                        for i in best:
                            cnt[i] += 1
                    want_rows.append([kb for kb in range(nv) if cnt[kb] >= t])
            got_rows = [list(col_idx[row_ptr[r]:row_ptr[r + 1]]) for r in range(H * nqb)]
            assert got_rows == want_rows, f"compile by enumeration (nkb_valid={nv}, min_agree={t})"


# ---------------------------------------------------------------- schedule

def pin_lpt(lpt_impl, seed=13):
    rng = _rng(seed)
    H, nqb = 11, 9
    counts = rng.integers(0, 5, size=H * nqb)
    row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    out = lpt_impl(row_ptr, H, nqb)
    rows = H * nqb
    order, off = out[:rows], out[rows:]
    assert len(out) == rows + 9 and off[0] == 0 and off[-1] == rows and np.all(np.diff(off) >= 0)
    assert sorted(order.tolist()) == list(range(rows)), "a permutation"
    for p in range(8):
        seg = order[off[p]:off[p + 1]]
        assert len(seg) % nqb == 0, "whole heads per partition"
        for i in range(0, len(seg), nqb):
            hs = seg[i:i + nqb]
            assert np.all(hs // nqb == hs[0] // nqb), "a head's rows are contiguous"
            c = counts[hs]
            for a in range(nqb - 1):
                assert c[a] > c[a + 1] or (c[a] == c[a + 1] and hs[a] < hs[a + 1]), "longest first, ties by index"
    # hand-worked greedy: 9 heads of one row with costs 9..1 over 8 partitions:
    # heads 0..7 (costs 9..2) open partitions 0..7, head 8 (cost 1) joins the
    # lightest, partition 7 (cost 2), after head 7.
    rp = np.concatenate([[0], np.cumsum(np.arange(9, 0, -1))]).astype(np.int32)
    out = lpt_impl(rp, 9, 1)
    assert out[:9].tolist() == [0, 1, 2, 3, 4, 5, 6, 7, 8]
    assert out[9:].tolist() == [0, 1, 2, 3, 4, 5, 6, 7, 9]
    # equal heads spread evenly, then by index: 16 equal heads -> two per partition
    rp = (np.arange(17) * 3).astype(np.int32)
    out = lpt_impl(rp, 16, 1)
    assert out[:16].tolist() == [0, 8, 1, 9, 2, 10, 3, 11, 4, 12, 5, 13, 6, 14, 7, 15]
    assert out[16:].tolist() == [0, 2, 4, 6, 8, 10, 12, 14, 16]


def _load_golden(name):
    import json, os
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        return json.load(f)


def pin_mass_fixed(fixed_impl):
    """Block mass in units of 2^-40: exact for dyadic values, round half to even, NaN/negative 0, cap 128."""
    got = fixed_impl(np.array([0.5, 0.25, 1.0, 128.0, 200.0, -1.0, np.nan, 0.0], np.float32))
    want = [2 ** 39, 2 ** 38, 2 ** 40, 2 ** 47, 2 ** 47, 0, 0, 0]
    assert [int(x) for x in got] == want, "fixed point of exact values"
    x = np.float32(0.1)
    exact = Fraction(float(x)) * 2 ** 40                    # float32 0.1 as a fraction
    assert int(fixed_impl(np.array([x]))[0]) == round(exact), "nearest multiple of 2^-40"
    tiny = np.float32(2.0 ** -41)                            # exactly half a unit: ties to even (0)
    assert int(fixed_impl(np.array([tiny]))[0]) == 0
    assert int(fixed_impl(np.array([np.float32(3 * 2.0 ** -41)]))[0]) == 2, "1.5 units -> 2"


def pin_energy_golden(energy_impl):
    for case in _load_golden("energy_rule.json")["cases"]:
        m = np.array([case["mass"]], np.float32)
        got = energy_impl(m, Fraction(case["eps"]))[0].astype(int).tolist()
        assert got == case["keep"], f"energy rule {case['mass']} eps {case['eps']}: {got}"


def pin_energy_brute(energy_impl, seed=14):
    """The kept count is the smallest k for which some k blocks hold (1 - eps) of the
    row's mass; the kept set is the lexicographically first heaviest such k-set."""
    rng = _rng(seed)
    for trial in range(250):
        nkb = int(rng.integers(1, 8))
        row = (rng.integers(0, 5, size=nkb) / 8.0).astype(np.float32)   # dyadic, many ties
        eps = Fraction(int(rng.integers(0, 9)), 8)
        total = sum(Fraction(float(v)) for v in row)
        target = (1 - eps) * total
        want = np.zeros(nkb, dtype=bool)
        for k in range(0, nkb + 1):
            best = max(itertools.combinations(range(nkb), k),
                       key=lambda s: (sum(Fraction(float(row[i])) for i in s), [-i for i in s]))
            if sum(Fraction(float(row[i])) for i in best) >= target:
                want[list(best)] = True
                break
        if total == 0:
            want[:] = False                       # nothing is short of a zero target
        got = energy_impl(row[None, :], eps)[0]
        assert np.array_equal(got, want), f"row {row} eps {eps}: {got} vs {want}"


def pin_energy_special(energy_impl, seed=15):
    rng = _rng(seed)
    m = rng.random((6, 12)).astype(np.float32)
    m[0, 3] = np.nan
    m[1] = 0.0
    m[2, :4] = 0.0
    assert np.array_equal(energy_impl(m, 0), (np.nan_to_num(m) > 0)), "eps 0 keeps every block with mass"
    assert not energy_impl(m, 1).any(), "eps 1 keeps nothing"
    assert not energy_impl(m, Fraction(1, 7))[0, 3], "NaN is never kept"
    assert not energy_impl(m, Fraction(1, 3))[1].any(), "an empty row keeps nothing"
    k9 = energy_impl(m, Fraction(1, 3), 9)
    assert not k9[:, 9:].any(), "nothing past nkb_valid"
    prev = None
    for e in [Fraction(i, 10) for i in range(11)]:
        cur = energy_impl(m, e)
        if prev is not None:
            assert not (cur & ~prev).any(), "a larger eps keeps a subset"
        prev = cur


def pin_compile_energy_brute(compile_impl, seed=16):
    """Energy compile on a tiny bank: per-prompt sets by enumeration, then the count rule."""
    rng = _rng(seed)
    P, H, nqb, nkb = 3, 2, 2, 5
    mass = (rng.integers(0, 4, size=(P, H, nqb, nkb)) / 4.0).astype(np.float32)
    for nv in (5, 4):
        for eps in (Fraction(0), Fraction(1, 4), Fraction(1, 2)):
            for t in (0, 1, 2, 3):
                row_ptr, col_idx = compile_impl(mass, eps, t, nv)
                want_rows = []
                for h in range(H):
                    for qb in range(nqb):
                        cnt = [0] * nkb
                        for p in range(P):
                            row = mass[p, h, qb, :nv]
                            total = sum(Fraction(float(v)) for v in row)
                            for k in range(0, nv + 1):
                                best = max(itertools.combinations(range(nv), k),
                                           key=lambda s: (sum(Fraction(float(row[i])) for i in s), [-i for i in s]))
                                if sum(Fraction(float(row[i])) for i in best) >= (1 - eps) * total:
                                    break
                            if total == 0:
                                best = ()
                            for i in best:
                                cnt[i] += 1
                        want_rows.append([kb for kb in range(nv) if cnt[kb] >= t])
                got = [list(col_idx[row_ptr[r]:row_ptr[r + 1]]) for r in range(H * nqb)]
                assert got == want_rows, f"energy compile (nkb_valid={nv}, eps={eps}, min_agree={t})"


def _golden_sharing():
    g = _load_golden("timestep_sharing.json")
    T = len(g["kept_head0"])
    kept = np.zeros((T, 2, 1, 4), dtype=bool)
    for t, ks in enumerate(g["kept_head0"]):
        kept[t, 0, 0, ks] = True
    kept[:, 1] = True
    return g, kept


def pin_sharing_golden(share_impl):
    """share_impl(kept, tau, nkb_valid) -> (clusters, shared, iou)."""
    g, kept = _golden_sharing()
    for case in g["cases"]:
        tau = float(Fraction(case["tau"]))
        clusters, shared, iou = share_impl(kept, tau, 4)
        want_iou = np.array([[float(Fraction(x)) for x in row] for row in g["iou_mean"]])
        assert np.max(np.abs(np.asarray(iou) - want_iou)) < 1e-15, "golden IoU"
        assert list(np.asarray(clusters)) == case["clusters"], f"clusters at tau {case['tau']}"
        got = [sorted(np.nonzero(shared[c, 0, 0])[0].tolist()) for c in range(len(shared))]
        assert got == case["shared_head0"], f"shared masks at tau {case['tau']}"
        assert np.asarray(shared)[:, 1].all(), "head 1 keeps everything"


def pin_iou_brute(iou_impl, seed=17):
    """Mean-over-heads IoU of skipped sets by Python sets and exact fractions."""
    rng = _rng(seed)
    for trial in range(20):
        T, H, nqb, nkb = int(rng.integers(1, 5)), int(rng.integers(1, 4)), 2, 6
        nv = int(rng.integers(1, nkb + 1))
        kept = rng.random((T, H, nqb, nkb)) < rng.random()
        got = np.asarray(iou_impl(kept, nv))
        for t1 in range(T):
            for t2 in range(T):
                acc = Fraction(0)
                for h in range(H):
                    s1 = {(q, k) for q in range(nqb) for k in range(nv) if not kept[t1, h, q, k]}
                    s2 = {(q, k) for q in range(nqb) for k in range(nv) if not kept[t2, h, q, k]}
                    acc += Fraction(1) if not (s1 | s2) else Fraction(len(s1 & s2), len(s1 | s2))
                assert abs(got[t1, t2] - float(acc / H)) < 1e-12, "IoU by sets"
        assert np.allclose(got, got.T) and np.all(np.diag(got) == 1.0)


def pin_cluster_props(cluster_impl, seed=18):
    """Runs of consecutive timesteps; every pair inside a run reaches tau; a run
    starts only where some member of the previous run falls below tau."""
    rng = _rng(seed)
    for trial in range(60):
        T = int(rng.integers(1, 12))
        a = rng.random((T, T))
        iou = (a + a.T) / 2
        np.fill_diagonal(iou, 1.0)
        tau = float(rng.random())
        cl = np.asarray(cluster_impl(iou, tau))
        assert cl[0] == 0 and np.all(np.diff(cl) >= 0) and np.all(np.diff(cl) <= 1), "consecutive runs"
        for c in range(int(cl.max()) + 1):
            mem = np.nonzero(cl == c)[0]
            for i in mem:
                for j in mem:
                    assert iou[i, j] >= tau or i == j, "pair below tau inside a run"
            if c > 0:
                prev = np.nonzero(cl == c - 1)[0]
                assert any(iou[u, mem[0]] < tau for u in prev), "run split without cause"
        assert np.all(np.asarray(cluster_impl(iou, 0.0)) == 0), "tau 0: one run"
        assert np.array_equal(np.asarray(cluster_impl(iou, 1.5)), np.arange(T)), "tau > 1: every step alone"


def pin_shared_union(share_impl, seed=19):
    rng = _rng(seed)
    kept = rng.random((7, 2, 3, 8)) < 0.5
    for tau in (0.0, 0.3, 0.6, 1.0):
        cl, shared, _ = share_impl(kept, tau, 7)
        cl = np.asarray(cl)
        for c in range(len(shared)):
            want = np.zeros(kept.shape[1:], dtype=bool)
            for t in np.nonzero(cl == c)[0]:
                want |= kept[t]
            want[..., 7:] = False
            assert np.array_equal(shared[c], want), "shared mask = union of the members' kept blocks"


def pin_intervals_golden(row_intervals_impl, merge_impl, pct_impl):
    g = _load_golden("skip_lists.json")
    for row in g["rows"]:
        assert [list(x) for x in row_intervals_impl(row["cols"])] == row["intervals"], f"intervals of {row['cols']}"
    for m in g["merges"]:
        got = [list(x) for x in merge_impl([tuple(x) for x in m["intervals"]], m["width"])]
        assert got == m["merged"], f"merge {m['intervals']} to {m['width']}: {got}"
    for p in g["percentiles"]:
        assert pct_impl(p["widths"], Fraction(p["pct"])) == p["width"], f"percentile {p}"


def pin_percentile_numpy(pct_impl, seed=21):
    """Nearest rank = NumPy's inverted-CDF percentile."""
    rng = _rng(seed)
    for trial in range(200):
        w = rng.integers(0, 30, size=int(rng.integers(1, 60)))
        pct = int(rng.integers(1, 101))
        want = int(np.percentile(w, pct, method="inverted_cdf"))
        assert pct_impl(list(w), Fraction(pct)) == want, f"percentile {pct} of {sorted(w)}"


def pin_merge_props(merge_impl, seed=22):
    """Merged rows keep the original blocks, have min(n, w) intervals, fill only gaps
    no longer than any gap left open (ties: leftmost filled), and add the fewest blocks
    of any choice of n - w gaps (enumeration)."""
    rng = _rng(seed)
    for trial in range(300):
        n = int(rng.integers(1, 9))
        lens = rng.integers(1, 3, size=n)
        iv, pos = [], 0
        for i in range(n):
            a = pos + int(rng.integers(1, 4)) if i else int(rng.integers(0, 3))
            b = a + int(lens[i])
            iv.append((a, b))
            pos = b
        w = int(rng.integers(1, n + 1))
        got = merge_impl(iv, w)
        assert len(got) == min(n, w)
        orig = {k for a, b in iv for k in range(a, b)}
        new = {k for a, b in got for k in range(a, b)}
        assert orig <= new, "merging drops no kept block"
        gaps = [(iv[i + 1][0] - iv[i][1], i) for i in range(n - 1)]
        filled = [g for g in gaps if all(k in new for k in range(iv[g[1]][1], iv[g[1] + 1][0]))]
        open_ = [g for g in gaps if g not in filled]
        assert len(filled) == n - len(got)
        for f in filled:
            for o in open_:
                assert f[0] < o[0] or (f[0] == o[0] and f[1] < o[1]), "a larger or later gap was filled"
        best = min(sum(g[0] for g in c) for c in itertools.combinations(gaps, n - min(n, w))) if n > w else 0
        assert len(new) - len(orig) == best, "not the fewest added blocks"


def pin_skip_round_trip(encode_impl, decode_impl, seed=23):
    """Without merging, decoding the encoded lists gives the sets back exactly; the
    width is the widest row."""
    rng = _rng(seed)
    T, H, nqb, nkb = 3, 2, 4, 23
    sets = [_rand_csr(rng, H, nqb, nkb, float(rng.random()))[1:] for _ in range(T)]
    w, counts, pairs = encode_impl(sets, H * nqb, 100)
    back = decode_impl(counts, pairs, T, H * nqb)
    for (rp, ci), (rb, cb) in zip(sets, back):
        assert np.array_equal(rp, rb) and np.array_equal(ci, cb), "round trip"
    widest = 0
    for rp, ci in sets:
        for r in range(H * nqb):
            c = ci[rp[r]:rp[r + 1]]
            widest = max(widest, int(np.sum(np.diff(c) != 1) + 1) if len(c) else 0)
    assert w == widest
    assert np.all(pairs[np.arange(pairs.shape[1])[None, :] >= counts[:, None]] == -1), "padding"


# ---------------------------------------------------------------- spatial repetition

def _eval_closed_form(expr):
    return eval(expr, {"__builtins__": {}}, {"sqrt": math.sqrt})


def _repetition_golden_inputs(case, pad=3):
    """d = 1, scale 1: key j = log(k_exp[j]); padded tokens get values that
    would dominate if they leaked into the softmax."""
    F, R, C = case["grid"]
    S = F * R * C
    L = S + pad
    q = np.full((1, 1, L, 1), 40.0)
    k = np.full((1, 1, L, 1), 40.0)
    q[0, 0, :S, 0] = case["q"]
    k[0, 0, :S, 0] = np.log(np.asarray(case["k_exp"], dtype=np.float64))
    return q, k, S, (F, R, C)


def pin_similarity_golden(sim_impl):
    """sim_impl(q, k, scale, seq_len, grid) -> [B, H]; hand-worked cosines."""
    for case in _load_golden("spatial_repetition.json")["similarity"]:
        q, k, S, grid = _repetition_golden_inputs(case)
        got = float(np.asarray(sim_impl(q, k, 1.0, S, grid))[0, 0])
        assert abs(got - _eval_closed_form(case["score"])) < 1e-12, f"golden score on grid {grid}"


def _brute_similarity(q, k, scale, S, grid):
    """Per token softmax and cosine in Python loops."""
    F, R, C = grid
    B, H = q.shape[:2]
    out = np.zeros((B, H))
    for b in range(B):
        for h in range(H):
            def prow(i):
                s = [scale * sum(q[b, h, i, c] * k[b, h, j, c] for c in range(q.shape[3])) for j in range(S)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                t = sum(e)
                return [x / t for x in e]
            tot, n = 0.0, 0
            for f in range(F):
                for y in range(R - 1):
                    for x in range(C):
                        a, c = prow((f * R + y) * C + x), prow((f * R + y + 1) * C + x)
                        dot = sum(u * v for u, v in zip(a, c))
                        tot += dot / math.sqrt(sum(u * u for u in a) * sum(v * v for v in c))
                        n += 1
            out[b, h] = tot / n
    return out


def pin_similarity_special(sim_impl, seed=24):
    rng = _rng(seed)
    # brute force on tiny random inputs (ragged padding, two prompts, two heads)
    for grid, pad in (((2, 3, 2), 5), ((1, 4, 3), 0), ((3, 2, 1), 2)):
        F, R, C = grid
        S = F * R * C
        q, k = (rng.standard_normal((2, 2, S + pad, 3)) for _ in range(2))
        got = np.asarray(sim_impl(q, k, 0.8, S, grid))
        assert np.max(np.abs(got - _brute_similarity(q, k, 0.8, S, grid))) < 1e-12, "brute-force cosines"
        assert np.all(got > 0) and np.all(got <= 1 + 1e-15), "cosine of positive vectors lies in (0, 1]"
    # Q = 0: every softmax row is uniform, so every cosine is 1
    F, R, C = 2, 4, 3
    S = F * R * C
    k = rng.standard_normal((1, 2, S + 4, 8))
    got = np.asarray(sim_impl(np.zeros_like(k), k, 1.0, S, (F, R, C)))
    assert np.max(np.abs(got - 1.0)) < 1e-12, "Q = 0 gives score 1"
    # queries repeated down the rows of each frame: identical softmax rows
    q = rng.standard_normal((1, 2, S + 4, 8))
    for f in range(F):
        for y in range(1, R):
            q[:, :, (f * R + y) * C:(f * R + y + 1) * C] = q[:, :, f * R * C:(f * R + 1) * C]
    got = np.asarray(sim_impl(q, k, 1.3, S, (F, R, C)))
    assert np.max(np.abs(got - 1.0)) < 1e-12, "rows that repeat give score 1"


def pin_row_groups(groups_impl, anchor_of_row_impl):
    """groups_impl(rows, k) -> [(lo, hi, anchor)]; golden cases, then the
    properties for every rows <= 40: contiguous cover, near-equal sizes, the
    lower middle row as anchor."""
    for case in _load_golden("spatial_repetition.json")["groups"]:
        got = [tuple(int(v) for v in t) for t in groups_impl(case["rows"], case["k"])]
        if "groups" in case:
            assert got == [tuple(t) for t in case["groups"]], f"groups rows={case['rows']} k={case['k']}"
        else:
            assert [t[2] for t in got] == case["anchors"], f"anchors rows={case['rows']} k={case['k']}"
    for R in range(1, 41):
        for k in range(1, R + 1):
            got = [tuple(int(v) for v in t) for t in groups_impl(R, k)]
            assert len(got) == k and got[0][0] == 0 and got[-1][1] == R
            assert all(got[i][1] == got[i + 1][0] for i in range(k - 1)), "contiguous"
            assert {hi - lo for lo, hi, _ in got} <= {R // k, -(-R // k)}, "near-equal sizes"
            for lo, hi, a in got:
                assert a - lo == (hi - 1 - lo) // 2, "lower middle row"
            amap = np.asarray(anchor_of_row_impl(R, k))
            assert [int(amap[y]) for y in range(R)] == [a for lo, hi, a in got for _ in range(lo, hi)]


def pin_anchor_sparsity_table(anchor_tokens_impl):
    """Table S4: the fraction of query rows skipped is 1 - k/30 at the Wan grid
    (21 frames x 30 rows x 52 columns = 32,760 tokens), printed in percent to
    one decimal."""
    for row in _load_golden("pages_tables.json")["anchor_rows"]["rows"]:
        n = len(np.unique(np.asarray(anchor_tokens_impl((21, 30, 52), row["k"]))))
        assert abs(100.0 * (1 - n / 32760) - row["sparsity"]) <= 0.05 + 1e-9, f"Table S4 sparsity at k={row['k']}"


def pin_anchor_broadcast(anchor_impl, seed=25):
    """anchor_impl(q, k, v, scale, seq_len, grid, k_anchor, heads) -> [B, len(heads), L, d].

    Query i attends (all but) only to key i (one-hot q and k, a large scale),
    so an output row is the V row of the token it was computed for: the
    golden source-token map shows through directly."""
    g = _load_golden("spatial_repetition.json")["broadcast"]
    F, R, C = g["grid"]
    S = F * R * C
    L = S + 2
    q = np.zeros((1, 1, L, S))
    q[0, 0, np.arange(S), np.arange(S)] = 1.0
    k = q.copy()
    v = _rng(seed).standard_normal((1, 1, L, 4))
    O = np.asarray(anchor_impl(q, k, v, 80.0, S, (F, R, C), g["k"], [0]))
    assert np.max(np.abs(O[0, 0, :S] - v[0, 0, g["source_token"]])) < 1e-12, "golden broadcast map"
    assert np.all(O[0, 0, S:] == 0.0), "padded rows are zero"


def pin_anchor_special(anchor_impl, seed=26):
    rng = _rng(seed)
    F, R, C = 2, 5, 3
    S = F * R * C
    L = S + 3
    q, k, v = (rng.standard_normal((2, 3, L, 8)) for _ in range(3))
    heads = [2, 0]
    ref = _sdpa(q[:, :, :S], k[:, :, :S], v[:, :, :S], 0.6)
    # every row its own anchor: ordinary attention (SDPA) for the listed heads
    O = np.asarray(anchor_impl(q, k, v, 0.6, S, (F, R, C), R, heads))
    assert np.max(np.abs(O[:, :, :S] - ref[:, heads])) < 1e-12, "k = rows gives dense attention"
    assert np.all(O[:, :, S:] == 0.0)
    # queries repeated down the rows of each frame: broadcasting is exact for any k
    for f in range(F):
        for y in range(1, R):
            q[:, :, (f * R + y) * C:(f * R + y + 1) * C] = q[:, :, f * R * C:(f * R + 1) * C]
    ref = _sdpa(q[:, :, :S], k[:, :, :S], v[:, :, :S], 0.6)
    for ka in (1, 2, 3):
        O = np.asarray(anchor_impl(q, k, v, 0.6, S, (F, R, C), ka, heads))
        assert np.max(np.abs(O[:, :, :S] - ref[:, heads])) < 1e-12, f"repeated rows, k={ka}"


def pin_select_golden(select_impl):
    g = _load_golden("spatial_repetition.json")["selection"]
    got = [int(x) for x in select_impl(np.array(g["sim"]), g["tau"])]
    assert got == g["heads_expected"], "heads whose mean score exceeds tau"
