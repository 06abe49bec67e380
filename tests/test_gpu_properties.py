"""GPU property tests: hypothesis draws the shapes, masks, valid lengths and
masses; each drawn case goes through the C-ABI and is compared with the oracle.

The draws are derandomized (a fixed sequence of cases per test), so a run on
the GPU is reproducible and every case prints its parameters before it runs.
Kept-block lists are well formed by construction: ascending columns below the
count of key blocks that hold a valid key, which the host validates before a
launch.  Tolerances are those of the other parity tests: 2e-2 (bf16) and 1e-4
(f32) on O, 1e-3 relative on pooled mass, bit-exact for compile, skip lists
and the work order.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle
import block_sparse_attention_calibatt_amd as cal
from tests.gpu_util import say, to_dev, i32, small_cfg, inputs, err

pytestmark = pytest.mark.gpu
GPU_SETTINGS = dict(deadline=None, derandomize=True, database=None, max_examples=12,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
TOL = {"bf16": 2e-2, "f32": 1e-4}
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


@st.composite
def sparse_case(draw):
    dtype = draw(st.sampled_from(["bf16", "bf16", "f32"]))
    if dtype == "f32":
        d, block = draw(st.sampled_from([(64, 64), (128, 128)]))
    else:
        d, block = draw(st.sampled_from([(64, 64), (128, 64), (64, 128), (128, 128)]))
    nqb = draw(st.integers(1, 6))
    L = nqb * block
    S = draw(st.one_of(st.integers(1, L), st.just(L), st.integers(max(1, L - block), L)))
    H = draw(st.integers(1, 2))
    B = draw(st.integers(1, 2))
    nv = -(-S // block)
    rows = []
    for _ in range(H * nqb):
        kind = draw(st.sampled_from(["empty", "one", "full", "random", "last"]))
        if kind == "empty":
            rows.append([])
        elif kind == "one":
            rows.append([draw(st.integers(0, nv - 1))])
        elif kind == "full":
            rows.append(list(range(nv)))
        elif kind == "last":
            rows.append([nv - 1])              # only the block holding the valid-length boundary
        else:
            rows.append(sorted(draw(st.sets(st.integers(0, nv - 1), max_size=nv))))
    rp = np.zeros(H * nqb + 1, dtype=np.int32)
    for r, c in enumerate(rows):
        rp[r + 1] = rp[r] + len(c)
    ci = np.array([c for row in rows for c in row], dtype=np.int32)
    seed = draw(st.integers(0, 2**20))
    persistent = draw(st.booleans())
    return dict(B=B, H=H, L=L, S=S, d=d, block=block, dtype=dtype, rp=rp, ci=ci, seed=seed,
                persistent=persistent)


@settings(**GPU_SETTINGS)
@given(sparse_case())
def test_sparse_forward_random_masks(gpu, c):
    say("case: sparse property", {k: c[k] for k in ("B", "H", "L", "S", "d", "block", "dtype", "seed", "persistent")},
        "nnz", len(c["ci"]))
    cfg = small_cfg(B=c["B"], H=c["H"], L=c["L"], S=c["S"], d=c["d"], block=c["block"], dtype=c["dtype"],
                    seed=c["seed"])
    q, k, v = inputs(cfg)
    cal.calibatt_validate_csr(c["rp"], c["ci"], cfg.rows, cfg.nkb_valid)
    ref = oracle.sparse_attention_gather(q, k, v, c["rp"], c["ci"], c["block"], cfg.scale, c["S"])
    dt = TDT[c["dtype"]]
    Q, K, V = (to_dev(x, dt) for x in (q, k, v))
    O = torch.full_like(Q, float("nan"))
    RP = i32(c["rp"])
    CI = i32(c["ci"] if len(c["ci"]) else np.zeros(1, np.int32))[: len(c["ci"])]
    cal.calibatt_sparse_attn_fwd(Q, K, V, O, RP, CI, c["block"], cfg.scale, c["S"], None,
                                 cal.new_queue("cuda:0") if c["persistent"] else None)
    torch.cuda.synchronize()
    e = err(O, ref)
    say(f"  max err {e:.3e}")
    assert e <= TOL[c["dtype"]]


@st.composite
def mass_case(draw):
    d, block = draw(st.sampled_from([(64, 64), (128, 64), (64, 128), (128, 128)]))
    nqb = draw(st.integers(1, 6))
    L = nqb * block
    S = draw(st.one_of(st.integers(1, L), st.integers(max(1, L - block), L)))
    return dict(B=draw(st.integers(1, 2)), H=draw(st.integers(1, 2)), L=L, S=S, d=d, block=block,
                seed=draw(st.integers(0, 2**20)), method=draw(st.sampled_from(["two_pass", "single_pass"])))


@settings(**GPU_SETTINGS)
@given(mass_case())
def test_block_mass_random_tails(gpu, c):
    say("case: block mass property", c)
    cfg = small_cfg(B=c["B"], H=c["H"], L=c["L"], S=c["S"], d=c["d"], block=c["block"], seed=c["seed"])
    q, k, _ = inputs(cfg)
    want = oracle.block_mass(q, k, c["block"], cfg.scale, c["S"])
    Q, K = (to_dev(x, torch.bfloat16) for x in (q, k))
    lse = torch.empty(c["B"] * c["H"] * c["L"], dtype=torch.float32, device="cuda:0")
    mass = torch.full((c["B"], c["H"], cfg.nqb, cfg.nkb), float("nan"), dtype=torch.float32, device="cuda:0")
    if c["method"] == "two_pass":
        cal.calibatt_block_mass(Q, K, c["block"], cfg.scale, lse, mass, c["S"])
    else:
        cal.calibatt_block_mass_single_pass(Q, K, c["block"], cfg.scale, lse, mass, c["S"])
    torch.cuda.synchronize()
    got = mass.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - want) <= 1e-3 * np.abs(want) + 1e-6)
    # each query block's row sums to its valid query count (softmax rows sum to one)
    for qb in range(cfg.nqb):
        vq = max(0, min((qb + 1) * c["block"], c["S"]) - qb * c["block"])
        assert np.all(np.abs(got[:, :, qb].sum(axis=-1) - vq) <= 1e-3 * max(vq, 1))


@st.composite
def compile_case(draw):
    P = draw(st.integers(1, 8))
    H = draw(st.integers(1, 3))
    nqb = draw(st.integers(1, 8))
    nkb = draw(st.integers(1, 40))
    nv = draw(st.integers(1, nkb))
    kind = draw(st.sampled_from(["ties", "nan", "rand"]))
    seed = draw(st.integers(0, 2**20))
    rng = np.random.default_rng(seed)
    if kind == "ties":
        m = rng.integers(0, 4, size=(P, H, nqb, nkb)).astype(np.float32) * np.float32(0.5)
    else:
        m = (rng.random((P, H, nqb, nkb)) ** 3).astype(np.float32)
        if kind == "nan":
            m[rng.random(m.shape) < 0.1] = np.nan
            m[..., ::3] = m[..., :1]                 # whole columns tied with the first
    return dict(m=m, nv=nv, K=draw(st.integers(0, nkb + 1)), t=draw(st.integers(0, P)),
                eps=draw(st.sampled_from(["0", "1/20", "1/10", "1/4", "1/2", "1"])),
                desc=dict(P=P, H=H, nqb=nqb, nkb=nkb, nv=nv, kind=kind, seed=seed))


@settings(**GPU_SETTINGS)
@given(compile_case())
def test_compile_topk_forced_ties(gpu, c):
    say("case: top-K compile property", c["desc"], "K", c["K"], "min_agree", c["t"])
    rp, ci = cal.calibatt_compile_masks(torch.from_numpy(c["m"]).cuda(), c["K"], c["t"], c["nv"])
    want_rp, want_ci = oracle.compile_masks(c["m"], c["K"], c["t"], c["nv"])
    assert np.array_equal(rp.cpu().numpy(), want_rp)
    assert np.array_equal(ci.cpu().numpy(), want_ci)


@settings(**GPU_SETTINGS)
@given(compile_case())
def test_compile_energy_forced_ties(gpu, c):
    say("case: energy compile property", c["desc"], "eps", c["eps"], "min_agree", c["t"])
    eps = Fraction(c["eps"])
    rp, ci = cal.calibatt_compile_masks_energy(torch.from_numpy(c["m"]).cuda(), eps, c["t"], c["nv"])
    want_rp, want_ci = oracle.compile_masks_energy(c["m"], eps, c["t"], c["nv"])
    assert np.array_equal(rp.cpu().numpy(), want_rp)
    assert np.array_equal(ci.cpu().numpy(), want_ci)


@st.composite
def bank_case(draw):
    T = draw(st.integers(1, 3))
    H = draw(st.integers(1, 2))
    nqb = draw(st.integers(1, 6))
    nkb = draw(st.integers(1, 48))
    sets = []
    for _ in range(T):
        rp, cols = [0], []
        for _ in range(H * nqb):
            kind = draw(st.sampled_from(["empty", "one", "alt", "random"]))
            if kind == "empty":
                c = []
            elif kind == "one":
                c = [draw(st.integers(0, nkb - 1))]
            elif kind == "alt":
                c = list(range(draw(st.integers(0, 1)), nkb, 2))
            else:
                c = sorted(draw(st.sets(st.integers(0, nkb - 1), max_size=nkb)))
            cols.extend(c)
            rp.append(len(cols))
        sets.append((np.array(rp, dtype=np.int32), np.array(cols, dtype=np.int32)))
    pct = draw(st.sampled_from([100, 99, 95, 90, 50, 1]))
    return dict(T=T, H=H, nqb=nqb, nkb=nkb, sets=sets, pct=pct)


@settings(**GPU_SETTINGS)
@given(bank_case())
def test_skip_lists_random_banks(gpu, c):
    say("case: skip-list property", {k: c[k] for k in ("T", "H", "nqb", "nkb", "pct")},
        "nnz", [len(s[1]) for s in c["sets"]])
    rows = c["H"] * c["nqb"]
    bank = cal.MaskBank(c["sets"], c["H"], c["nqb"], c["nkb"], torch.device("cuda:0"))
    sk = bank.encode_skip_lists(c["pct"], c["nkb"])
    w, counts, pairs = oracle.encode_skip_lists(c["sets"], rows, c["pct"])
    assert sk.width == w
    assert np.array_equal(sk.counts.cpu().numpy(), counts)
    assert np.array_equal(sk.pairs.cpu().numpy(), pairs)


@settings(**GPU_SETTINGS)
@given(st.integers(1, 24), st.integers(1, 8), st.data())
def test_work_order_random_counts(gpu, H, nqb, data):
    counts = data.draw(st.lists(st.integers(0, 12), min_size=H * nqb, max_size=H * nqb))
    say("case: work-order property", dict(H=H, nqb=nqb, nnz=sum(counts)))
    rp = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    wo = cal.calibatt_build_schedule(i32(rp), H, nqb)
    torch.cuda.synchronize()
    assert np.array_equal(wo.cpu().numpy(), oracle.lpt_work_order(rp, H, nqb))
