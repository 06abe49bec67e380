"""GPU parity: calibration pooling, mask compile, work order, mask bank, and the
calibrate -> compile -> infer pipeline, against the float64 oracle.

* block mass: |mass_gpu - mass_oracle| <= 1e-3 * |mass_oracle| + 1e-6.  The
  kernel multiplies bf16 inputs exactly in float32 and accumulates 128 products
  per score, so a logit carries at most ~1e-4 relative error; 1e-3 leaves a
  tenfold margin.
* compile and work order: bit-exact on float32 masses drawn by the seeded
  generator (integer-valued draws force ties, NaN draws test the ordering).
* pipeline: the GPU pools its own masses, so top-K decisions may differ from
  the oracle's only where the masses' tolerance intervals overlap the K-th
  boundary.  Decisions outside that band must match; the band is reported.
"""

import math

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
import block_sparse_attention_calibatt_amd as cal
from synth.configs import Config
from tests.gpu_util import say, to_dev, i32

pytestmark = pytest.mark.gpu


def mass_tol(m):
    return 1e-3 * np.abs(m) + 1e-6


def gpu_mass(q, k, cfg, method="two_pass"):
    Q, K = (to_dev(x, torch.bfloat16) for x in (q, k))
    B, H = q.shape[:2]
    lse = torch.empty(B * H * cfg.L, dtype=torch.float32, device="cuda:0")
    mass = torch.full((B, H, cfg.nqb, cfg.nkb), float("nan"), dtype=torch.float32, device="cuda:0")
    if method == "two_pass":
        cal.calibatt_block_mass(Q, K, cfg.block, cfg.scale, lse, mass, cfg.S)
    else:
        cal.calibatt_block_mass_single_pass(Q, K, cfg.block, cfg.scale, lse, mass, cfg.S)
    torch.cuda.synchronize()
    return mass, lse


METHODS = ["two_pass", "single_pass"]


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("shape", [
    (1, 2, 1024, 1000, 128, 128),
    (2, 1, 768, 768, 128, 128),
    (1, 2, 512, 449, 64, 64),
    (1, 1, 1024, 1000, 128, 64),
    (1, 1, 1024, 1000, 64, 128),
], ids=lambda s: "x".join(map(str, s)))
def test_block_mass_small(gpu, shape, method):
    B, H, L, S, d, block = shape
    cfg = Config("m", B=B, H=H, L=L, S=S, d=d, block=block, dtype="bf16", data_seed=40, mask_seed=0,
                 grid=(4, 8, 16))
    say("case: block mass", method, shape)
    q, k, _ = synth.gen_qkv(cfg)
    mass, lse = gpu_mass(q, k, cfg, method)
    ref = oracle.block_mass(q, k, block, cfg.scale, S)
    got = mass.cpu().numpy().astype(np.float64)
    excess = np.abs(got - ref) - mass_tol(ref)
    rel = np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30))
    say(f"  max rel err {rel:.2e}, worst excess over tolerance {excess.max():.2e}")
    assert np.all(excess <= 0)
    lse_h = lse.cpu().numpy().reshape(B, H, L)
    assert np.all(np.isneginf(lse_h[:, :, S:])), "padded rows hold -inf"
    assert np.all(np.isfinite(lse_h[:, :, :S]))
    # fixed reduction order: a second run gives the same bits
    mass2, lse2 = gpu_mass(q, k, cfg, method)
    assert torch.equal(mass2, mass) and torch.equal(lse2, lse), "repeat run"


@pytest.mark.parametrize("method", METHODS)
def test_block_mass_wan_sampled(gpu, method):
    cfg = synth.get_config("calib")
    say("case: block mass at Wan size, whole head 7 and sampled query blocks (prompt seed 100)", method)
    q, k = synth.gen_qk(cfg, cfg.prompt_seeds[0])
    mass, _ = gpu_mass(q, k, cfg, method)
    rng = np.random.default_rng(3)
    # every query block of head 7, then rows of other heads
    items = [(7, qb) for qb in range(cfg.nqb)]
    items += [(0, 0), (cfg.H - 1, cfg.nqb - 1)] + [(int(rng.integers(cfg.H)), int(rng.integers(cfg.nqb))) for _ in range(6)]
    worst = -1.0
    f64 = {}
    for h, qb in items:
        if h not in f64:
            f64 = {h: (q[0, h].astype(np.float64), k[0, h].astype(np.float64))}
        ref = oracle.block_mass_rows(f64[h][0], f64[h][1], cfg.block, cfg.scale, cfg.S, qb)
        got = mass[0, h, qb].cpu().numpy().astype(np.float64)
        worst = max(worst, float((np.abs(got - ref) - mass_tol(ref)).max()))
        nvalid = min((qb + 1) * cfg.block, cfg.S) - qb * cfg.block
        assert abs(got.sum() - nvalid) < 1e-3 * nvalid
    say(f"  {len(items)} rows, worst excess over tolerance {worst:.2e}")
    assert worst <= 0


def test_block_mass_methods_agree_wan(gpu):
    """Every tile at the Wan shape: the single pass against the two passes
    (both are float32 sums of the same bf16 products)."""
    cfg = synth.get_config("calib")
    q, k = synth.gen_qk(cfg, cfg.prompt_seeds[1])
    a, la = gpu_mass(q, k, cfg, "two_pass")
    b, lb = gpu_mass(q, k, cfg, "single_pass")
    assert torch.equal(la, lb), "the same log-sum-exp pass"
    d = (a - b).abs()
    rel = float((d / a.abs().clamp_min(1e-30)).max())
    say(f"case: block mass methods at Wan size: max abs diff {float(d.max()):.2e}, max rel {rel:.2e}")
    assert bool((d <= 1e-5 * a.abs() + 1e-9).all())


def _masses(rng, P, H, nqb, nkb, kind):
    if kind == "ties":
        m = rng.integers(0, 6, size=(P, H, nqb, nkb)).astype(np.float32)
    elif kind == "nan":
        m = rng.random((P, H, nqb, nkb)).astype(np.float32)
        m[rng.random(m.shape) < 0.05] = np.nan
        m[..., 3] = m[..., 5]                       # exact duplicates
    else:
        m = (rng.random((P, H, nqb, nkb)) ** 4).astype(np.float32)
    return m


@pytest.mark.parametrize("case", [
    dict(P=8, H=3, nqb=16, nkb=16, nv=16, K=4, t=4, kind="ties"),
    dict(P=8, H=3, nqb=16, nkb=16, nv=13, K=4, t=4, kind="nan"),
    dict(P=5, H=2, nqb=8, nkb=24, nv=24, K=6, t=3, kind="rand"),
    dict(P=1, H=2, nqb=8, nkb=8, nv=8, K=2, t=1, kind="ties"),
    dict(P=4, H=2, nqb=8, nkb=8, nv=8, K=0, t=1, kind="rand"),
    dict(P=4, H=2, nqb=8, nkb=8, nv=7, K=3, t=0, kind="rand"),
    dict(P=3, H=1, nqb=4, nkb=1024, nv=1000, K=250, t=2, kind="ties"),
    dict(P=8, H=40, nqb=256, nkb=256, nv=256, K=64, t=4, kind="ties"),
], ids=lambda c: "P{P}H{H}q{nqb}k{nkb}v{nv}K{K}t{t}{kind}".format(**c))
def test_compile_bitexact(gpu, case):
    say("case: compile", case)
    rng = np.random.default_rng(case["P"] * 1000 + case["nkb"])
    m = _masses(rng, case["P"], case["H"], case["nqb"], case["nkb"], case["kind"])
    wo = torch.full((case["H"] * case["nqb"] + 9,), -7, dtype=torch.int32, device="cuda")
    rp, ci = cal.calibatt_compile_masks(torch.from_numpy(m).cuda(), case["K"], case["t"], case["nv"], work_order=wo)
    want_rp, want_ci = oracle.compile_masks(m, case["K"], case["t"], case["nv"])
    assert np.array_equal(rp.cpu().numpy(), want_rp)
    assert np.array_equal(ci.cpu().numpy(), want_ci)
    # the optional work order of the compiled set: the schedule rule's, bit for bit
    assert np.array_equal(wo.cpu().numpy(), oracle.lpt_work_order(want_rp, case["H"], case["nqb"]))
    say(f"  nnz {len(want_ci)}")


@pytest.mark.parametrize("case", [
    dict(P=8, H=3, nqb=16, nkb=16, nv=16, eps="1/4", t=4, kind="ties"),
    dict(P=8, H=3, nqb=16, nkb=16, nv=13, eps="1/10", t=4, kind="nan"),
    dict(P=5, H=2, nqb=8, nkb=24, nv=24, eps="0", t=3, kind="rand"),
    dict(P=5, H=2, nqb=8, nkb=24, nv=24, eps="1", t=0, kind="rand"),
    dict(P=4, H=2, nqb=8, nkb=8, nv=7, eps="1/2", t=1, kind="big"),
    dict(P=3, H=1, nqb=4, nkb=1024, nv=1000, eps="1/20", t=2, kind="ties"),
    dict(P=8, H=4, nqb=64, nkb=256, nv=256, eps="1/20", t=4, kind="rand"),
], ids=lambda c: "P{P}H{H}q{nqb}k{nkb}v{nv}e{eps}t{t}{kind}".format(**c).replace("/", "_"))
def test_compile_energy_bitexact(gpu, case):
    """Energy-threshold compile (Fig. S8 caption reading) against the oracle, bit-exact."""
    say("case: energy compile", case)
    rng = np.random.default_rng(case["P"] * 1000 + case["nkb"] + 7)
    if case["kind"] == "big":
        m = (rng.random((case["P"], case["H"], case["nqb"], case["nkb"])) * 300.0).astype(np.float32)
    else:
        m = _masses(rng, case["P"], case["H"], case["nqb"], case["nkb"], case["kind"])
    eps = Fraction(case["eps"])
    wo = torch.full((case["H"] * case["nqb"] + 9,), -7, dtype=torch.int32, device="cuda")
    rp, ci = cal.calibatt_compile_masks_energy(torch.from_numpy(m).cuda(), eps, case["t"], case["nv"], work_order=wo)
    want_rp, want_ci = oracle.compile_masks_energy(m, eps, case["t"], case["nv"])
    assert np.array_equal(rp.cpu().numpy(), want_rp)
    assert np.array_equal(ci.cpu().numpy(), want_ci)
    assert np.array_equal(wo.cpu().numpy(), oracle.lpt_work_order(want_rp, case["H"], case["nqb"]))
    say(f"  nnz {len(want_ci)}")


def test_compile_energy_pooled_masses_sampled(gpu):
    """Energy compile at the Wan shape on pooled masses of 8 prompts (their row sums are the
    query counts, the rule's intended input); rows sampled and checked against the oracle."""
    cfg = synth.get_config("calib")
    say("case: energy compile of 8 prompts' pooled masses at Wan size, eps 1/20, min_agree 4")
    masses = []
    for seed in cfg.prompt_seeds[:8]:
        q, k = synth.gen_qk(cfg, seed)
        mass, _ = gpu_mass(q, k, cfg)
        masses.append(mass[0])
    M = torch.stack(masses).contiguous()
    rp, ci = cal.calibatt_compile_masks_energy(M, Fraction(1, 20), 4, cfg.nkb_valid)
    rp_h, ci_h = rp.cpu().numpy(), ci.cpu().numpy()
    m_h = M.cpu().numpy()
    rng = np.random.default_rng(11)
    rows = [0, cfg.H * cfg.nqb - 1] + [int(x) for x in rng.integers(0, cfg.H * cfg.nqb, size=10)]
    for r in rows:
        h, qb = divmod(r, cfg.nqb)
        keep = oracle.energy_keep(m_h[:, h, qb], Fraction(1, 20), cfg.nkb_valid)
        want = np.nonzero(oracle.agreement(keep, 4))[0]
        assert np.array_equal(ci_h[rp_h[r]:rp_h[r + 1]], want), f"row {r}"
    say(f"  {len(rows)} rows match; kept density {len(ci_h) / (cfg.H * cfg.nqb * cfg.nkb_valid):.4f}")


def test_compile_capacity_error(gpu):
    rng = np.random.default_rng(1)
    m = torch.from_numpy(_masses(rng, 4, 2, 8, 8, "rand")).cuda()
    small = torch.empty(5, dtype=torch.int32, device="cuda:0")
    with pytest.raises(cal.CalibattError) as e:
        cal.calibatt_compile_masks(m, 3, 2, 8, col_idx=small)
    assert e.value.status == 6 and "nnz_cap" in str(e.value)


def test_schedule_bitexact(gpu):
    rng = np.random.default_rng(5)
    for H, nqb, hi in [(40, 256, 257), (3, 7, 4), (2, 1024, 40)]:
        counts = rng.integers(0, hi, size=H * nqb)
        rp = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        wo = cal.calibatt_build_schedule(i32(rp), H, nqb)
        assert np.array_equal(wo.cpu().numpy(), oracle.lpt_work_order(rp, H, nqb)), (H, nqb)


def test_mask_bank_lookup(gpu):
    cfg = synth.get_config("imbalance")
    say("case: mask bank of 6 timestep sets, lookup vs direct upload (bitwise) + oracle rows")
    sets = [synth.csr_for_config(cfg, t) for t in range(6)]
    bank = cal.MaskBank(sets, cfg.H, cfg.nqb, cfg.nkb_valid, torch.device("cuda:0"))
    q, k, v = synth.gen_qkv(cfg)
    Q, K, V = (to_dev(x, torch.bfloat16) for x in (q, k, v))
    qws = cal.new_queue("cuda:0")
    for t in (0, 3, 5):
        rp, ci, wo, nnz = bank.lookup(t)
        assert nnz == len(sets[t][1])
        assert np.array_equal(wo.cpu().numpy(), oracle.lpt_work_order(sets[t][0], cfg.H, cfg.nqb))
        O1 = torch.empty_like(Q)
        cal.calibatt_sparse_attn_fwd(Q, K, V, O1, rp, ci, cfg.block, cfg.scale, cfg.S, wo, qws)
        O2 = torch.empty_like(Q)
        cal.calibatt_sparse_attn_fwd(Q, K, V, O2, i32(sets[t][0]), i32(sets[t][1]), cfg.block, cfg.scale, cfg.S)
        torch.cuda.synchronize()
        assert torch.equal(O1, O2)
        if t == 3:
            items = [(0, 5, 17), (0, 39, 255), (0, 20, 0)]
            ref = oracle.sparse_attention_rows(q, k, v, sets[t][0], sets[t][1], cfg.block, cfg.scale, cfg.S, items)
            for (b, h, qb), rr in zip(items, ref):
                g = O1[b, h, qb * 128:(qb + 1) * 128].float().cpu().numpy()
                assert np.max(np.abs(g - rr)) <= 2e-2


def certain_keep(ms, K, nv):
    """Per-block keep decision that holds for every mass inside the tolerance intervals.

    ms: oracle masses of one row (float64).  Returns +1 (kept whatever the
    rounding), -1 (dropped whatever the rounding) or 0 (depends on it)."""
    m = ms[:nv]
    lo, hi = m - mass_tol(m), m + mass_tol(m)
    out = np.full(len(ms), -1)
    for kb in range(nv):
        can_beat = np.sum(hi >= lo[kb]) - 1           # others that might precede it
        surely_beat = np.sum(lo > hi[kb])             # others that surely precede it
        out[kb] = 1 if can_beat < K else (-1 if surely_beat >= K else 0)
    return out


def _pipeline(cfg, prompt_seeds, infer_seed, check_rows, tag, single_pass=False):
    P = len(prompt_seeds)
    K = math.ceil(cfg.keep_frac * cfg.nkb_valid)
    t = oracle.min_agree_count(cfg.rho, P)
    dev = torch.device("cuda:0")
    mass = torch.empty((P, cfg.H, cfg.nqb, cfg.nkb), dtype=torch.float32, device=dev)
    lse = torch.empty(cfg.H * cfg.L, dtype=torch.float32, device=dev)
    heads = sorted({h for h, _ in check_rows})
    ref_mass = {}
    for p, seed in enumerate(prompt_seeds):
        q, k = synth.gen_qk(cfg, seed)
        Q, Kt = (to_dev(x, torch.bfloat16) for x in (q, k))
        if single_pass:
            cal.calibatt_block_mass_single_pass(Q, Kt, cfg.block, cfg.scale, lse, mass[p], cfg.S)
        else:
            cal.calibatt_block_mass(Q, Kt, cfg.block, cfg.scale, lse, mass[p], cfg.S)
        for h in heads:
            qh, kh = q[0, h].astype(np.float64), k[0, h].astype(np.float64)
            for hh, qb in check_rows:
                if hh == h:
                    ref_mass[(p, h, qb)] = oracle.block_mass_rows(qh, kh, cfg.block, cfg.scale, cfg.S, qb)
        del Q, Kt, q, k
    rp, ci = cal.calibatt_compile_masks(mass, K, t, cfg.nkb_valid)
    wo = cal.calibatt_build_schedule(rp, cfg.H, cfg.nqb)
    torch.cuda.synchronize()
    rp_h, ci_h, mass_h = rp.cpu().numpy(), ci.cpu().numpy(), mass.cpu().numpy().astype(np.float64)
    cal.calibatt_validate_csr(rp_h, ci_h, cfg.rows, cfg.nkb_valid)
    assert np.array_equal(wo.cpu().numpy(), oracle.lpt_work_order(rp_h, cfg.H, cfg.nqb))

    q, k, v = synth.gen_qkv(cfg, infer_seed)
    Q, Kt, V = (to_dev(x, torch.bfloat16) for x in (q, k, v))
    O = torch.empty_like(Q)
    qws = cal.new_queue(dev)
    cal.calibatt_sparse_attn_fwd(Q, Kt, V, O, rp, ci, cfg.block, cfg.scale, cfg.S, wo, qws)
    torch.cuda.synchronize()

    ambiguous, checked, worst = 0, 0, 0.0
    for h, qb in check_rows:
        r = h * cfg.nqb + qb
        dec = np.zeros(cfg.nkb, dtype=int)
        surely = np.zeros(cfg.nkb, dtype=int)
        maybe = np.zeros(cfg.nkb, dtype=int)
        for p in range(P):
            ref = ref_mass[(p, h, qb)]
            got = mass_h[p, h, qb]
            assert np.all(np.abs(got - ref) <= mass_tol(ref)), f"{tag}: mass row ({p},{h},{qb})"
            c = certain_keep(ref, K, cfg.nkb_valid)
            surely += c == 1
            maybe += c == 0
        dec[surely >= t] = 1
        dec[surely + maybe < t] = -1
        kept = np.zeros(cfg.nkb, dtype=bool)
        kept[ci_h[rp_h[r]:rp_h[r + 1]]] = True
        assert np.all(kept[dec == 1]), f"{tag}: row {r} misses a surely kept block"
        assert not np.any(kept[dec == -1]), f"{tag}: row {r} keeps a surely dropped block"
        ambiguous += int(np.sum(dec == 0))
        # attention on the inference input over the row's compiled list: it
        # holds every surely kept block and no surely dropped one (asserted
        # above); a block whose decision rests on a near-tie may go either way
        row_ci = np.flatnonzero(kept).astype(np.int32)
        # one-head CSR whose only non-empty row is qb
        one_rp = np.where(np.arange(cfg.nqb + 1) > qb, len(row_ci), 0).astype(np.int32)
        rr = oracle.sparse_attention_rows(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], one_rp, row_ci,
                                          cfg.block, cfg.scale, cfg.S, [(0, 0, qb)])
        g = O[0, h, qb * cfg.block:(qb + 1) * cfg.block].float().cpu().numpy()
        worst = max(worst, float(np.max(np.abs(g - rr[0]))))
        checked += 1
    say(f"  {tag}: nnz {len(ci_h)} ({len(ci_h) / (cfg.rows * cfg.nkb_valid):.3f}), rows checked {len(check_rows)}, "
        f"undecided blocks {ambiguous}, attention rows compared {checked}, max err {worst:.2e}")
    assert checked == len(check_rows)
    assert worst <= 2e-2


def test_pipeline_small(gpu):
    cfg = Config("calib-small", B=1, H=2, L=2048, S=2040, d=128, block=128, dtype="bf16", data_seed=60,
                 mask_seed=0, grid=(2, 30, 34))
    say("case: calibrate 4 prompts -> compile -> infer, small")
    rows = [(h, qb) for h in range(cfg.H) for qb in range(cfg.nqb)]
    _pipeline(cfg, (61, 62, 63, 64), 65, rows, "small")


def test_pipeline_wan_sampled(gpu):
    cfg = synth.get_config("calib")
    say("case: calibrate 8 Wan prompts (single-pass pooling) -> compile -> infer on the 9th, sampled rows")
    rng = np.random.default_rng(8)
    rows = [(0, 0), (39, 255)] + [(int(rng.integers(cfg.H)), int(rng.integers(cfg.nqb))) for _ in range(22)]
    _pipeline(cfg, cfg.prompt_seeds, cfg.infer_seed, rows, "wan", single_pass=True)
