"""Timestep sharing on the GPU against the oracle (Fig. S11 and Table S3 captions)."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
import block_sparse_attention_calibatt_amd as cal
from tests import pins
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _bank_from_kept(kept, nkb_valid):
    T, H, nqb, nkb = kept.shape
    sets = [oracle.to_csr(kept[t] & (np.arange(nkb) < nkb_valid)) for t in range(T)]
    return cal.MaskBank(sets, H, nqb, nkb_valid, torch.device("cuda:0")), sets


def _check(kept, nkb, nkb_valid, tau):
    T, H, nqb, _ = kept.shape
    bank, sets = _bank_from_kept(kept, nkb_valid)
    sb = bank.share(tau, nkb)
    kept_v = oracle.kept_from_csr_sets(sets, H, nqb, nkb)
    cl, shared, iou = oracle.share_timesteps(kept_v, tau, nkb_valid)
    got_iou = sb.iou.cpu().numpy()
    assert np.array_equal(got_iou, iou), f"IoU differs: max {np.max(np.abs(got_iou - iou))}"
    assert np.array_equal(sb.cluster_of, cl)
    assert sb.n_sets == shared.shape[0]
    for c in range(shared.shape[0]):
        want_rp, want_ci = oracle.to_csr(shared[c])
        rp, ci, _, nnz = sb.shared.lookup(c)
        assert np.array_equal(rp.cpu().numpy(), want_rp), f"shared set {c} row offsets"
        assert np.array_equal(ci.cpu().numpy(), want_ci), f"shared set {c} columns"
    for t in range(T):
        assert sb.lookup(t)[3] == len(oracle.to_csr(shared[cl[t]])[1])
    return sb, cl


@pytest.mark.parametrize("case", [
    dict(T=1, H=2, nqb=3, nkb=8, nv=8, p=0.5),
    dict(T=6, H=3, nqb=4, nkb=40, nv=37, p=0.4),
    dict(T=8, H=2, nqb=5, nkb=64, nv=64, p=0.7),
    dict(T=5, H=1, nqb=2, nkb=33, nv=1, p=0.5),
], ids=lambda c: "T{T}H{H}q{nqb}k{nkb}v{nv}".format(**c))
def test_share_random_banks(gpu, case):
    rng = np.random.default_rng(case["T"] * 100 + case["nkb"])
    base = rng.random((case["H"], case["nqb"], case["nkb"])) < case["p"]
    kept = np.stack([base ^ (rng.random(base.shape) < 0.1 * t / case["T"]) for t in range(case["T"])])
    for tau in (0.0, 0.5, 0.8, 0.95, 1.0, 1.5):
        say(f"case: sharing {case} tau {tau}")
        _check(kept, case["nkb"], case["nv"], tau)


def test_share_golden(gpu):
    g, kept = pins._golden_sharing()
    for case in g["cases"]:
        tau = float(Fraction(case["tau"]))
        sb, cl = _check(kept, 4, 4, tau)
        assert list(cl) == case["clusters"]


def test_share_wan_drifting(gpu):
    cfg = synth.get_config("wan")
    T = 12
    say(f"case: sharing of {T} drifting Wan-shaped timestep sets, tau 0.9 and 0.97")
    sets = synth.drifting_sets(cfg, T)
    bank = cal.MaskBank(sets, cfg.H, cfg.nqb, cfg.nkb_valid, torch.device("cuda:0"))
    kept = oracle.kept_from_csr_sets(sets, cfg.H, cfg.nqb, cfg.nkb)
    for tau in (0.9, 0.97):
        sb = bank.share(tau, cfg.nkb)
        cl, shared, iou = oracle.share_timesteps(kept, tau, cfg.nkb_valid)
        assert np.array_equal(sb.iou.cpu().numpy(), iou)
        assert np.array_equal(sb.cluster_of, cl)
        for c in range(shared.shape[0]):
            want_rp, want_ci = oracle.to_csr(shared[c])
            rp, ci, _, _ = sb.shared.lookup(c)
            assert np.array_equal(rp.cpu().numpy(), want_rp) and np.array_equal(ci.cpu().numpy(), want_ci)
        say(f"  tau {tau}: {sb.n_sets} shared sets for {T} timesteps, clusters {list(cl)}")


def test_share_capacity_error(gpu):
    rng = np.random.default_rng(3)
    kept = rng.random((3, 2, 4, 8)) < 0.5
    bank, _ = _bank_from_kept(kept, 8)
    off = torch.from_numpy(bank.offsets).cuda()
    lib = cal.load()
    import ctypes
    from block_sparse_attention_calibatt_amd.capi import _ptr, _stream
    T, rows = 3, 8
    iou = torch.empty((T, T), dtype=torch.float64, device="cuda:0")
    cl = torch.empty(T, dtype=torch.int32, device="cuda:0")
    srp = torch.empty((T, rows + 1), dtype=torch.int32, device="cuda:0")
    soff = torch.empty(T + 1, dtype=torch.int64, device="cuda:0")
    sci = torch.empty(2, dtype=torch.int32, device="cuda:0")
    need = cal.calibatt_share_ws_bytes(T, 2, 4, 8)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    C, nnz = ctypes.c_int32(0), ctypes.c_int64(0)
    st = lib.calibatt_share_timesteps(_ptr(bank.row_ptr), _ptr(bank.col_idx), _ptr(off), T, 2, 4, 8, 8, 0.0,
                                      _ptr(iou), _ptr(cl), _ptr(srp), _ptr(soff), _ptr(sci), 2, ctypes.byref(C),
                                      ctypes.byref(nnz), _ptr(ws), need, _stream(iou))
    assert st == 6 and C.value == 1 and nnz.value == int(np.count_nonzero(kept.any(0)))
