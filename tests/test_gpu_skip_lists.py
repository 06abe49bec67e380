"""Interval skip lists on the GPU against the oracle (Fig. S9, Fig. S10, Table S3)."""

import ctypes
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


def _check_bank(sets, H, nqb, nkb, nkb_valid, pct):
    rows = H * nqb
    bank = cal.MaskBank(sets, H, nqb, nkb_valid, torch.device("cuda:0"))
    sk = bank.encode_skip_lists(pct, nkb)
    w, counts, pairs = oracle.encode_skip_lists(sets, rows, pct)
    assert sk.width == w, f"width {sk.width} vs {w}"
    widest = max(len(oracle.row_intervals(ci[rp[r]:rp[r + 1]])) for rp, ci in sets for r in range(rows))
    assert sk.widest == widest
    assert np.array_equal(sk.counts.cpu().numpy(), counts)
    assert np.array_equal(sk.pairs.cpu().numpy(), pairs)
    back = sk.decode()
    want = oracle.decode_skip_lists(counts, pairs, len(sets), rows)
    for t, (wrp, wci) in enumerate(want):
        rp, ci, _, _ = back.lookup(t)
        assert np.array_equal(rp.cpu().numpy(), wrp) and np.array_equal(ci.cpu().numpy(), wci), f"decoded set {t}"
    return sk, back


@pytest.mark.parametrize("case", [
    dict(T=3, H=2, nqb=4, nkb=23, p=0.5),
    dict(T=2, H=3, nqb=8, nkb=64, p=0.3),
    dict(T=4, H=1, nqb=16, nkb=200, p=0.6),
    dict(T=2, H=2, nqb=3, nkb=1024, p=0.5),
    dict(T=2, H=2, nqb=3, nkb=9, p=0.0),
], ids=lambda c: "T{T}H{H}q{nqb}k{nkb}p{p}".format(**c))
def test_skip_lists_random(gpu, case):
    rng = np.random.default_rng(case["T"] * 1000 + case["nkb"])
    sets = [pins._rand_csr(rng, case["H"], case["nqb"], case["nkb"], case["p"])[1:] for _ in range(case["T"])]
    for pct in (100, 99, 95, 90, 50, Fraction(1, 3)):
        say(f"case: skip lists {case} merge {pct}%")
        _check_bank(sets, case["H"], case["nqb"], case["nkb"], case["nkb"], pct)


def test_skip_lists_wan_drifting(gpu):
    cfg = synth.get_config("wan")
    sets = synth.drifting_sets(cfg, 3)
    kept0 = sum(len(ci) for _, ci in sets)
    for pct in (100, 99, 95):
        sk, back = _check_bank(sets, cfg.H, cfg.nqb, cfg.nkb, cfg.nkb_valid, pct)
        kept = int(back.nnz.sum())
        say(f"  Wan, 3 drifting sets, merge {pct}%: width {sk.widest} -> {sk.width}, "
            f"{sk.size_bytes / 1e6:.2f} MB, kept blocks {kept0} -> {kept}")
        assert kept >= kept0


def test_skip_lists_capacity(gpu):
    rng = np.random.default_rng(5)
    sets = [pins._rand_csr(rng, 2, 4, 16, 0.5)[1:] for _ in range(2)]
    bank = cal.MaskBank(sets, 2, 4, 16, torch.device("cuda:0"))
    lib = cal.load()
    from block_sparse_attention_calibatt_amd.capi import _ptr, _stream
    off = torch.from_numpy(bank.offsets).cuda()
    counts = torch.empty(16, dtype=torch.int32, device="cuda:0")
    pairs = torch.empty(2, dtype=torch.int32, device="cuda:0")
    need = cal.calibatt_skip_ws_bytes(2, 2, 4)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    w, wd = ctypes.c_int32(0), ctypes.c_int32(0)
    st = lib.calibatt_encode_skip_lists(_ptr(bank.row_ptr), _ptr(bank.col_idx), _ptr(off), 2, 2, 4, 16, 100, 1,
                                        _ptr(counts), _ptr(pairs), 0, ctypes.byref(w), ctypes.byref(wd), _ptr(ws),
                                        need, _stream(counts))
    want_w, _, _ = oracle.encode_skip_lists(sets, 8, 100)
    assert st == 6 and w.value == want_w and wd.value == want_w
