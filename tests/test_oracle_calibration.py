"""Oracle calibration steps against their pins (no GPU)."""

import numpy as np
import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("pin", [
    pins.pin_mass_row_sums,
    pins.pin_mass_zero_query,
    pins.pin_mass_brute_force,
    pins.pin_mass_golden,
])
def test_mass_pins(pin):
    pin(oracle.block_mass)


def test_mass_rows_match_full():
    rng = np.random.default_rng(30)
    q, k = (rng.standard_normal((1, 2, 64, 8)) for _ in range(2))
    full = oracle.block_mass(q, k, 16, 0.5, 61)
    for h in range(2):
        for qb in range(4):
            r = oracle.block_mass_rows(q[0, h], k[0, h], 16, 0.5, 61, qb)
            assert np.array_equal(r, full[0, h, qb])


def test_topk_pins():
    pins.pin_topk_subsets(oracle.topk_keep)
    pins.pin_topk_counts(oracle.topk_keep)


def test_agreement_pins():
    pins.pin_agreement_brute(oracle.agreement)
    pins.pin_min_agree(oracle.min_agree_count)


def test_agreement_frequency_range():
    """Keep frequency count/P lies in [0, 1]; 0 = skipped by all, 1 = kept by all (Fig. 3(b))."""
    rng = np.random.default_rng(31)
    mass = rng.random((8, 2, 16, 16)).astype(np.float32)
    keep = oracle.topk_keep(mass, 4)
    freq = keep.sum(0) / 8.0
    assert freq.min() >= 0.0 and freq.max() <= 1.0
    assert np.array_equal(oracle.agreement(keep, 8), freq == 1.0)
    assert np.array_equal(~oracle.agreement(keep, 1), freq == 0.0)


def test_csr_pin():
    pins.pin_csr(oracle.to_csr)


def test_compile_pin():
    pins.pin_compile_brute(oracle.compile_masks)


def test_compile_decides_in_float32():
    """Two masses that differ only below float32 resolution compile identically."""
    m64 = np.array([[[[1.0, 1.0 + 1e-12, 0.5, 0.25]]]])
    rp, ci = oracle.compile_masks(m64, 1, 1)
    assert ci.tolist() == [0], "float32 rounding makes the two equal; index breaks the tie"


def test_energy_rule_pins():
    """Energy-threshold row rule (Fig. S8 caption): fixed point, hand-worked cases,
    enumeration, special cases, and the whole compile by enumeration."""
    pins.pin_mass_fixed(oracle.mass_fixed)
    pins.pin_energy_golden(oracle.energy_keep)
    pins.pin_energy_brute(oracle.energy_keep)
    pins.pin_energy_special(oracle.energy_keep)
    pins.pin_compile_energy_brute(oracle.compile_masks_energy)
