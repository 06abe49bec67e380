"""Oracle skip lists against their pins (no GPU): Fig. S9, Fig. S10, Table S3."""

import numpy as np

import oracle
from tests import pins


def test_intervals_golden():
    pins.pin_intervals_golden(oracle.row_intervals, oracle.merge_row, oracle.width_percentile)


def test_percentile_is_numpy_inverted_cdf():
    pins.pin_percentile_numpy(oracle.width_percentile)


def test_merge_props():
    pins.pin_merge_props(oracle.merge_row)


def test_round_trip():
    pins.pin_skip_round_trip(oracle.encode_skip_lists, oracle.decode_skip_lists)


def test_merging_lowers_width_and_keeps_blocks():
    rng = np.random.default_rng(24)
    sets = [pins._rand_csr(rng, 3, 8, 40, 0.3)[1:] for _ in range(4)]
    w100, c100, p100 = oracle.encode_skip_lists(sets, 24, 100)
    w90, c90, p90 = oracle.encode_skip_lists(sets, 24, 90)
    assert w90 <= w100 and c90.max() <= w90
    for (rp, ci), (rb, cb) in zip(sets, oracle.decode_skip_lists(c90, p90, 4, 24)):
        for r in range(24):
            assert set(ci[rp[r]:rp[r + 1]]) <= set(cb[rb[r]:rb[r + 1]])
