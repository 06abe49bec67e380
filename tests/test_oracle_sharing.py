"""Oracle timestep sharing against its pins (no GPU): Fig. S11 and Table S3 captions."""

import numpy as np

import oracle
from tests import pins


def test_sharing_golden():
    pins.pin_sharing_golden(oracle.share_timesteps)


def test_iou_brute():
    pins.pin_iou_brute(oracle.iou_matrix)


def test_cluster_props():
    pins.pin_cluster_props(oracle.cluster_timesteps)


def test_shared_union():
    pins.pin_shared_union(oracle.share_timesteps)


def test_kept_from_csr_round_trip():
    rng = np.random.default_rng(20)
    kept = rng.random((3, 2, 4, 9)) < 0.4
    sets = [oracle.to_csr(kept[t]) for t in range(3)]
    assert np.array_equal(oracle.kept_from_csr_sets(sets, 2, 4, 9), kept)
