"""Spatial-repetition oracle against its pins (hand-worked scores, brute force,
closed forms, SDPA, Table S4)."""

import oracle
from tests import pins


def test_similarity_golden():
    pins.pin_similarity_golden(oracle.spatial_similarity)


def test_similarity_special():
    pins.pin_similarity_special(oracle.spatial_similarity)


def test_similarity_in_passes():
    """The bounded-memory form (softmax rows of a few adjacent pairs at a
    time) meets the same golden values and special cases, and equals the
    whole-map form on a random grid."""
    import numpy as np
    passes = lambda *a, **kw: oracle.spatial_similarity(*a, pairs_per_pass=7, **kw)
    pins.pin_similarity_golden(passes)
    pins.pin_similarity_special(passes)
    rng = np.random.default_rng(12)
    grid = (2, 5, 9)
    q = rng.standard_normal((1, 2, 90, 16))
    k = rng.standard_normal((1, 2, 96, 16))
    whole = oracle.spatial_similarity(q, k, 0.3, 90, grid)
    for n in (1, 7, 36, 1000):
        assert np.allclose(oracle.spatial_similarity(q, k, 0.3, 90, grid, pairs_per_pass=n), whole,
                           rtol=0, atol=1e-14)


def test_row_groups():
    pins.pin_row_groups(oracle.row_groups, oracle.anchor_of_row)


def test_anchor_sparsity_matches_table_s4():
    pins.pin_anchor_sparsity_table(oracle.anchor_tokens)


def test_anchor_broadcast():
    pins.pin_anchor_broadcast(oracle.anchor_attention)


def test_anchor_special():
    pins.pin_anchor_special(oracle.anchor_attention)


def test_select_golden():
    pins.pin_select_golden(oracle.select_repetitive_heads)
