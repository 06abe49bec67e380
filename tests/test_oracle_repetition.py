"""Spatial-repetition oracle against its pins (hand-worked scores, brute force,
closed forms, SDPA, Table S4)."""

import oracle
from tests import pins


def test_similarity_golden():
    pins.pin_similarity_golden(oracle.spatial_similarity)


def test_similarity_special():
    pins.pin_similarity_special(oracle.spatial_similarity)


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
