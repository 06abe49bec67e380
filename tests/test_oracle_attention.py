"""Oracle attention against its pins (no GPU)."""

import numpy as np
import pytest

import oracle
from tests import pins


def _sparse(q, k, v, row_ptr, col_idx, block, scale, seq_len):
    return oracle.sparse_attention_gather(q, k, v, row_ptr, col_idx, block, scale, seq_len)


def _sparse_masked(q, k, v, row_ptr, col_idx, block, scale, seq_len):
    B, H, L, d = np.shape(q)
    nqb = L // block
    bm = oracle.csr_to_block_mask(row_ptr, col_idx, H, nqb, nqb)
    return oracle.sparse_attention_masked_dense(q, k, v, bm, block, scale, seq_len)


def _sparse_rows(q, k, v, row_ptr, col_idx, block, scale, seq_len):
    B, H, L, d = np.shape(q)
    nqb = L // block
    items = [(b, h, qb) for b in range(B) for h in range(H) for qb in range(nqb)]
    out = oracle.sparse_attention_rows(q, k, v, row_ptr, col_idx, block, scale, seq_len, items)
    return out.reshape(B, H, nqb * block, d)


FORMS = {"gather": _sparse, "masked_dense": _sparse_masked, "rows": _sparse_rows}


@pytest.mark.parametrize("form", sorted(FORMS))
@pytest.mark.parametrize("pin", [
    pins.pin_sparse_all_kept_is_sdpa,
    pins.pin_sparse_is_masked_sdpa,
    pins.pin_lone_valid_key,
    pins.pin_zero_query_is_mean,
    pins.pin_golden_attention,
])
def test_sparse_pins(form, pin):
    pin(FORMS[form])


def test_dense_pin():
    pins.pin_dense_is_sdpa(oracle.dense_attention)


def test_gather_equals_masked_dense():
    rng = np.random.default_rng(20)
    B, H, L, S, d, blk = 2, 3, 256, 250, 16, 32
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    nqb = L // blk
    nkv = -(-S // blk)
    m, row_ptr, col_idx = pins._rand_csr(rng, H, nqb, nkv, 0.35, force_empty=2, force_full=2)
    a = _sparse(q, k, v, row_ptr, col_idx, blk, 0.25, S)
    b = _sparse_masked(q, k, v, row_ptr, col_idx, blk, 0.25, S)
    assert np.max(np.abs(a - b)) <= 1e-12


def test_all_kept_sparse_equals_dense_oracle():
    rng = np.random.default_rng(21)
    B, H, L, S, d, blk = 1, 2, 128, 128, 8, 32
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    nqb = L // blk
    row_ptr = (np.arange(H * nqb + 1) * nqb).astype(np.int32)
    col_idx = np.tile(np.arange(nqb), H * nqb).astype(np.int32)
    a = _sparse(q, k, v, row_ptr, col_idx, blk, 0.3, S)
    b = oracle.dense_attention(q, k, v, 0.3, S)
    assert np.max(np.abs(a - b)) <= 1e-12
