"""Attention over kept key blocks, float64 (test infrastructure only).

Pages: CalibAtt abstract (the selected connections are computed densely, the
unselected ones skipped) and the Fig. 5(b) caption (for non-repetitive heads
the block masks are loaded and the unset blocks are not computed).  Skipping a
block removes its keys from the softmax, so for query token i with kept key
tokens J_i:

    s_ij = scale * <q_i, k_j>
    O_i  = sum_{j in J_i} exp(s_ij - max_J s) v_j / sum_{j in J_i} exp(s_ij - max_J s)

Readings where the pages are silent:
* keys j >= seq_len are padding and never part of J_i; query rows i >= seq_len
  output zero;
* a query whose kept set holds no valid key outputs zero;
* one block mask per (head, query block) serves every batch entry (masks are
  keyed by layer, head and timestep only, abstract).

Inputs are float64 arrays [B, H, L, d]; bfloat16 workloads pass their exact
bfloat16 values.  Two independent forms are given (gather and masked-dense)
so each can be checked against the other.
"""

import numpy as np


def csr_to_block_mask(row_ptr, col_idx, H, nqb, nkb):
    """CSR kept lists -> [H, nqb, nkb] bool block mask."""
    m = np.zeros((H * nqb, nkb), dtype=bool)
    for r in range(H * nqb):
        m[r, col_idx[row_ptr[r]:row_ptr[r + 1]]] = True
    return m.reshape(H, nqb, nkb)


def _kept_key_tokens(kbs, block, seq_len):
    toks = [np.arange(kb * block, min((kb + 1) * block, seq_len)) for kb in kbs]
    toks = [t for t in toks if len(t)]
    return np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)


def _row_block(qs, ks, vs, kbs, qb, block, scale, seq_len):
    """O for the `block` query tokens of query block qb of one (b, h) slab."""
    d = vs.shape[1]
    out = np.zeros((block, d), dtype=np.float64)
    lo, hi = qb * block, min((qb + 1) * block, seq_len)
    if hi <= lo:
        return out
    J = _kept_key_tokens(kbs, block, seq_len)
    if len(J) == 0:
        return out
    s = scale * (qs[lo:hi] @ ks[J].T)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    out[: hi - lo] = (e @ vs[J]) / e.sum(axis=1, keepdims=True)
    return out


def sparse_attention_gather(q, k, v, row_ptr, col_idx, block, scale, seq_len):
    """Gather form: per query block, one product against the concatenated kept keys."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, L, d = q.shape
    nqb = L // block
    O = np.zeros((B, H, L, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for qb in range(nqb):
                r = h * nqb + qb
                kbs = col_idx[row_ptr[r]:row_ptr[r + 1]]
                O[b, h, qb * block:(qb + 1) * block] = _row_block(
                    q[b, h], k[b, h], v[b, h], kbs, qb, block, scale, seq_len)
    return O


def sparse_attention_rows(q, k, v, row_ptr, col_idx, block, scale, seq_len, items):
    """O of selected query blocks only: items = [(b, h, qb), ...] -> [n, block, d].

    q, k, v may be any array-likes indexable as [b, h] -> [L, d]."""
    out = []
    nqb = None
    for (b, h, qb) in items:
        qs = np.asarray(q[b, h], dtype=np.float64)
        ks = np.asarray(k[b, h], dtype=np.float64)
        vs = np.asarray(v[b, h], dtype=np.float64)
        nqb = qs.shape[0] // block
        r = h * nqb + qb
        kbs = col_idx[row_ptr[r]:row_ptr[r + 1]]
        out.append(_row_block(qs, ks, vs, kbs, qb, block, scale, seq_len))
    return np.stack(out) if out else np.zeros((0, block, 0))


def sparse_attention_masked_dense(q, k, v, block_mask, block, scale, seq_len):
    """Masked-dense form: the full score matrix with -inf outside kept blocks, then softmax."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, L, d = q.shape
    O = np.zeros((B, H, L, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            allowed = np.kron(block_mask[h].astype(np.int8),
                              np.ones((block, block), dtype=np.int8)).astype(bool)
            allowed[:, seq_len:] = False
            s = np.where(allowed, scale * (q[b, h] @ k[b, h].T), -np.inf)
            m = s.max(axis=1, keepdims=True)
            live = np.isfinite(m[:, 0])
            e = np.zeros_like(s)
            e[live] = np.exp(s[live] - m[live])
            num = e @ v[b, h]
            den = e.sum(axis=1, keepdims=True)
            O[b, h, live] = num[live] / den[live]
            O[b, h, seq_len:] = 0.0
    return O


def dense_attention(q, k, v, scale, seq_len):
    """Ordinary softmax attention over the valid keys j < seq_len."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, L, d = q.shape
    O = np.zeros((B, H, L, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h, :seq_len] @ k[b, h, :seq_len].T)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            O[b, h, :seq_len] = (e @ v[b, h, :seq_len]) / e.sum(axis=1, keepdims=True)
    return O
