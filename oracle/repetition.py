"""Spatial-repetition heads: similarity score, head selection, anchor rows (test infrastructure only).

Pages (CalibAtt, arXiv 2603.05503):
* Fig. 4 caption: in some heads the attention pattern of a query frame
  repeats from one spatial row of the frame to the next.
* Fig. 5 caption: calibration also finds the heads with spatial row
  repetition; at inference such a head computes attention only for a few
  anchor rows per frame and hands each anchor's outputs to the rows around
  it.
* Fig. 6 caption: one spatial-similarity score per attention map, stable
  across calibration prompts.
* Fig. S12 caption: k anchor rows per frame (k = 1..15), heads chosen by a
  similarity threshold; Fig. S13 caption: heads whose score exceeds
  tau = 0.87.
* Table S4: anchors computed over all keys (dense attention for the anchor
  queries), sparsity = fraction of query rows skipped = 1 - k/30 at 30
  spatial rows per frame.

Readings (the pages give no formula):
* Tokens are laid out frame-major on a (frames, rows, cols) grid:
  token n = (f*rows + y)*cols + x, and the grid covers exactly the valid
  tokens (frames*rows*cols = seq_len).
* The score of a map is the mean, over every vertically adjacent token pair
  (f, y, x), (f, y+1, x) of the same frame, of the cosine similarity of the
  two tokens' softmax rows (over the valid keys, unshifted: the broadcast
  copies an anchor's output unchanged, which is exact when the rows are
  equal).
* A head is repetitive when its score, averaged over the calibration
  prompts, is strictly greater than tau ("exceeds").
* The rows of a frame form k contiguous groups, group g holding rows
  [floor(g*rows/k), floor((g+1)*rows/k)); its anchor is the middle row
  floor((lo + hi - 1)/2).  Every token takes the output of the token at the
  same frame and column in its group's anchor row; padded tokens
  (n >= seq_len) output 0.
"""

import numpy as np


def row_groups(rows, k):
    """Fig. 5(b): k groups of consecutive spatial rows -> list of (lo, hi, anchor)."""
    if not 1 <= k <= rows:
        raise ValueError("need 1 <= k <= rows")
    out = []
    for g in range(k):
        lo, hi = (g * rows) // k, ((g + 1) * rows) // k
        out.append((lo, hi, (lo + hi - 1) // 2))
    return out


def anchor_of_row(rows, k):
    """Row y -> the anchor row whose output it takes."""
    a = np.empty(rows, dtype=np.int64)
    for lo, hi, anc in row_groups(rows, k):
        a[lo:hi] = anc
    return a


def anchor_tokens(grid, k):
    """Ascending token indices of the anchor queries: frame, then group, then column."""
    F, R, C = grid
    anc = [a for _, _, a in row_groups(R, k)]
    return np.array([(f * R + a) * C + x for f in range(F) for a in anc for x in range(C)], dtype=np.int64)


def _softmax_rows(q, k, scale, seq_len):
    """Softmax over the valid keys for each query row of q (float64)."""
    s = scale * (q @ k[:seq_len].T)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def _pair_cosines(a, c):
    return (a * c).sum(axis=1) / np.sqrt((a * a).sum(axis=1) * (c * c).sum(axis=1))


def spatial_similarity(q, k, scale, seq_len, grid, pairs_per_pass=None):
    """Fig. 6 / Fig. S13 score per (b, h): mean cosine of vertically adjacent softmax rows.

    pairs_per_pass: form the softmax rows of that many adjacent pairs at a
    time instead of the whole map (the same mean in bounded memory: the
    cosines are summed pass by pass and divided by their count)."""
    q, k = (np.asarray(x, dtype=np.float64) for x in (q, k))
    B, H, L, d = q.shape
    F, R, C = grid
    if F * R * C != seq_len or R < 2:
        raise ValueError("grid must cover seq_len exactly with at least two rows")
    top = np.array([(f * R + y) * C + x for f in range(F) for y in range(R - 1) for x in range(C)])
    sim = np.zeros((B, H), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            if pairs_per_pass is None:
                P = _softmax_rows(q[b, h, :seq_len], k[b, h], scale, seq_len)
                sim[b, h] = _pair_cosines(P[top], P[top + C]).mean()
            else:
                tot = 0.0
                for i in range(0, len(top), pairs_per_pass):
                    t = top[i:i + pairs_per_pass]
                    a = _softmax_rows(q[b, h, t], k[b, h], scale, seq_len)
                    c = _softmax_rows(q[b, h, t + C], k[b, h], scale, seq_len)
                    tot += _pair_cosines(a, c).sum()
                sim[b, h] = tot / len(top)
    return sim


def select_repetitive_heads(sim, tau):
    """Fig. S13: heads whose prompt-averaged score exceeds tau, ascending.

    sim is [P, H]; the mean over prompts is taken in prompt order in float64.
    """
    sim = np.asarray(sim, dtype=np.float64)
    mean = np.zeros(sim.shape[1])
    for p in range(sim.shape[0]):
        mean = mean + sim[p]
    mean = mean / sim.shape[0]
    return np.nonzero(mean > tau)[0].astype(np.int64)


def anchor_attention(q, k, v, scale, seq_len, grid, k_anchor, heads):
    """Fig. 5(b), bottom: dense attention for the anchor queries, broadcast to every row.

    Returns O [B, len(heads), L, d] in float64 for the listed heads, in the
    listed order.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, L, _ = q.shape
    dv = v.shape[3]
    F, R, C = grid
    if F * R * C != seq_len:
        raise ValueError("grid must cover seq_len exactly")
    anc_row = anchor_of_row(R, k_anchor)
    n = np.arange(seq_len)
    f, y, x = n // (R * C), (n // C) % R, n % C
    src = (f * R + anc_row[y]) * C + x          # the anchor token each token copies
    anchors = anchor_tokens(grid, k_anchor)
    O = np.zeros((B, len(heads), L, dv), dtype=np.float64)
    for b in range(B):
        for i, h in enumerate(heads):
            out = np.zeros((L, dv))
            P = _softmax_rows(q[b, h, anchors], k[b, h], scale, seq_len)
            out[anchors] = P @ v[b, h, :seq_len]
            O[b, i, :seq_len] = out[src]
    return O
