"""Interval-encoded skip lists with per-layer trimming and outlier merging
(test infrastructure only).

Pages (CalibAtt, arXiv 2603.05503):
* Fig. S10 caption: each row of a layer's "2D skip list" stores interval
  pairs for one (timestep, head, query block) entry; columns past a row's
  data are padding.  (a) allocation to the theoretical maximum width, (b)
  per-layer trimming to the widest row of the layer, (c) merging outlier rows
  lowers the layer's maximum width and allows further trimming.
* Fig. S9 caption: rows need very different numbers of intervals (95% at
  most 50, maximum 295 at N = 75,600).
* Table S3: merge at 99% / 95% shrinks the lists by 45% / 63% while the
  sparsity dips only from 62.50% to 62.41%, so merging fills gaps (computes
  a few skipped blocks).

Readings (no algorithm survives in the text):
* A row's intervals are its maximal runs of consecutive kept key blocks,
  half-open [start, end), ascending.  Its width is their number.
* "Merge p%": the layer width becomes the nearest-rank p-th percentile of
  the row widths of the layer (the smallest w such that at least
  ceil(p/100 * E) of the E rows have width <= w; p = 100 is the plain
  trimming of (b)).  A row wider than that is merged down to it by filling
  its smallest gaps between consecutive intervals, ties to the leftmost gap
  (equivalently: fill the n - w gaps that come first in (gap length,
  position) order).  Filled gaps become kept blocks.
* Padding pairs are (-1, -1).  When the percentile width is 0 (most rows
  empty) but some row keeps blocks, the width is 1.
"""

import math
from fractions import Fraction

import numpy as np


def row_intervals(cols):
    """Ascending unique kept blocks -> list of half-open runs [(start, end), ...]."""
    out = []
    for c in cols:
        c = int(c)
        if out and out[-1][1] == c:
            out[-1][1] = c + 1
        else:
            out.append([c, c + 1])
    return [(a, b) for a, b in out]


def width_percentile(widths, pct):
    """Nearest-rank percentile: the smallest w with at least ceil(pct/100 * E) widths <= w."""
    widths = sorted(int(w) for w in widths)
    if not widths:
        return 0
    p = Fraction(str(pct)) if isinstance(pct, float) else Fraction(pct)
    if not (0 < p <= 100):
        raise ValueError("pct must lie in (0, 100]")
    need = math.ceil(p * len(widths) / 100)
    return widths[need - 1]


def merge_row(intervals, width):
    """Fill the smallest gaps (ties: leftmost first) until at most `width` intervals remain."""
    n = len(intervals)
    if n <= width:
        return list(intervals)
    gaps = [(intervals[i + 1][0] - intervals[i][1], i) for i in range(n - 1)]
    fill = {i for _, i in sorted(gaps)[: n - max(width, 1)]}
    out = [list(intervals[0])]
    for i in range(1, n):
        if (i - 1) in fill:
            out[-1][1] = intervals[i][1]
        else:
            out.append(list(intervals[i]))
    return [(a, b) for a, b in out]


def encode_skip_lists(sets, rows, merge_pct=100):
    """T CSR sets (row_ptr, col_idx) of `rows` rows -> (width, counts [T*rows], pairs [T*rows, width, 2]).

    Entry e = t * rows + r.  `width` is the layer width after trimming and
    merging; pairs past a row's count are (-1, -1)."""
    ivs = []
    for rp, ci in sets:
        for r in range(rows):
            ivs.append(row_intervals(ci[rp[r]:rp[r + 1]]))
    widths = [len(v) for v in ivs]
    w = width_percentile(widths, merge_pct)
    if w == 0 and max(widths, default=0) > 0:
        w = 1          # a row that keeps anything needs one interval
    
    counts = np.zeros(len(ivs), dtype=np.int32)
    pairs = np.full((len(ivs), w, 2), -1, dtype=np.int32)
    for e, v in enumerate(ivs):
        m = merge_row(v, w)
        counts[e] = len(m)
        for j, (a, b) in enumerate(m):
            pairs[e, j] = (a, b)
    return w, counts, pairs


def decode_skip_lists(counts, pairs, T, rows):
    """-> list of T CSR sets (row_ptr, col_idx) int32."""
    sets = []
    for t in range(T):
        rp = [0]
        cols = []
        for r in range(rows):
            e = t * rows + r
            for j in range(int(counts[e])):
                a, b = int(pairs[e, j, 0]), int(pairs[e, j, 1])
                cols.extend(range(a, b))
            rp.append(len(cols))
        sets.append((np.array(rp, dtype=np.int32), np.array(cols, dtype=np.int32)))
    return sets
