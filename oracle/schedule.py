"""Work order for the block-sparse forward pass (test infrastructure only).

The pages do not describe a scheduler.  Kept counts differ from row to row
(Fig. S9: most skip-list rows hold at most 50 intervals, the largest 295), so
rows are ordered by their cost.  The order the library uses is defined here
as a plain rule:

1. head cost = kept blocks of the head; heads sorted by (cost descending,
   head ascending) are given one at a time to the partition with the smallest
   total so far (ties: lowest partition), 8 partitions;
2. partition p lists its heads in the order they were given to it; inside a
   head, rows by kept count descending, ties by ascending query block;
3. the result is the 8 lists concatenated (row indices h*nqb + qb), followed
   by the 9 list offsets (0, ..., H*nqb).
"""

import numpy as np

PARTS = 8


def head_partitions(row_ptr, H, nqb):
    """Greedy longest-first assignment of heads to PARTS partitions -> list of head lists."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    cost = [int(row_ptr[(h + 1) * nqb] - row_ptr[h * nqb]) for h in range(H)]
    heads = sorted(range(H), key=lambda h: (-cost[h], h))
    load = [0] * PARTS
    parts = [[] for _ in range(PARTS)]
    for h in heads:
        p = min(range(PARTS), key=lambda i: (load[i], i))
        parts[p].append(h)
        load[p] += cost[h]
    return parts


def lpt_work_order(row_ptr, H, nqb):
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    order, offsets = [], [0]
    for heads in head_partitions(row_ptr, H, nqb):
        for h in heads:
            rows = [(int(row_ptr[h * nqb + qb + 1] - row_ptr[h * nqb + qb]), qb) for qb in range(nqb)]
            rows.sort(key=lambda t: (-t[0], t[1]))
            order.extend(h * nqb + qb for _, qb in rows)
        offsets.append(len(order))
    return np.array(order + offsets, dtype=np.int32)
