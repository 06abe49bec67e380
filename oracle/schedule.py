"""Work order for the block-sparse forward pass (test infrastructure only).

The pages do not describe a scheduler.  Kept counts differ from row to row
(Fig. S9: most skip-list rows hold at most 50 intervals, the largest 295), so
rows are ordered by their cost.
The order the library uses is defined here as a plain rule: heads in
ascending order; inside a head, rows by kept count descending (longest
first), ties by ascending query block.  Entry i is a row index h*nqb + qb.
"""

import numpy as np


def lpt_work_order(row_ptr, H, nqb):
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    order = []
    for h in range(H):
        cost = [(int(row_ptr[h * nqb + qb + 1] - row_ptr[h * nqb + qb]), qb) for qb in range(nqb)]
        cost.sort(key=lambda t: (-t[0], t[1]))
        order.extend(h * nqb + qb for _, qb in cost)
    return np.array(order, dtype=np.int32)
