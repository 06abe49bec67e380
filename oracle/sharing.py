"""Timestep sharing of calibrated masks (test infrastructure only).

Pages (CalibAtt, arXiv 2603.05503):
* Fig. S11 caption: the intersection-over-union between the skipped-block
  masks of two timesteps, averaged over layers and heads; later timesteps
  are more alike, so masks can be shared across consecutive late steps.
* Table S3 caption: timestep sharing clusters masks whose pair-wise IoU is
  at least tau.

Readings (the pages give no algorithm):
* The skipped set of (timestep t, head h) is every valid key block
  (kb < nkb_valid) of every row of head h that t does not keep.  One bank
  holds one layer, so the average runs over heads.
* IoU(t1, t2) = mean over heads of |S1 & S2| / |S1 | S2|, taken as 1 when
  both sets are empty.  Computed in float64: each head's ratio by one
  division, summed over heads in ascending order, divided by H.
* Clusters are runs of consecutive timesteps, formed greedily in t: a
  timestep joins the current cluster when its IoU with every member is at
  least tau, and otherwise opens a new cluster.
* A cluster's shared mask keeps every block that any member keeps (it skips
  only what all members skip), so no timestep computes less than its own
  calibrated mask.
"""

import numpy as np


def kept_from_csr_sets(sets, H, nqb, nkb):
    """list of T (row_ptr, col_idx) -> kept [T, H, nqb, nkb] bool."""
    kept = np.zeros((len(sets), H, nqb, nkb), dtype=bool)
    for t, (rp, ci) in enumerate(sets):
        for r in range(H * nqb):
            kept[t, r // nqb, r % nqb, ci[rp[r]:rp[r + 1]]] = True
    return kept


def skipped_sets(kept, nkb_valid):
    """kept [T, H, nqb, nkb] -> skipped [T, H, nqb, nkb]: valid blocks not kept."""
    kept = np.asarray(kept, dtype=bool)
    valid = np.arange(kept.shape[-1]) < nkb_valid
    return ~kept & valid


def iou_matrix(kept, nkb_valid):
    """Mean-over-heads IoU of the skipped sets of every pair of timesteps: [T, T] float64."""
    s = skipped_sets(kept, nkb_valid)
    T, H = s.shape[0], s.shape[1]
    out = np.ones((T, T), dtype=np.float64)
    for t1 in range(T):
        for t2 in range(t1 + 1, T):
            acc = 0.0
            for h in range(H):
                inter = int(np.count_nonzero(s[t1, h] & s[t2, h]))
                union = int(np.count_nonzero(s[t1, h] | s[t2, h]))
                acc += 1.0 if union == 0 else inter / union
            out[t1, t2] = out[t2, t1] = acc / H
    return out


def cluster_timesteps(iou, tau):
    """Greedy runs of consecutive timesteps whose pair-wise IoU is >= tau: cluster id per t."""
    T = iou.shape[0]
    cluster = np.zeros(T, dtype=np.int32)
    start, c = 0, 0
    for t in range(1, T):
        if all(iou[u, t] >= tau for u in range(start, t)):
            cluster[t] = c
        else:
            c += 1
            start = t
            cluster[t] = c
    return cluster


def share_timesteps(kept, tau, nkb_valid):
    """-> (cluster id per timestep [T] int32, shared kept masks [C, H, nqb, nkb] bool, IoU [T, T])."""
    kept = np.asarray(kept, dtype=bool)
    iou = iou_matrix(kept, nkb_valid)
    cluster = cluster_timesteps(iou, tau)
    C = int(cluster.max()) + 1 if len(cluster) else 0
    valid = np.arange(kept.shape[-1]) < nkb_valid
    shared = np.zeros((C,) + kept.shape[1:], dtype=bool)
    for t in range(kept.shape[0]):
        shared[cluster[t]] |= kept[t] & valid
    return cluster, shared, iou
