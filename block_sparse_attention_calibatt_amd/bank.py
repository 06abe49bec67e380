"""Mask bank: the compiled kept-block lists of many timesteps, resident on the GPU.

The pages keep one calibrated mask per (layer, head, timestep) in a mask
dictionary that inference loads from (abstract; Fig. 5 caption).  Here one
bank holds the CSR lists of T timesteps for one layer: the row offsets of
all sets in one [T, H*nqb+1] tensor and the column lists concatenated, plus
each set's longest-row-first work order.  Looking a set up is host pointer
arithmetic: it returns views, nothing is copied or launched.
"""

import numpy as np
import torch

from .capi import calibatt_build_schedule, calibatt_validate_csr


class MaskBank:
    def __init__(self, sets, H, nqb, nkb_valid, device, validate=True):
        """sets: list of (row_ptr, col_idx) host int32 arrays, one per timestep."""
        self.H, self.nqb, self.nkb_valid = int(H), int(nqb), int(nkb_valid)
        rows = self.H * self.nqb
        if validate:
            for rp, ci in sets:
                calibatt_validate_csr(rp, ci, rows, self.nkb_valid)
        self.nnz = np.array([len(ci) for _, ci in sets], dtype=np.int64)
        self.offsets = np.concatenate([[0], np.cumsum(self.nnz)]).astype(np.int64)
        rp_all = np.stack([np.asarray(rp, dtype=np.int32) for rp, _ in sets])
        ci_all = np.concatenate([np.asarray(ci, dtype=np.int32) for _, ci in sets] + [np.zeros(1, np.int32)])
        self.row_ptr = torch.from_numpy(rp_all).to(device)
        self.col_idx = torch.from_numpy(ci_all).to(device)
        self.work_order = torch.empty((len(sets), rows + 9), dtype=torch.int32, device=device)
        for t in range(len(sets)):
            calibatt_build_schedule(self.row_ptr[t], self.H, self.nqb, self.work_order[t])

    def __len__(self):
        return len(self.nnz)

    def lookup(self, t):
        """(row_ptr, col_idx, work_order, nnz) of set t: views into the bank."""
        a, b = int(self.offsets[t]), int(self.offsets[t + 1])
        return self.row_ptr[t], self.col_idx[a:b], self.work_order[t], b - a
