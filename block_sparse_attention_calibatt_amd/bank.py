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

from .capi import (
    calibatt_build_schedule,
    calibatt_decode_skip_lists,
    calibatt_encode_skip_lists,
    calibatt_share_timesteps,
    calibatt_validate_csr,
)


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

    @classmethod
    def from_device(cls, row_ptr, col_idx, offsets, H, nqb, nkb_valid):
        """A bank over sets already on the GPU: row_ptr [T, H*nqb+1], col_idx (concatenated),
        offsets [T+1] (host int64, where each set's columns start)."""
        self = cls.__new__(cls)
        self.H, self.nqb, self.nkb_valid = int(H), int(nqb), int(nkb_valid)
        self.offsets = np.asarray(offsets, dtype=np.int64)
        self.nnz = np.diff(self.offsets)
        self.row_ptr = row_ptr
        self.col_idx = torch.cat([col_idx, torch.zeros(1, dtype=torch.int32, device=col_idx.device)])
        rows = self.H * self.nqb
        self.work_order = torch.empty((len(self.nnz), rows + 9), dtype=torch.int32, device=row_ptr.device)
        for t in range(len(self.nnz)):
            calibatt_build_schedule(self.row_ptr[t], self.H, self.nqb, self.work_order[t])
        return self

    def share(self, tau, nkb=None):
        """Timestep sharing (calibatt_share_timesteps): a SharedMaskBank serving every
        timestep of this bank from one mask per run of alike timesteps."""
        nkb = self.nkb_valid if nkb is None else int(nkb)
        off = torch.from_numpy(self.offsets).to(self.row_ptr.device)
        cluster_of, iou, rp, soff, ci = calibatt_share_timesteps(self.row_ptr, self.col_idx, off, self.H, self.nqb,
                                                                 nkb, self.nkb_valid, tau)
        shared = MaskBank.from_device(rp, ci, soff.cpu().numpy(), self.H, self.nqb, self.nkb_valid)
        return SharedMaskBank(shared, cluster_of.cpu().numpy(), iou)

    def encode_skip_lists(self, merge_pct=100, nkb=None):
        """The bank as interval skip lists (calibatt_encode_skip_lists)."""
        nkb = self.nkb_valid if nkb is None else int(nkb)
        off = torch.from_numpy(self.offsets).to(self.row_ptr.device)
        width, widest, counts, pairs = calibatt_encode_skip_lists(self.row_ptr, self.col_idx, off, self.H, self.nqb,
                                                                  nkb, merge_pct)
        return SkipLists(width, widest, counts, pairs, len(self), self.H, self.nqb, self.nkb_valid)

    def __len__(self):
        return len(self.nnz)

    def lookup(self, t):
        """(row_ptr, col_idx, work_order, nnz) of set t: views into the bank."""
        a, b = int(self.offsets[t]), int(self.offsets[t + 1])
        return self.row_ptr[t], self.col_idx[a:b], self.work_order[t], b - a


class SharedMaskBank:
    """Timesteps mapped onto the shared masks of their runs (Table S3 caption's timestep
    sharing): lookup(t) returns the shared set of t's run."""

    def __init__(self, shared, cluster_of, iou):
        self.shared = shared
        self.cluster_of = np.asarray(cluster_of, dtype=np.int64)
        self.iou = iou

    def __len__(self):
        return len(self.cluster_of)

    @property
    def n_sets(self):
        return len(self.shared)

    def lookup(self, t):
        return self.shared.lookup(int(self.cluster_of[t]))


class SkipLists:
    """A layer's 2D skip lists (Fig. S10 caption): per (timestep, head, query block) entry
    up to `width` (start, end) pairs of kept key blocks, padded with (-1, -1)."""

    def __init__(self, width, widest, counts, pairs, T, H, nqb, nkb_valid):
        self.width, self.widest = int(width), int(widest)
        self.counts, self.pairs = counts, pairs
        self.T, self.H, self.nqb, self.nkb_valid = int(T), int(H), int(nqb), int(nkb_valid)

    @property
    def size_bytes(self):
        """Storage of the trimmed lists: int32 pairs of every entry at the layer width."""
        return self.T * self.H * self.nqb * self.width * 2 * 4

    def decode(self):
        """A MaskBank of the kept blocks the lists encode (calibatt_decode_skip_lists)."""
        rp, off, ci = calibatt_decode_skip_lists(self.counts, self.pairs.reshape(-1), self.width, self.T, self.H,
                                                 self.nqb)
        return MaskBank.from_device(rp, ci, off.cpu().numpy(), self.H, self.nqb, self.nkb_valid)
