"""Calibrated block-sparse attention (CalibAtt) for AMD MI355X (gfx950).

The compute lives in libcalibatt.so (HIP kernels behind a C ABI, declared in
include/calibatt.h).  This package is the thin binding: ``capi`` mirrors the
C entry points one to one, ``MaskBank`` keeps the compiled lists of many
timesteps on the GPU (``SharedMaskBank``: one mask per run of alike
timesteps), and the spatial-repetition entry points score heads and run
their anchor rows.  Build the library with
``python -m block_sparse_attention_calibatt_amd.build``.
"""

from ._lib import CalibattError, LIB_PATH, load
from .capi import (
    new_queue,
    calibatt_transpose_v,
    calibatt_sparse_attn_fwd,
    calibatt_sparse_attn_fwd_noalloc,
    calibatt_dense_attn_fwd,
    calibatt_block_mass,
    calibatt_block_mass_single_pass,
    calibatt_block_mass_ws_bytes,
    calibatt_compile_ws_bytes,
    calibatt_compile_masks,
    calibatt_compile_masks_energy,
    calibatt_build_schedule,
    calibatt_share_ws_bytes,
    calibatt_share_timesteps,
    calibatt_skip_ws_bytes,
    calibatt_encode_skip_lists,
    calibatt_decode_skip_lists,
    calibatt_similarity_ws_bytes,
    calibatt_spatial_similarity,
    calibatt_select_repetitive_heads,
    calibatt_anchor_ws_bytes,
    calibatt_anchor_parts,
    calibatt_anchor_attn_fwd,
    calibatt_validate_csr,
    calibatt_status_string,
    calibatt_last_error,
    calibatt_version,
)
from .bank import MaskBank, SharedMaskBank, SkipLists

__all__ = [
    "CalibattError",
    "LIB_PATH",
    "load",
    "new_queue",
    "calibatt_transpose_v",
    "calibatt_sparse_attn_fwd",
    "calibatt_sparse_attn_fwd_noalloc",
    "calibatt_dense_attn_fwd",
    "calibatt_block_mass",
    "calibatt_block_mass_single_pass",
    "calibatt_block_mass_ws_bytes",
    "calibatt_compile_ws_bytes",
    "calibatt_compile_masks",
    "calibatt_compile_masks_energy",
    "calibatt_build_schedule",
    "calibatt_share_ws_bytes",
    "calibatt_share_timesteps",
    "calibatt_skip_ws_bytes",
    "calibatt_encode_skip_lists",
    "calibatt_decode_skip_lists",
    "calibatt_similarity_ws_bytes",
    "calibatt_spatial_similarity",
    "calibatt_select_repetitive_heads",
    "calibatt_anchor_ws_bytes",
    "calibatt_anchor_parts",
    "calibatt_anchor_attn_fwd",
    "calibatt_validate_csr",
    "calibatt_status_string",
    "calibatt_last_error",
    "calibatt_version",
    "MaskBank",
    "SharedMaskBank",
    "SkipLists",
]
