"""CPU oracle for calibrated block-sparse attention (CalibAtt, arXiv 2603.05503).

TEST INFRASTRUCTURE ONLY.  Plain, slow, float64 NumPy written from the
pages' description of the method.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it; the library path never calls
it, and it imports nothing from the library or its kernels.

What it computes (each function cites the passage it follows):

* ``attention``   - attention restricted to kept key blocks, the skipped
  blocks being absent from the softmax (abstract; Fig. 5(b) caption); the
  dense special case.
* ``calibration`` - pooled post-softmax mass per (query block, key block)
  (Fig. 2 caption's block-level maps; "block energies", Table S5 caption),
  top key blocks per query block (Fig. 5(a) caption), cross-prompt agreement
  with a threshold (Fig. 3(b) caption, Fig. 7 caption), and the kept lists as
  CSR rows keyed by (head, query block) (abstract: per layer, head and
  timestep); the energy-threshold row rule (Fig. S8 caption) as the variant
  of the top-K rule.
* ``sharing``     - timestep sharing: the IoU of two timesteps' skipped-block
  masks averaged over heads (Fig. S11 caption), runs of consecutive
  timesteps with pair-wise IoU >= tau (Table S3 caption), one shared mask
  per run.
* ``intervals``   - 2D skip lists: each row's kept blocks as intervals, the
  layer width trimmed to a percentile of the row widths and wider rows
  merged by filling their smallest gaps (Fig. S9, Fig. S10, Table S3).
* ``repetition``  - spatial-repetition heads: the mean cosine similarity of
  vertically adjacent softmax rows (Fig. 4, Fig. 6), heads above tau
  (Fig. S13), and attention for k anchor rows per frame broadcast to the
  other rows (Fig. 5(b), Table S4).
* ``schedule``    - the work order: heads spread over 8 partitions longest
  first, rows inside a head longest first.

Pins: every function is checked by ``tests/test_oracle_*.py`` against facts
that do not come from this code (library routines on the special cases they
cover, closed forms, invariants, brute-force enumeration on tiny inputs,
hand-worked fixtures under ``tests/golden/``).  No function here is
"parity unpinned".
"""

from .attention import (
    dense_attention,
    sparse_attention_gather,
    sparse_attention_masked_dense,
    sparse_attention_rows,
    csr_to_block_mask,
)
from .calibration import (
    block_mass,
    block_mass_rows,
    topk_keep,
    agreement,
    min_agree_count,
    to_csr,
    compile_masks,
    mass_fixed,
    energy_keep,
    compile_masks_energy,
)
from .schedule import lpt_work_order
from .intervals import (
    row_intervals,
    width_percentile,
    merge_row,
    encode_skip_lists,
    decode_skip_lists,
)
from .repetition import (
    row_groups,
    anchor_of_row,
    anchor_tokens,
    spatial_similarity,
    select_repetitive_heads,
    anchor_attention,
)
from .sharing import (
    kept_from_csr_sets,
    skipped_sets,
    iou_matrix,
    cluster_timesteps,
    share_timesteps,
)

__all__ = [
    "dense_attention",
    "sparse_attention_gather",
    "sparse_attention_masked_dense",
    "sparse_attention_rows",
    "csr_to_block_mask",
    "block_mass",
    "block_mass_rows",
    "topk_keep",
    "agreement",
    "min_agree_count",
    "to_csr",
    "compile_masks",
    "mass_fixed",
    "energy_keep",
    "compile_masks_energy",
    "lpt_work_order",
    "kept_from_csr_sets",
    "skipped_sets",
    "iou_matrix",
    "cluster_timesteps",
    "share_timesteps",
    "row_intervals",
    "width_percentile",
    "merge_row",
    "encode_skip_lists",
    "decode_skip_lists",
    "row_groups",
    "anchor_of_row",
    "anchor_tokens",
    "spatial_similarity",
    "select_repetitive_heads",
    "anchor_attention",
]
