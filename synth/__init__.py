"""Seeded synthetic inputs for the block-sparse attention workloads.

This package is shared by the CPU oracle tests, the GPU parity tests and the
benchmark.  It holds no step of the attention or calibration arithmetic: only
random draws, the positional term added to them, rounding to bfloat16, and
the kept key-block lists (CSR) of the benchmark masks.  Neither the oracle nor
the HIP library is imported from here.

Shapes follow the pages' video-transformer workloads (CalibAtt, arXiv
2603.05503): the Wan 2.1 14B attention call is batch 1, 40 heads, head dim
128, 32,760 tokens (Table S4 caption), which is 21 latent frames of 1,560
tokens (Fig. 2 and Fig. 4 captions) laid out as 30 spatial rows (the anchor
sparsities of Table S4 are 1 - k/30) of 52 tokens.
"""

from .bf16 import round_bf16, f32_to_bf16_bits, bf16_bits_to_f32
from .configs import CONFIGS, Config, get_config
from .inputs import gen_qkv, gen_qk, positional_term, repeat_rows
from .masks import (
    tiny_csr,
    wan_csr,
    mochi_csr,
    imbalance_csr,
    random_csr,
    csr_for_config,
    drifting_sets,
)

__all__ = [
    "round_bf16",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "CONFIGS",
    "Config",
    "get_config",
    "gen_qkv",
    "gen_qk",
    "positional_term",
    "repeat_rows",
    "tiny_csr",
    "wan_csr",
    "mochi_csr",
    "imbalance_csr",
    "random_csr",
    "csr_for_config",
    "drifting_sets",
]
