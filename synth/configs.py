"""The synthetic workloads.

* ``tiny``      - 1 head, d=64, 512 tokens (2 frames x 256), 64-token blocks,
                  float32, i.i.d. N(0,1) inputs; mask = the 8 diagonal blocks
                  plus 28 of the 56 off-diagonal blocks.
* ``wan``       - one Wan 2.1 14B attention call: B=1, 40 heads, d=128,
                  32,760 valid tokens (21 frames x 30 rows x 52 columns) padded
                  to 32,768, bfloat16, 128-token blocks; structured ~30% masks.
* ``wan720``    - the Wan call at 720p: 75,600 valid tokens (21 frames x 45
                  rows x 80 columns) padded to 75,648 (591 blocks), structured
                  masks at 37.5% kept (the 62.5% sparsity of the pages' 720p
                  rows, Table S3).
* ``mochi``     - B=1, 24 heads, d=128, 16,384 tokens (16 x 32 x 32 grid),
                  bfloat16, 128-token blocks; band + random rows of exactly 26
                  kept blocks (20.3%).
* ``imbalance`` - Wan shape; 50 mask sets (one per diffusion timestep) with
                  per-head densities U(5%, 90%) and Zipf-skewed row counts.
* ``calib``     - Wan shape; 8 calibration prompts (seeds 100..107) pooled into
                  block mass, top 25% key blocks per query block, agreement
                  >= 1/2 across prompts, then inference on a 9th input (seed 108).
"""

from dataclasses import dataclass, field
from fractions import Fraction
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    L: int            # padded token count (multiple of block)
    S: int            # valid tokens; tokens >= S are padding
    d: int
    block: int
    dtype: str        # "bf16" or "f32"
    data_seed: int
    mask_seed: int
    grid: Optional[Tuple[int, int, int]] = None   # (frames, rows, cols) of the positional term
    n_sets: int = 1                               # mask sets (timesteps)
    prompt_seeds: Tuple[int, ...] = field(default_factory=tuple)
    infer_seed: Optional[int] = None
    keep_frac: Fraction = Fraction(1, 4)
    rho: Fraction = Fraction(1, 2)

    @property
    def nqb(self) -> int:
        return self.L // self.block

    @property
    def nkb(self) -> int:
        return self.L // self.block

    @property
    def nkb_valid(self) -> int:
        return -(-self.S // self.block)

    @property
    def rows(self) -> int:
        return self.H * self.nqb

    @property
    def scale(self) -> float:
        return 1.0 / float(self.d) ** 0.5


CONFIGS = {
    "tiny": Config("tiny", B=1, H=1, L=512, S=512, d=64, block=64, dtype="f32",
                   data_seed=0, mask_seed=1, grid=None),
    "wan": Config("wan", B=1, H=40, L=32768, S=32760, d=128, block=128, dtype="bf16",
                  data_seed=10, mask_seed=11, grid=(21, 30, 52)),
    "mochi": Config("mochi", B=1, H=24, L=16384, S=16384, d=128, block=128, dtype="bf16",
                    data_seed=20, mask_seed=21, grid=(16, 32, 32)),
    # 720p: 21 latent frames of 45 x 80 tokens (75,600, padded to 591 blocks),
    # structured masks at the pages' 720p sparsity (62.5% skipped, Table S3)
    "wan720": Config("wan720", B=1, H=40, L=75648, S=75600, d=128, block=128, dtype="bf16",
                     data_seed=50, mask_seed=51, grid=(21, 45, 80)),
    "imbalance": Config("imbalance", B=1, H=40, L=32768, S=32760, d=128, block=128,
                        dtype="bf16", data_seed=30, mask_seed=1000, grid=(21, 30, 52),
                        n_sets=50),
    "calib": Config("calib", B=1, H=40, L=32768, S=32760, d=128, block=128, dtype="bf16",
                    data_seed=108, mask_seed=0, grid=(21, 30, 52),
                    prompt_seeds=tuple(range(100, 108)), infer_seed=108),
}


def get_config(name: str) -> Config:
    return CONFIGS[name]
