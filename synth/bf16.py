"""Round-to-nearest-even conversion between float32 and bfloat16 bit patterns.

bfloat16 keeps the top 16 bits of an IEEE float32.  Rounding to nearest, ties
to even, adds 0x7FFF plus the lowest kept bit before truncating.  Inputs here
are finite Gaussian draws, so NaN and overflow handling are not needed.
"""

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bfloat16 bit patterns (round to nearest even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array -> float32 array holding the nearest bfloat16 values."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))
