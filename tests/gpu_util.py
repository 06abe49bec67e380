"""Helpers shared by the GPU parity tests (no method arithmetic here)."""

import sys

import numpy as np
import torch

import synth
from synth.configs import Config


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x, dtype, device="cuda:0"):
    """float32 numpy array (bf16-exact for bf16) -> GPU tensor of `dtype`."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device).to(dtype).contiguous()


def i32(x, device="cuda:0"):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(device)


def small_cfg(B=1, H=2, L=1024, S=1000, d=128, block=128, dtype="bf16", seed=5, grid=None):
    return Config("small", B=B, H=H, L=L, S=S, d=d, block=block, dtype=dtype, data_seed=seed,
                  mask_seed=seed + 1, grid=grid)


def inputs(cfg, seed=None):
    q, k, v = synth.gen_qkv(cfg, seed)
    return q, k, v


def err(gpu_out, ref):
    g = gpu_out.float().cpu().numpy().astype(np.float64)
    return float(np.max(np.abs(g - ref))) if ref.size else 0.0
