"""GPU parity at the size limits the C ABI accepts.

* Sparse forward with B*H*L*d just under 2^31 (the limit the host checks):
  H = 127 heads of L = 131,072 tokens, d = 128, a ragged tail (S = L - 37),
  ~1.5% random kept blocks with empty rows and rows keeping all 1,024 valid
  blocks (the longest list a row can hold), launched as the benchmark does
  (persistent grid, longest-first work order).  Sampled rows against the
  oracle, including the last row of the last head (the largest offsets).
* Both calibration pooling methods at the largest key-block count the
  pooling kernels keep in LDS (1,024 blocks of 128: L = 131,072), with a
  ragged tail: every query block's mass row sums to its valid query count,
  and sampled rows match the oracle.

Inputs come from the seeded per-head generator, so a head regenerated on
the host for the oracle is bit for bit the one uploaded."""

import numpy as np
import pytest
import torch

import oracle
import synth
import block_sparse_attention_calibatt_amd as cal
from synth.configs import Config
from tests.gpu_util import say, i32, err

pytestmark = pytest.mark.gpu


def _upload_heads(cfg, dev, chunk=16):
    """Q, K, V bf16 [1, H, L, d] on the GPU, generated and uploaded chunk by chunk of heads."""
    shape = (cfg.B, cfg.H, cfg.L, cfg.d)
    Q, K, V = (torch.empty(shape, dtype=torch.bfloat16, device=dev) for _ in range(3))
    for h0 in range(0, cfg.H, chunk):
        heads = list(range(h0, min(cfg.H, h0 + chunk)))
        q, k, v = synth.gen_qkv(cfg, heads=heads)
        for T, x in ((Q, q), (K, k), (V, v)):
            T[:, heads[0]:heads[-1] + 1] = torch.from_numpy(x).to(dev).to(torch.bfloat16)
        del q, k, v
    return Q, K, V


class _Heads:
    """[b, h] -> float32 [L, d] of the generator's head h (for the oracle's row form).
    The Q, K and V views share one cache of regenerated heads."""

    def __init__(self, cfg, which, cache):
        self.cfg, self.which, self.cache = cfg, which, cache

    def __getitem__(self, bh):
        b, h = bh
        if h not in self.cache:
            self.cache[h] = synth.gen_qkv(self.cfg, heads=[h])
        return self.cache[h][self.which][b, 0]


@pytest.mark.timeout(900)
def test_sparse_forward_largest_tensors(gpu):
    cfg = Config("max", B=1, H=127, L=131072, S=131072 - 37, d=128, block=128, dtype="bf16",
                 data_seed=61, mask_seed=62)
    assert cfg.B * cfg.H * cfg.L * cfg.d < 2 ** 31
    say(f"case: sparse forward at B*H*L*d = {cfg.B * cfg.H * cfg.L * cfg.d} (limit 2^31), "
        f"H={cfg.H} L={cfg.L} S={cfg.S} nqb={cfg.nqb}")
    rng = np.random.default_rng(cfg.mask_seed)
    rp, ci = synth.random_csr(rng, cfg.H, cfg.nqb, cfg.nkb_valid, 0.015, empty_rows=3, full_rows=2)
    cal.calibatt_validate_csr(rp, ci, cfg.rows, cfg.nkb_valid)
    lens = np.diff(rp)
    full = [int(r) for r in np.nonzero(lens == cfg.nkb_valid)[0]]
    empty = [int(r) for r in np.nonzero(lens == 0)[0]]
    say(f"  kept blocks {len(ci)}, full rows {full}, empty rows {empty[:3]}")
    Q, K, V = _upload_heads(cfg, "cuda:0")
    O = torch.full_like(Q, float("nan"))
    RP, CI = i32(rp), i32(ci)
    wo = cal.calibatt_build_schedule(RP, cfg.H, cfg.nqb)
    cal.calibatt_sparse_attn_fwd(Q, K, V, O, RP, CI, cfg.block, cfg.scale, cfg.S, wo, cal.new_queue("cuda:0"))
    torch.cuda.synchronize()
    rows = [0, cfg.rows - 1] + full + empty[:1] + [int(r) for r in rng.integers(0, cfg.rows, size=3)]
    items = [(0, r // cfg.nqb, r % cfg.nqb) for r in rows]
    cache = {}
    ref = oracle.sparse_attention_rows(_Heads(cfg, 0, cache), _Heads(cfg, 1, cache), _Heads(cfg, 2, cache), rp, ci,
                                       cfg.block, cfg.scale, cfg.S, items)
    worst = 0.0
    for n, (b, h, qb) in enumerate(items):
        got = O[b, h, qb * cfg.block:(qb + 1) * cfg.block]
        e = err(got, ref[n])
        worst = max(worst, e)
        say(f"  row (h={h}, qb={qb}) kept {int(lens[h * cfg.nqb + qb])}: max err {e:.3e}")
    assert worst <= 2e-2
    # query rows past S are zero in the last block of every head
    tail = O[0, :, cfg.S:].float()
    assert torch.count_nonzero(tail).item() == 0


@pytest.mark.timeout(600)
@pytest.mark.parametrize("method", ["two_pass", "single_pass"])
def test_block_mass_most_key_blocks(gpu, method):
    cfg = Config("maxkb", B=1, H=2, L=131072, S=131072 - 5, d=128, block=128, dtype="bf16",
                 data_seed=63, mask_seed=0)
    assert cfg.nkb == 1024
    say(f"case: block mass {method} at {cfg.nkb} key blocks, S={cfg.S}")
    q, k = synth.gen_qk(cfg, cfg.data_seed)
    Q, K = (torch.from_numpy(x).to("cuda:0").to(torch.bfloat16) for x in (q, k))
    lse = torch.empty(cfg.B * cfg.H * cfg.L, dtype=torch.float32, device="cuda:0")
    mass = torch.full((cfg.B, cfg.H, cfg.nqb, cfg.nkb), float("nan"), dtype=torch.float32, device="cuda:0")
    if method == "two_pass":
        cal.calibatt_block_mass(Q, K, cfg.block, cfg.scale, lse, mass, cfg.S)
    else:
        cal.calibatt_block_mass_single_pass(Q, K, cfg.block, cfg.scale, lse, mass, cfg.S)
    torch.cuda.synchronize()
    m = mass.cpu().numpy().astype(np.float64)
    valid_q = np.minimum((np.arange(cfg.nqb) + 1) * cfg.block, cfg.S) - np.arange(cfg.nqb) * cfg.block
    sums = m.sum(axis=-1)
    assert np.all(np.abs(sums - valid_q) <= 1e-3 * valid_q), "mass rows sum to the valid query count"
    for h, qb in [(0, 0), (1, cfg.nqb - 1), (1, 517)]:
        ref = oracle.block_mass_rows(q[0, h], k[0, h], cfg.block, cfg.scale, cfg.S, qb)
        excess = np.abs(m[0, h, qb] - ref) - (1e-3 * np.abs(ref) + 1e-6)
        say(f"  row (h={h}, qb={qb}): worst excess over tolerance {excess.max():.2e}")
        assert np.all(excess <= 0)
