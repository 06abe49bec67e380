"""The sparse forward without a queue workspace (its counters in the
library's static scratch) against calibatt_sparse_attn_fwd with a queue
workspace: bit-identical output, two calls in a row, the second smaller, so
that the second call starts from the counters the first one left."""

import numpy as np
import pytest
import torch

import synth
import block_sparse_attention_calibatt_amd as cal
from tests.gpu_util import say, to_dev, i32, small_cfg, inputs

pytestmark = pytest.mark.gpu
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}

# (B, H, L, S, d, block, dtype): a larger call, then a smaller one
PAIRS = [
    ((1, 6, 2048, 1990, 128, 128, "bf16"), (1, 2, 1024, 1000, 128, 128, "bf16")),
    ((2, 3, 1024, 1000, 64, 128, "bf16"), (1, 1, 512, 400, 64, 128, "bf16")),
    ((1, 4, 1024, 1000, 128, 64, "bf16"), (1, 2, 512, 449, 128, 64, "bf16")),
    ((1, 3, 1024, 1000, 64, 64, "f32"), (1, 1, 256, 200, 64, 64, "f32")),
]


def _case(shape, seed, v_transposed):
    B, H, L, S, d, block, dtype = shape
    cfg = small_cfg(B=B, H=H, L=L, S=S, d=d, block=block, dtype=dtype, seed=seed)
    q, k, v = inputs(cfg)
    rng = np.random.default_rng(seed)
    rp, ci = synth.random_csr(rng, H, L // block, cfg.nkb_valid, 0.35, empty_rows=1, full_rows=1)
    dt = TDT[dtype]
    Q, K, V = (to_dev(x, dt) for x in (q, k, v))
    if v_transposed:
        V = V.transpose(2, 3).contiguous()
    RP = i32(rp)
    CI = i32(ci if len(ci) else np.zeros(1, np.int32))[: len(ci)]
    WO = cal.calibatt_build_schedule(RP, H, L // block)
    return cfg, Q, K, V, RP, CI, WO


def _both(cfg, Q, K, V, RP, CI, WO, v_transposed):
    ref = torch.full_like(Q, float("nan"))
    cal.calibatt_sparse_attn_fwd(Q, K, V, ref, RP, CI, cfg.block, cfg.scale, cfg.S, WO, cal.new_queue(Q.device),
                                 v_transposed=v_transposed)
    out = torch.full_like(Q, float("nan"))
    before = torch.cuda.memory_allocated()
    cal.calibatt_sparse_attn_fwd_noalloc(Q, K, V, out, RP, CI, cfg.block, cfg.scale, cfg.S, WO,
                                         v_transposed=v_transposed)
    assert torch.cuda.memory_allocated() == before
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: "x".join(map(str, p[0])))
@pytest.mark.parametrize("v_transposed", [False, True])
def test_noalloc_matches_workspace_call(gpu, pair, v_transposed):
    for i, shape in enumerate(pair):
        say("case: noalloc", shape, "v_transposed", v_transposed, "call", i)
        cfg, Q, K, V, RP, CI, WO = _case(shape, 31 + i, v_transposed)
        ref, out = _both(cfg, Q, K, V, RP, CI, WO, v_transposed)
        assert not torch.isnan(ref).any()
        assert torch.equal(out.view(torch.int16 if cfg.dtype == "bf16" else torch.int32),
                           ref.view(torch.int16 if cfg.dtype == "bf16" else torch.int32)), f"call {i} differs"


def test_noalloc_natural_order_and_empty_list(gpu):
    """No work order (natural partition), then a call whose list keeps no
    block at all: every row is written as zero."""
    cfg, Q, K, V, RP, CI, _ = _case((1, 5, 1024, 1000, 128, 128, "bf16"), 77, False)
    say("case: noalloc natural order")
    ref = torch.full_like(Q, float("nan"))
    cal.calibatt_sparse_attn_fwd(Q, K, V, ref, RP, CI, cfg.block, cfg.scale, cfg.S, None, cal.new_queue(Q.device))
    out = torch.full_like(Q, float("nan"))
    cal.calibatt_sparse_attn_fwd_noalloc(Q, K, V, out, RP, CI, cfg.block, cfg.scale, cfg.S)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    say("case: noalloc empty list")
    H, nqb = 2, 4
    cfg2, Q2, K2, V2, _, _, _ = _case((1, H, 512, 500, 128, 128, "bf16"), 78, False)
    RP2 = torch.zeros(H * nqb + 1, dtype=torch.int32, device=Q2.device)
    CI2 = torch.zeros(0, dtype=torch.int32, device=Q2.device)
    out2 = torch.full_like(Q2, float("nan"))
    cal.calibatt_sparse_attn_fwd_noalloc(Q2, K2, V2, out2, RP2, CI2, 128, cfg2.scale, cfg2.S)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out2).item() == 0
