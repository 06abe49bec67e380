"""GPU parity: block-sparse and dense attention forward vs the float64 oracle.

Tolerances: max |O_gpu - O_oracle| <= 1e-4 for float32 inputs and <= 2e-2 for
bfloat16 inputs (float32 accumulation; probabilities and O rounded to bf16)."""

import numpy as np
import pytest
import torch

import oracle
import synth
import block_sparse_attention_calibatt_amd as cal
from tests.gpu_util import say, to_dev, i32, small_cfg, inputs, err

pytestmark = pytest.mark.gpu
TOL = {"bf16": 2e-2, "f32": 1e-4}
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


def run_sparse(q, k, v, rp, ci, cfg, work_order=None, persistent=False):
    dt = TDT[cfg.dtype]
    Q, K, V = (to_dev(x, dt) for x in (q, k, v))
    O = torch.full_like(Q, float("nan"))
    RP, CI = i32(rp), i32(ci if len(ci) else np.zeros(1, np.int32))[: len(ci)]
    WO = None if work_order is None else i32(work_order)
    qws = cal.new_queue("cuda:0") if persistent else None
    cal.calibatt_sparse_attn_fwd(Q, K, V, O, RP, CI, cfg.block, cfg.scale, cfg.S, WO, qws)
    torch.cuda.synchronize()
    return O


def as_order(perm):
    """A row permutation with an even 8-way split, in the work-order format."""
    rows = len(perm)
    return np.concatenate([perm, np.linspace(0, rows, 9).astype(np.int64)]).astype(np.int32)


def run_dense(q, k, v, cfg, persistent=False):
    dt = TDT[cfg.dtype]
    Q, K, V = (to_dev(x, dt) for x in (q, k, v))
    O = torch.full_like(Q, float("nan"))
    cal.calibatt_dense_attn_fwd(Q, K, V, O, cfg.block, cfg.scale, cfg.S,
                                cal.new_queue("cuda:0") if persistent else None)
    torch.cuda.synchronize()
    return O


def test_tiny_f32_config(gpu):
    cfg = synth.get_config("tiny")
    say("case: tiny f32 config", cfg)
    q, k, v = inputs(cfg)
    rp, ci = synth.csr_for_config(cfg)
    ref = oracle.sparse_attention_gather(q, k, v, rp, ci, cfg.block, cfg.scale, cfg.S)
    for persistent in (False, True):
        O = run_sparse(q, k, v, rp, ci, cfg, persistent=persistent)
        e = err(O, ref)
        say(f"  persistent={persistent} max err {e:.3e}")
        assert e <= TOL["f32"]


SHAPES = [
    # B, H, L, S, d, block, dtype
    (1, 2, 1024, 1000, 128, 128, "bf16"),
    (2, 1, 768, 700, 128, 128, "bf16"),
    (1, 2, 512, 449, 64, 64, "bf16"),
    (1, 2, 1024, 1000, 128, 64, "bf16"),
    (1, 2, 1024, 1000, 64, 128, "bf16"),
    (1, 2, 512, 449, 64, 64, "f32"),
    (1, 1, 512, 500, 128, 128, "f32"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_sparse_small(gpu, shape):
    B, H, L, S, d, block, dtype = shape
    cfg = small_cfg(B=B, H=H, L=L, S=S, d=d, block=block, dtype=dtype, grid=(4, 8, 16) if dtype == "bf16" else None)
    say("case: sparse small", shape)
    q, k, v = inputs(cfg)
    rng = np.random.default_rng(sum(shape[:6]))
    rp, ci = synth.random_csr(rng, H, L // block, cfg.nkb_valid, 0.4, empty_rows=1, full_rows=1)
    ref = oracle.sparse_attention_gather(q, k, v, rp, ci, block, cfg.scale, S)
    for persistent in (False, True):
        O = run_sparse(q, k, v, rp, ci, cfg, persistent=persistent)
        e = err(O, ref)
        say(f"  persistent={persistent} max err {e:.3e}")
        assert e <= TOL[dtype]


@pytest.mark.parametrize("shape", SHAPES[:3] + SHAPES[5:6], ids=lambda s: "x".join(map(str, s)))
def test_dense_small(gpu, shape):
    B, H, L, S, d, block, dtype = shape
    cfg = small_cfg(B=B, H=H, L=L, S=S, d=d, block=block, dtype=dtype)
    say("case: dense small", shape)
    q, k, v = inputs(cfg)
    ref = oracle.dense_attention(q, k, v, cfg.scale, S)
    for persistent in (False, True):
        O = run_dense(q, k, v, cfg, persistent)
        e = err(O, ref)
        say(f"  persistent={persistent} max err {e:.3e}")
        assert e <= TOL[dtype]


def test_all_kept_sparse_is_dense_bitwise(gpu):
    cfg = small_cfg(H=3, L=1024, S=1000)
    say("case: all-kept sparse vs dense, bitwise")
    q, k, v = inputs(cfg)
    nqb, nkv = cfg.nqb, cfg.nkb_valid
    rp = (np.arange(cfg.rows + 1) * nkv).astype(np.int32)
    ci = np.tile(np.arange(nkv), cfg.rows).astype(np.int32)
    a = run_sparse(q, k, v, rp, ci, cfg)
    b = run_dense(q, k, v, cfg)
    c = run_dense(q, k, v, cfg, persistent=True)
    assert torch.equal(a, b) and torch.equal(a, c)


@pytest.mark.parametrize("B", [1, 2])
def test_schedule_invariance_bitwise(gpu, B):
    cfg = small_cfg(B=B, H=4, L=2048, S=2040)
    say(f"case: work order / persistence invariance, B={B}")
    q, k, v = inputs(cfg)
    rng = np.random.default_rng(9)
    rp, ci = synth.random_csr(rng, cfg.H, cfg.nqb, cfg.nkb_valid, 0.3, empty_rows=2, full_rows=2)
    base = run_sparse(q, k, v, rp, ci, cfg)
    lpt = oracle.lpt_work_order(rp, cfg.H, cfg.nqb)
    orders = [lpt, as_order(lpt[:cfg.rows][::-1]), as_order(rng.permutation(cfg.rows))]
    for wo in orders:
        for persistent in (False, True):
            o = run_sparse(q, k, v, rp, ci, cfg, work_order=wo, persistent=persistent)
            assert torch.equal(o, base)
    again = run_sparse(q, k, v, rp, ci, cfg)
    assert torch.equal(again, base), "repeat run"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_transpose_v_exact(gpu, dtype, d):
    """V [B,H,L,d] -> V^T [B,H,d,L]: a pure layout change, keys >= seq_len zeroed."""
    cfg = small_cfg(B=2, H=3, L=640, S=601, d=d, block=64, dtype=dtype)
    say("case: V transpose", dtype, d)
    _, _, v = inputs(cfg)
    V = to_dev(v, TDT[dtype])
    Vt = cal.calibatt_transpose_v(V, seq_len=cfg.S)
    torch.cuda.synchronize()
    want = np.swapaxes(V.float().cpu().numpy(), 2, 3).copy()
    want[:, :, :, cfg.S:] = 0.0
    assert np.array_equal(Vt.float().cpu().numpy(), want)


@pytest.mark.parametrize("d,block,dtype", [(128, 128, "bf16"), (64, 128, "bf16"), (128, 64, "bf16"),
                                           (64, 64, "bf16"), (64, 64, "f32")])
def test_v_transposed_input_bitwise(gpu, d, block, dtype):
    """Passing V^T gives the same bits as passing V: the kernels read either
    layout into the same matrix-core operands."""
    cfg = small_cfg(H=3, L=1024, S=1000, d=d, block=block, dtype=dtype)
    say("case: V^T input == V input, bitwise", d, block, dtype)
    q, k, v = inputs(cfg)
    rng = np.random.default_rng(17)
    rp, ci = synth.random_csr(rng, cfg.H, cfg.nqb, cfg.nkb_valid, 0.5, empty_rows=1, full_rows=1)
    Q, K, V = (to_dev(x, TDT[dtype]) for x in (q, k, v))
    RP, CI = i32(rp), i32(ci)
    O1, O2 = torch.empty_like(Q), torch.empty_like(Q)
    cal.calibatt_sparse_attn_fwd(Q, K, V, O1, RP, CI, cfg.block, cfg.scale, cfg.S)
    Vt = cal.calibatt_transpose_v(V, seq_len=cfg.S)
    cal.calibatt_sparse_attn_fwd(Q, K, Vt, O2, RP, CI, cfg.block, cfg.scale, cfg.S, v_transposed=True)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2)


@pytest.mark.parametrize("d,block,dtype", [(128, 128, "bf16"), (64, 64, "bf16"), (64, 64, "f32")])
def test_nan_padding_rows(gpu, d, block, dtype):
    """Padded rows of Q, K and V (tokens >= seq_len) holding NaN: padded O rows
    are still zero, and the valid rows equal those of zero padding bit for bit."""
    cfg = small_cfg(H=2, L=1024, S=1000, d=d, block=block, dtype=dtype)
    say("case: NaN in the padding of Q, K, V", d, block, dtype)
    q, k, v = inputs(cfg)
    rng = np.random.default_rng(29)
    rp, ci = synth.random_csr(rng, cfg.H, cfg.nqb, cfg.nkb_valid, 0.5, empty_rows=1, full_rows=1)
    RP, CI = i32(rp), i32(ci)
    outs = []
    for fill in (0.0, float("nan")):
        Q, K, V = (to_dev(x, TDT[dtype]) for x in (q, k, v))
        for t in (Q, K, V):
            t[:, :, cfg.S:] = fill
        for persistent in (False, True):
            O = torch.full_like(Q, 3.0)
            cal.calibatt_sparse_attn_fwd(Q, K, V, O, RP, CI, cfg.block, cfg.scale, cfg.S, None,
                                         cal.new_queue("cuda:0") if persistent else None)
            torch.cuda.synchronize()
            assert torch.count_nonzero(O[:, :, cfg.S:].float()).item() == 0
            outs.append(O)
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_row_lengths_one_to_nine_blocks(gpu):
    """Rows of 0..9 kept blocks: every remainder of the sub-tile pipeline."""
    cfg = small_cfg(H=2, L=2048, S=2000)
    say("case: row lengths 0..9 blocks")
    q, k, v = inputs(cfg)
    rng = np.random.default_rng(23)
    rows, counts = [], []
    for r in range(cfg.rows):
        c = r % 10
        counts.append(c)
        rows.append(np.sort(rng.choice(cfg.nkb_valid, size=c, replace=False)))
    rp = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    ci = np.concatenate(rows).astype(np.int32)
    ref = oracle.sparse_attention_gather(q, k, v, rp, ci, cfg.block, cfg.scale, cfg.S)
    for persistent in (False, True):
        O = run_sparse(q, k, v, rp, ci, cfg, persistent=persistent)
        e = err(O, ref)
        say(f"  persistent={persistent} max err {e:.3e}")
        assert e <= TOL["bf16"]


def test_empty_mask(gpu):
    cfg = small_cfg(H=1, L=512, S=512)
    say("case: every row empty")
    q, k, v = inputs(cfg)
    rp = np.zeros(cfg.rows + 1, np.int32)
    ci = np.zeros(0, np.int32)
    O = run_sparse(q, k, v, rp, ci, cfg, persistent=True)
    assert torch.count_nonzero(O.float()).item() == 0


def test_lone_valid_key(gpu):
    """S = 449, block 64: rows keeping only the last block return v[448]."""
    cfg = small_cfg(H=1, L=512, S=449, d=64, block=64)
    say("case: lone valid key")
    q, k, v = inputs(cfg)
    rp = np.arange(cfg.rows + 1).astype(np.int32)
    ci = np.full(cfg.rows, 7, np.int32)
    O = run_sparse(q, k, v, rp, ci, cfg)
    want = torch.from_numpy(v[0, 0, 448]).to(torch.bfloat16)
    got = O[0, 0, :449].cpu()
    assert torch.equal(got, want.expand_as(got))
    assert torch.count_nonzero(O[0, 0, 449:].float()).item() == 0


def test_single_valid_token(gpu):
    """seq_len = 1 in one 128-token block: every valid row attends to key 0 only,
    so its output is V[0] exactly (after bf16 rounding of O); padded rows are zero."""
    cfg = small_cfg(H=2, L=128, S=1, d=128, block=128)
    say("case: seq_len 1")
    q, k, v = inputs(cfg)
    rp = np.arange(cfg.rows + 1).astype(np.int32)
    ci = np.zeros(cfg.rows, np.int32)
    for persistent in (False, True):
        O = run_sparse(q, k, v, rp, ci, cfg, persistent=persistent)
        Od = run_dense(q, k, v, cfg, persistent=persistent)
        for out in (O, Od):
            want = torch.from_numpy(v[0, :, 0]).to(torch.bfloat16)
            assert torch.equal(out[0, :, 0].cpu(), want)
            assert torch.count_nonzero(out[0, :, 1:].float()).item() == 0


def _sample_items(cfg, rng, n):
    items = [(0, 0, 0), (0, cfg.H - 1, cfg.nqb - 1)]
    while len(items) < n:
        items.append((int(rng.integers(cfg.B)), int(rng.integers(cfg.H)), int(rng.integers(cfg.nqb))))
    return items


def _head_ref(q, k, v, rp, ci, cfg, b, h, qbs):
    """Oracle rows qbs of head h, batch entry b, computed from that head's
    arrays (float64) and its slice of the kept lists alone."""
    r0 = h * cfg.nqb
    base = int(rp[r0])
    rp_h = (np.asarray(rp[r0:r0 + cfg.nqb + 1], dtype=np.int64) - base)
    ci_h = np.asarray(ci[base:int(rp[r0 + cfg.nqb])])
    qh, kh, vh = (np.asarray(x[b:b + 1, h:h + 1], dtype=np.float64) for x in (q, k, v))
    return oracle.sparse_attention_rows(qh, kh, vh, rp_h, ci_h, cfg.block, cfg.scale, cfg.S,
                                        [(0, 0, qb) for qb in qbs])


def _length_class_rows(rp):
    """Rows by kept count: the longest, the first and last empty ones, and for
    T = 64, 128, 192 (the kernel reads a row's list 64 entries at a time) a
    row with exactly T and T + 1 entries and the shortest row above T."""
    cnt = np.diff(np.asarray(rp, dtype=np.int64))
    picks = {int(np.argmax(cnt))}
    empty = np.nonzero(cnt == 0)[0]
    if len(empty):
        picks.update((int(empty[0]), int(empty[-1])))
    for T in (64, 128, 192):
        for want in (T, T + 1):
            ex = np.nonzero(cnt == want)[0]
            if len(ex):
                picks.add(int(ex[0]))
        above = np.nonzero(cnt > T)[0]
        if len(above):
            picks.add(int(above[np.argmin(cnt[above])]))
    return sorted(picks)


def _compare_rows(O, cfg, b, h, qbs, ref):
    worst = 0.0
    for qb, rr in zip(qbs, ref):
        g = O[b, h, qb * cfg.block:(qb + 1) * cfg.block].float().cpu().numpy()
        worst = max(worst, float(np.max(np.abs(g - rr))))
    return worst


def _full_size_check(cfg, rp, ci, seed_items, n_items, tol=2e-2):
    """The persistent longest-first launch at full size against the oracle:
    every row of the heaviest head, rows chosen by length class over the whole
    mask, and sampled rows; padded rows zero, everything finite."""
    q, k, v = inputs(cfg)
    wo = oracle.lpt_work_order(rp, cfg.H, cfg.nqb)
    O = run_sparse(q, k, v, rp, ci, cfg, work_order=wo, persistent=True)
    per_head = np.diff(np.asarray(rp, dtype=np.int64)[::cfg.nqb])
    hw = int(np.argmax(per_head))
    worst = _compare_rows(O, cfg, 0, hw, range(cfg.nqb), _head_ref(q, k, v, rp, ci, cfg, 0, hw, range(cfg.nqb)))
    say(f"  whole head {hw} ({cfg.nqb} query blocks, {int(per_head[hw])} kept), max err {worst:.3e}")
    assert worst <= tol
    classes = _length_class_rows(rp)
    cnt = np.diff(np.asarray(rp, dtype=np.int64))
    worst = 0.0
    for r in classes:
        h, qb = divmod(r, cfg.nqb)
        worst = max(worst, _compare_rows(O, cfg, 0, h, [qb], _head_ref(q, k, v, rp, ci, cfg, 0, h, [qb])))
    say(f"  length-class rows {[(r, int(cnt[r])) for r in classes]}, max err {worst:.3e}")
    assert worst <= tol
    items = _sample_items(cfg, np.random.default_rng(seed_items), n_items)
    ref = oracle.sparse_attention_rows(q, k, v, rp, ci, cfg.block, cfg.scale, cfg.S, items)
    worst = 0.0
    for (b, h, qb), rr in zip(items, ref):
        g = O[b, h, qb * cfg.block:(qb + 1) * cfg.block].float().cpu().numpy()
        worst = max(worst, float(np.max(np.abs(g - rr))))
    say(f"  {len(items)} sampled query blocks, max err {worst:.3e}")
    assert worst <= tol
    tail = O[:, :, cfg.S:].float()
    assert torch.count_nonzero(tail).item() == 0, "padded rows must be zero"
    assert torch.isfinite(O.float()).all()


def test_wan_full_size(gpu):
    cfg = synth.get_config("wan")
    say("case: Wan full size, persistent + longest-first order")
    rp, ci = synth.csr_for_config(cfg)
    _full_size_check(cfg, rp, ci, 11, 24)


def test_wan720_full_size(gpu):
    cfg = synth.get_config("wan720")
    say("case: Wan 720p full size (591 blocks per head)")
    rp, ci = synth.csr_for_config(cfg)
    _full_size_check(cfg, rp, ci, 51, 12)


def test_mochi_full_size(gpu):
    cfg = synth.get_config("mochi")
    say("case: Mochi full size")
    rp, ci = synth.csr_for_config(cfg)
    _full_size_check(cfg, rp, ci, 21, 24)


def test_imbalance_sets(gpu):
    cfg = synth.get_config("imbalance")
    for t in (0, 49):
        say(f"case: imbalance set {t}")
        rp, ci = synth.csr_for_config(cfg, t)
        _full_size_check(cfg, rp, ci, 31 + t, 12)


def test_mochi_dense_sampled(gpu):
    cfg = synth.get_config("mochi")
    say("case: Mochi dense, sampled rows")
    q, k, v = inputs(cfg)
    O = run_dense(q, k, v, cfg, persistent=True)
    nkv = cfg.nkb_valid
    rp = (np.arange(cfg.rows + 1) * nkv).astype(np.int32)
    ci = np.tile(np.arange(nkv), cfg.rows).astype(np.int32)
    items = _sample_items(cfg, np.random.default_rng(5), 6)
    ref = oracle.sparse_attention_rows(q, k, v, rp, ci, cfg.block, cfg.scale, cfg.S, items)
    worst = max(float(np.max(np.abs(O[b, h, qb * 128:(qb + 1) * 128].float().cpu().numpy() - rr)))
                for (b, h, qb), rr in zip(items, ref))
    say(f"  max err {worst:.3e}")
    assert worst <= 2e-2


def test_wan_dense_whole_head(gpu):
    """The Wan-size dense launch: every row of one head against the oracle."""
    cfg = synth.get_config("wan")
    say("case: Wan dense, whole head 17")
    q, k, v = inputs(cfg)
    O = run_dense(q, k, v, cfg, persistent=True)
    nkv = cfg.nkb_valid
    rp = (np.arange(cfg.rows + 1) * nkv).astype(np.int64)
    ci = np.tile(np.arange(nkv), cfg.rows).astype(np.int32)
    h = 17
    worst = _compare_rows(O, cfg, 0, h, range(cfg.nqb), _head_ref(q, k, v, rp, ci, cfg, 0, h, range(cfg.nqb)))
    say(f"  max err {worst:.3e}")
    assert worst <= 2e-2
    assert torch.count_nonzero(O[:, :, cfg.S:].float()).item() == 0
