"""The C-ABI library loads, exports what include/calibatt.h declares, and
rejects bad arguments on the host before any GPU work (no GPU needed)."""

import ctypes
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import block_sparse_attention_calibatt_amd as cal
from block_sparse_attention_calibatt_amd import _lib


@pytest.fixture(scope="module")
def lib():
    return cal.load()


def test_exports_every_declared_symbol(lib):
    names = _lib.header_symbols()
    assert len(names) == 26
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in names:
        assert n in exported, f"{n} is declared but not exported"
        getattr(lib, n)
    assert set(_lib.SIGNATURES) == set(names), "binding and header disagree"


def test_version_and_strings(lib):
    assert cal.calibatt_version() == 303
    for code, name in _lib.STATUS.items():
        assert cal.calibatt_status_string(code) != "unknown status"
    assert cal.calibatt_status_string(99) == "unknown status"


V = ctypes.c_void_p
P16, P32, P48, P64 = V(16), V(32), V(48), V(64)     # aligned fake addresses, never dereferenced
# fake Q, K, V, O far enough apart not to overlap at any accepted size
TQ, TK, TV, TO = V(1 << 36), V(2 << 36), V(3 << 36), V(4 << 36)


def _sparse(lib, **kw):
    a = dict(Q=TQ, K=TK, V=TV, O=TO, row_ptr=V(128), col_idx=V(256), block=128, scale=0.1, B=1, H=2,
             L=1024, seq_len=1000, d=128, dt=0, work_order=None, queue_ws=None, nnz=10, v_layout=1, stream=None)
    a.update(kw)
    return lib.calibatt_sparse_attn_fwd(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), 1),
    (dict(O=None), 1),
    (dict(row_ptr=None), 1),
    (dict(col_idx=None), 1),
    (dict(Q=V((1 << 36) + 17)), 4),
    (dict(row_ptr=V(130)), 4),
    (dict(queue_ws=V(132)), 4),
    (dict(dt=7), 3),
    (dict(block=96), 7),
    (dict(d=96), 7),
    (dict(L=1000), 2),
    (dict(seq_len=0), 2),
    (dict(seq_len=1025), 2),
    (dict(B=0), 2),
    (dict(H=-1), 2),
    (dict(B=1024, H=64, L=65536), 2),
    (dict(nnz=-1), 5),
    (dict(nnz=2 * 8 * 8 + 1), 5),
    (dict(v_layout=2), 2),
    (dict(v_layout=-1), 2),
    (dict(scale=0.0), 2),
    (dict(scale=-0.1), 2),
    (dict(scale=float("nan")), 2),
    (dict(scale=float("inf")), 2),
    (dict(O=V((1 << 36) + 4096)), 2),            # O overlaps Q
    (dict(O=V((3 << 36) - 4096)), 2),            # O overlaps K
    (dict(V=V((4 << 36) + 1024 * 128 * 2)), 2),  # V overlaps O
])
def test_sparse_rejects(lib, kw, status):
    assert _sparse(lib, **kw) == status
    assert cal.calibatt_last_error() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), 1),
    (dict(row_ptr=V(130)), 4),
    (dict(block=96), 7),
    (dict(seq_len=1025), 2),
    (dict(nnz=2 * 8 * 8 + 1), 5),
    (dict(v_layout=2), 2),
    (dict(scale=float("nan")), 2),
    (dict(O=V((1 << 36) + 4096)), 2),
])
def test_sparse_noalloc_rejects(lib, kw, status):
    """The variant without a queue workspace checks the same arguments the
    same way, before any HIP call."""
    a = dict(Q=TQ, K=TK, V=TV, O=TO, row_ptr=V(128), col_idx=V(256), block=128, scale=0.1, B=1, H=2,
             L=1024, seq_len=1000, d=128, dt=0, work_order=None, nnz=10, v_layout=1, stream=None)
    a.update(kw)
    assert lib.calibatt_sparse_attn_fwd_noalloc(*a.values()) == status
    assert cal.calibatt_last_error() != ""


def test_dense_and_mass_reject(lib):
    def dense(*a, layout=1):
        return lib.calibatt_dense_attn_fwd(*a, layout, None)
    assert dense(None, TK, TV, TO, 128, 0.1, 1, 1, 256, 256, 128, 0, None) == 1
    assert dense(TQ, TK, TV, TO, 32, 0.1, 1, 1, 256, 256, 128, 0, None) == 7
    assert dense(TQ, TK, TV, TO, 128, 0.1, 1, 1, 256, 256, 128, 0, V(132)) == 4
    assert dense(TQ, TK, TV, TO, 128, 0.1, 1, 1, 256, 256, 128, 0, None, layout=5) == 2
    assert dense(TQ, TK, TV, TO, 128, 0.0, 1, 1, 256, 256, 128, 0, None) == 2
    assert dense(TQ, TK, TV, TO, 128, float("nan"), 1, 1, 256, 256, 128, 0, None) == 2
    assert dense(TQ, TK, TV, TQ, 128, 0.1, 1, 1, 256, 256, 128, 0, None) == 2, "O aliases Q"
    assert lib.calibatt_block_mass(P16, P32, 1, 1, 256, 256, 128, 0, 128, -1.0, P48, P64, None) == 2, "scale"
    assert lib.calibatt_block_mass(P16, P32, 1, 1, 256, 256, 128, 1, 128, 0.1, P48, P64, None) == 7, "f32 mass"
    assert lib.calibatt_block_mass(P16, P32, 1, 1, 256, 300, 128, 0, 128, 0.1, P48, P64, None) == 2
    assert lib.calibatt_block_mass(P16, None, 1, 1, 256, 256, 128, 0, 128, 0.1, P48, P64, None) == 1
    assert lib.calibatt_block_mass(P16, P32, 1, 1, 128 * 2048, 256, 64, 0, 128, 0.1, P48, P64, None) == 7


def test_transpose_rejects(lib):
    def tr(V_, Vt, B=1, H=2, L=1024, S=1000, d=128, dt=0):
        return lib.calibatt_transpose_v(V_, Vt, B, H, L, S, d, dt, None)
    assert tr(None, P32) == 1
    assert tr(P16, None) == 1
    assert tr(V(17), P32) == 4
    assert tr(P16, V(1 << 30), L=1000) == 2
    assert tr(P16, V(1 << 30), d=96) == 7
    assert tr(P16, V(1 << 30), dt=5) == 3
    assert tr(P16, V(1 << 30), S=1025) == 2
    assert tr(P16, V(16 + 1024)) == 2        # in place / overlapping
    assert cal.calibatt_last_error() != ""


def test_compile_and_schedule_reject(lib):
    n = ctypes.c_int64(0)
    ws = lib.calibatt_compile_ws_bytes(8, 40, 256, 256)
    assert ws == 40 * 256 * 256 + 40 * 256 * 4
    assert lib.calibatt_compile_ws_bytes(0, 1, 1, 1) == 0
    base = dict(mass=P16, P=8, H=40, nqb=256, nkb=256, nkb_valid=256, K=64, t=4, row_ptr=P32, col_idx=P48,
                cap=10, wo=None, nnz=ctypes.byref(n), ws=P64, ws_bytes=ws, stream=None)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return lib.calibatt_compile_masks(*a.values())
    assert call(mass=None) == 1
    assert call(P=0) == 2
    assert call(t=9) == 2
    assert call(t=-1) == 2
    assert call(K=-1) == 2
    assert call(nkb_valid=257) == 2
    assert call(nkb=2048, nkb_valid=2048) == 7
    assert call(ws_bytes=ws - 1) == 6
    assert call(ws=V(72)) == 4
    assert call(wo=V(66)) == 4                        # work_order must be 4-byte aligned
    assert call(H=2048, nqb=8, nkb=8, nkb_valid=8, wo=V(80), ws_bytes=1 << 20) == 7   # too many heads to schedule
    ebase = dict(mass=P16, P=8, H=40, nqb=256, nkb=256, nkb_valid=256, num=1, den=20, t=4, row_ptr=P32,
                 col_idx=P48, cap=10, wo=None, nnz=ctypes.byref(n), ws=P64, ws_bytes=ws, stream=None)

    def ecall(**kw):
        a = dict(ebase)
        a.update(kw)
        return lib.calibatt_compile_masks_energy(*a.values())
    assert ecall(mass=None) == 1
    assert ecall(den=0) == 2
    assert ecall(num=-1) == 2
    assert ecall(num=21) == 2
    assert ecall(den=1 << 31, num=0) == 2
    assert ecall(t=9) == 2
    assert ecall(nkb=2048, nkb_valid=2048) == 7
    assert ecall(ws_bytes=ws - 1) == 6
    assert lib.calibatt_build_schedule(None, 1, 1, P16, None) == 1
    assert lib.calibatt_build_schedule(P16, 0, 1, P32, None) == 2
    assert lib.calibatt_build_schedule(P16, 1, 4096, P32, None) == 7
    assert lib.calibatt_build_schedule(P16, 2048, 8, P32, None) == 7


def test_share_reject(lib):
    ws = lib.calibatt_share_ws_bytes(50, 40, 256, 256)
    assert ws > 2 * 50 * 40 * 256 * 8 * 4
    assert lib.calibatt_share_ws_bytes(0, 1, 1, 1) == 0
    c, n = ctypes.c_int32(0), ctypes.c_int64(0)
    W = V(1 << 20)   # 256-byte aligned
    base = dict(row_ptr=P16, col_idx=P32, set_off=P48, T=50, H=40, nqb=256, nkb=256, nkb_valid=256, tau=0.9,
                iou=P64, cluster_of=V(80), srp=V(96), soff=V(112), sci=V(128), cap=10, C=ctypes.byref(c),
                nnz=ctypes.byref(n), ws=W, ws_bytes=ws, stream=None)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return lib.calibatt_share_timesteps(*a.values())
    assert call(row_ptr=None) == 1
    assert call(iou=None) == 1
    assert call(sci=None) == 1
    assert call(T=0) == 2
    assert call(T=2000) == 7
    assert call(nkb=2048, nkb_valid=2048) == 7
    assert call(nkb_valid=300) == 2
    assert call(tau=float("nan")) == 2
    assert call(ws_bytes=ws - 1) == 6
    assert call(ws=V((1 << 20) + 16)) == 4
    assert call(set_off=V(52)) == 4


def test_skip_lists_reject(lib):
    ws = lib.calibatt_skip_ws_bytes(50, 40, 256)
    assert ws >= 2 * 50 * 40 * 256 * 4
    assert lib.calibatt_skip_ws_bytes(0, 1, 1) == 0
    w, wd, n = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int64(0)
    W = V(1 << 20)
    base = dict(row_ptr=P16, col_idx=P32, set_off=P48, T=50, H=40, nqb=256, nkb=256, num=95, den=1, counts=P64,
                pairs=V(80), cap=129, w=ctypes.byref(w), wd=ctypes.byref(wd), ws=W, ws_bytes=ws, stream=None)

    def enc(**kw):
        a = dict(base)
        a.update(kw)
        return lib.calibatt_encode_skip_lists(*a.values())
    assert enc(row_ptr=None) == 1
    assert enc(pairs=None) == 1
    assert enc(T=0) == 2
    assert enc(num=0) == 2
    assert enc(num=101) == 2
    assert enc(den=0) == 2
    assert enc(nkb=2048) == 7
    assert enc(ws_bytes=ws - 1) == 6
    assert enc(ws=V((1 << 20) + 8)) == 4
    dbase = dict(counts=P16, pairs=P32, width=8, T=50, H=40, nqb=256, row_ptr=P48, set_off=P64, col_idx=V(96),
                 cap=10, nnz=ctypes.byref(n), ws=W, ws_bytes=ws, stream=None)

    def dec(**kw):
        a = dict(dbase)
        a.update(kw)
        return lib.calibatt_decode_skip_lists(*a.values())
    assert dec(counts=None) == 1
    assert dec(width=-1) == 2
    assert dec(width=600) == 7
    assert dec(ws_bytes=ws - 1) == 6
    assert dec(set_off=V(68)) == 4


def test_validate_csr(lib):
    ok_rp = np.array([0, 2, 2, 5], np.int32)
    ok_ci = np.array([0, 3, 1, 2, 7], np.int32)
    cal.calibatt_validate_csr(ok_rp, ok_ci, 3, 8)
    bad = [
        (np.array([1, 2, 2, 5], np.int32), ok_ci),             # row_ptr[0] != 0
        (np.array([0, 3, 2, 5], np.int32), ok_ci),             # decreasing
        (ok_rp, np.array([0, 3, 1, 2, 8], np.int32)),          # column out of range
        (ok_rp, np.array([0, 3, 2, 1, 7], np.int32)),          # not ascending
        (ok_rp, np.array([0, 3, 1, 1, 7], np.int32)),          # duplicate
        (ok_rp, np.array([0, -1, 1, 2, 7], np.int32)),         # negative
        (ok_rp, ok_ci[:4]),                                    # nnz mismatch
    ]
    for rp, ci in bad:
        with pytest.raises(cal.CalibattError) as e:
            cal.calibatt_validate_csr(rp, ci, 3, 8)
        assert e.value.status == 5 or e.value.status == 1



@settings(max_examples=200, deadline=None, derandomize=True, database=None)
@given(st.integers(1, 6), st.integers(1, 10), st.data())
def test_validate_csr_property(lib, rows, nkb, data):
    """Random kept-block lists: a well-formed list is accepted, and each single
    defect (a column out of range, a repeated or descending column, a row_ptr
    that starts off zero or decreases) is rejected on the host."""
    lists = [sorted(data.draw(st.sets(st.integers(0, nkb - 1), max_size=nkb))) for _ in range(rows)]
    rp = np.concatenate([[0], np.cumsum([len(c) for c in lists])]).astype(np.int32)
    ci = np.array([c for row in lists for c in row], dtype=np.int32)
    cal.calibatt_validate_csr(rp, ci, rows, nkb)
    bad = []
    if len(ci):
        i = data.draw(st.integers(0, len(ci) - 1))
        for val in (nkb, -1, nkb + 1000):
            c2 = ci.copy()
            c2[i] = val
            bad.append((rp, c2))
        r = int(np.searchsorted(rp, i, side="right")) - 1        # the row holding entry i
        if i > rp[r]:
            c2 = ci.copy()
            c2[i] = c2[i - 1]                                     # repeated column
            bad.append((rp, c2))
        rp2 = rp.copy()
        rp2[0] = 1
        bad.append((rp2, ci))
    if rows >= 2 and rp[1] > 0:
        rp2 = rp.copy()
        rp2[1] = rp[2] + 1                                        # row 1 would end before it starts
        bad.append((rp2, ci))
    for brp, bci in bad:
        with pytest.raises(cal.CalibattError) as e:
            cal.calibatt_validate_csr(brp, bci, rows, nkb)
        assert e.value.status == 5

def test_repetition_entry_points_reject(lib):
    ws = lib.calibatt_similarity_ws_bytes(1, 40, 32768)
    assert ws == 40 * 32768 * 4 + 40 * 256 * 8
    assert lib.calibatt_similarity_ws_bytes(1, 1, 100) == 0

    def sim(**kw):
        a = dict(Q=P16, K=P32, B=1, H=40, L=32768, S=32760, d=128, dt=0, scale=0.1, F=21, R=30, C=52,
                 lse=None, sim=V(1 << 20), ws=V(1 << 30), ws_bytes=ws, stream=None)
        a.update(kw)
        return lib.calibatt_spatial_similarity(*a.values())
    assert sim(Q=None) == 1
    assert sim(sim=V(4)) == 4
    assert sim(ws=V((1 << 30) + 16)) == 4
    assert sim(dt=1) == 7
    assert sim(F=20) == 2                    # grid does not cover seq_len
    assert sim(R=1, C=52 * 30) == 2          # one row per frame: no pairs
    assert sim(ws_bytes=ws - 1) == 6
    assert sim(L=32760) == 2
    assert sim(lse=V((1 << 21) + 2)) == 4
    assert sim(scale=float("-inf")) == 2

    n = ctypes.c_int32(0)
    heads = np.zeros(4, dtype=np.int32)
    hp = heads.ctypes.data_as(ctypes.c_void_p)
    assert lib.calibatt_select_repetitive_heads(None, 2, 4, 0.87, hp, ctypes.byref(n), None) == 1
    assert lib.calibatt_select_repetitive_heads(P16, 0, 4, 0.87, hp, ctypes.byref(n), None) == 2
    assert lib.calibatt_select_repetitive_heads(V(12), 2, 4, 0.87, hp, ctypes.byref(n), None) == 4

    aws = lib.calibatt_anchor_ws_bytes(1, 40, 21, 52, 5, 128)
    lq = (21 * 5 * 52 + 127) // 128 * 128
    # anchor outputs, then the order: up to 8 parts per row, 9 partition offsets
    assert aws == 40 * lq * 128 * 2 + (40 * lq // 128 * 8 + 9) * 4
    assert lib.calibatt_anchor_ws_bytes(1, 40, 21, 52, 0, 128) == 0
    hl = np.array([3, 7], dtype=np.int32)

    def anchor(heads_arr=hl, **kw):
        a = dict(Q=TQ, K=TK, V=TV, O=TO, heads=heads_arr.ctypes.data_as(ctypes.c_void_p), n=len(heads_arr),
                 F=21, R=30, C=52, k=5, scale=0.1, B=1, H=40, L=32768, S=32760, d=128, dt=0, queue=V(1 << 20),
                 layout=1, ws=V(1 << 30), ws_bytes=aws, stream=None)
        a.update(kw)
        return lib.calibatt_anchor_attn_fwd(*a.values())
    assert anchor(Q=None) == 1
    assert anchor(queue=None) == 1
    assert anchor(ws=V((1 << 30) + 64)) == 4
    assert anchor(dt=1) == 7
    assert anchor(k=0) == 2
    assert anchor(k=31) == 2
    assert anchor(C=51) == 2
    assert anchor(n=41) == 2
    assert anchor(np.array([3, 40], dtype=np.int32)) == 2
    assert anchor(np.array([-1], dtype=np.int32)) == 2
    assert anchor(np.array([5, 5], dtype=np.int32)) == 2
    assert anchor(ws_bytes=aws - 1) == 6
    assert anchor(heads=None) == 1
    assert anchor(layout=3) == 2
    assert anchor(scale=0.0) == 2
    assert anchor(O=TK) == 2
    assert cal.calibatt_last_error() != ""


def test_single_pass_mass_rejects(lib):
    ws = lib.calibatt_block_mass_ws_bytes(1, 40, 32768, 128)
    assert ws == 40 * 256 * 32768 * 4
    assert lib.calibatt_block_mass_ws_bytes(1, 1, 100, 128) == 0

    def call(**kw):
        a = dict(Q=P16, K=P32, B=1, H=40, L=32768, S=32760, d=128, dt=0, block=128, scale=0.1, lse=P48, mass=P64,
                 ws=V(1 << 30), ws_bytes=ws, stream=None)
        a.update(kw)
        return lib.calibatt_block_mass_single_pass(*a.values())
    assert call(ws=None) == 1
    assert call(ws=V((1 << 30) + 64)) == 4
    assert call(ws_bytes=ws - 1) == 6
    assert call(dt=1) == 7
    assert call(S=32769) == 2
    assert call(block=32) == 7
    assert call(scale=0.0) == 2


def test_anchor_parts_rule(lib):
    """Parts per anchor row: ceil(rows*S/groups) * (ceil(n/S) + 4) minimised,
    a larger S only when 2% cheaper, within the O-capacity bound.  Wan (40
    heads, 21 x 30 x 52 grid, 256 CUs): k = 3 gives 1,040 rows for 512
    groups: costs 780 / 660 / 612 / 612 for S = 1 / 2 / 4 / 8, so 4; k = 5:
    1,040 / 924 / 952 -> 2; k = 4: 780 / 792 / 748 -> 4; k = 10, 15 -> 1."""
    wan = dict(B=1, n_heads=40, grid=(21, 30, 52), L=32768, seq_len=32760, d=128, num_cu=256)
    assert [cal.calibatt_anchor_parts(k_anchor=k, **wan) for k in (15, 10, 5, 4, 3)] == [1, 1, 2, 4, 4]
    # fewer CUs, more rows per group, less to gain: 64 CUs give 2,340 /
    # 2,244 / 2,244 (S = 2), 32 CUs 4,420 / 4,356 (1.4%: S = 1)
    assert cal.calibatt_anchor_parts(k_anchor=3, **dict(wan, num_cu=64)) == 2
    assert cal.calibatt_anchor_parts(k_anchor=3, **dict(wan, num_cu=32)) == 1
    # small grids: the capacity bound S*Lq*(2d+4) <= L*2d caps S
    small = dict(B=1, n_heads=2, grid=(3, 5, 20), L=384, seq_len=300, d=128, num_cu=256)
    assert cal.calibatt_anchor_parts(k_anchor=1, **small) == 2     # 2 rows, n = 3, capacity 2.95
    assert cal.calibatt_anchor_parts(k_anchor=5, **small) == 1     # Lq = 384 = L
    g8 = dict(B=1, n_heads=2, grid=(8, 8, 64), L=4096, seq_len=4096, d=128, num_cu=256)
    assert cal.calibatt_anchor_parts(k_anchor=1, **g8) == 4        # capacity 7.9
    g4 = dict(B=1, n_heads=2, grid=(4, 16, 64), L=4096, seq_len=4096, d=64, num_cu=256)
    assert cal.calibatt_anchor_parts(k_anchor=1, **g4) == 8
    assert cal.calibatt_anchor_parts(k_anchor=1, **dict(g4, seq_len=3 * 128)) == 2   # S <= n = 3
    for bad in (dict(k_anchor=0), dict(k_anchor=1, d=96), dict(k_anchor=1, num_cu=0), dict(k_anchor=1, L=100)):
        kw = dict(g8, **bad)
        assert cal.calibatt_anchor_parts(**kw) == 0
