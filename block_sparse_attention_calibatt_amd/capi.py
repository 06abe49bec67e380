"""Python binding of the C ABI: one function per entry point, same names.

Each function only marshals arguments: it checks that the torch tensors have
the shapes, dtypes and devices the raw-pointer ABI assumes (the library cannot
see tensor sizes), passes their device pointers and torch's current HIP
stream, and raises CalibattError on a non-OK status.  All computation runs in
the library's HIP kernels.
"""

import ctypes

import numpy as np
import torch

from ._lib import BF16, F32, V_BHDL, V_BHLD, CalibattError, check, load

_DT = {torch.bfloat16: BF16, torch.float32: F32}


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _dev_tensor(t, name, dtype=None):
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor")
    _need(t.is_cuda, f"{name} must be on a GPU device")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if dtype is not None:
        _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")


PARTS = 8            # work partitions (one per XCD)
QUEUE_INTS = 128     # persistent-launch counters: 8 partitions x 16 int32


def new_queue(device):
    """A zeroed persistent-launch workspace for the attention entry points."""
    return torch.zeros(QUEUE_INTS, dtype=torch.int32, device=device)


def _queue(queue_ws):
    if queue_ws is not None:
        _dev_tensor(queue_ws, "queue_ws", torch.int32)
        _need(queue_ws.numel() >= QUEUE_INTS, f"queue_ws needs >= {QUEUE_INTS} int32 entries")


def _qkv(Q, K, V, O, v_transposed=False):
    for n, t in (("Q", Q), ("K", K), ("V", V), ("O", O)):
        _dev_tensor(t, n)
    _need(Q.dim() == 4, "Q must be [B, H, L, d]")
    for n, t in (("K", K), ("O", O)):
        _need(t.shape == Q.shape and t.dtype == Q.dtype and t.device == Q.device,
              f"{n} must match Q in shape, dtype and device")
    B, H, L, d = Q.shape
    vshape = (B, H, d, L) if v_transposed else (B, H, L, d)
    _need(tuple(V.shape) == vshape and V.dtype == Q.dtype and V.device == Q.device,
          f"V must be {list(vshape)} of Q's dtype on Q's device")
    _need(Q.dtype in _DT, f"unsupported dtype {Q.dtype} (bfloat16 or float32)")
    return Q.shape


def calibatt_sparse_attn_fwd(Q, K, V, O, row_ptr, col_idx, block, scale, seq_len=None,
                             work_order=None, queue_ws=None, v_transposed=False):
    """V is [B, H, L, d], or V^T [B, H, d, L] with v_transposed=True."""
    B, H, L, d = _qkv(Q, K, V, O, v_transposed)
    seq_len = L if seq_len is None else int(seq_len)
    _dev_tensor(row_ptr, "row_ptr", torch.int32)
    _dev_tensor(col_idx, "col_idx", torch.int32)
    _need(block > 0 and L % block == 0, "L must be a multiple of block")
    rows = H * (L // block)
    _need(row_ptr.numel() == rows + 1, f"row_ptr must have H*nqb+1 = {rows + 1} entries")
    if work_order is not None:
        _dev_tensor(work_order, "work_order", torch.int32)
        _need(work_order.numel() == rows + PARTS + 1, f"work_order must have H*nqb+9 = {rows + PARTS + 1} entries")
    _queue(queue_ws)
    lib = load()
    check(lib.calibatt_sparse_attn_fwd(
        _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(row_ptr), _ptr(col_idx), int(block), float(scale),
        B, H, L, seq_len, d, _DT[Q.dtype], _ptr(work_order), _ptr(queue_ws), col_idx.numel(),
        V_BHDL if v_transposed else V_BHLD, _stream(Q)))
    return O


def calibatt_sparse_attn_fwd_noalloc(Q, K, V, O, row_ptr, col_idx, block, scale, seq_len=None,
                                     work_order=None, v_transposed=False):
    """calibatt_sparse_attn_fwd with its queue in the library's static scratch."""
    B, H, L, d = _qkv(Q, K, V, O, v_transposed)
    seq_len = L if seq_len is None else int(seq_len)
    _dev_tensor(row_ptr, "row_ptr", torch.int32)
    _dev_tensor(col_idx, "col_idx", torch.int32)
    _need(block > 0 and L % block == 0, "L must be a multiple of block")
    rows = H * (L // block)
    _need(row_ptr.numel() == rows + 1, f"row_ptr must have H*nqb+1 = {rows + 1} entries")
    if work_order is not None:
        _dev_tensor(work_order, "work_order", torch.int32)
        _need(work_order.numel() == rows + PARTS + 1, f"work_order must have H*nqb+9 = {rows + PARTS + 1} entries")
    lib = load()
    check(lib.calibatt_sparse_attn_fwd_noalloc(
        _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(row_ptr), _ptr(col_idx), int(block), float(scale),
        B, H, L, seq_len, d, _DT[Q.dtype], _ptr(work_order), col_idx.numel(),
        V_BHDL if v_transposed else V_BHLD, _stream(Q)))
    return O


def calibatt_dense_attn_fwd(Q, K, V, O, block, scale, seq_len=None, queue_ws=None, v_transposed=False):
    B, H, L, d = _qkv(Q, K, V, O, v_transposed)
    seq_len = L if seq_len is None else int(seq_len)
    _queue(queue_ws)
    lib = load()
    check(lib.calibatt_dense_attn_fwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), int(block), float(scale),
                                      B, H, L, seq_len, d, _DT[Q.dtype], _ptr(queue_ws),
                                      V_BHDL if v_transposed else V_BHLD, _stream(Q)))
    return O


def calibatt_transpose_v(V, Vt=None, seq_len=None):
    """V [B, H, L, d] -> V^T [B, H, d, L] (keys >= seq_len written as 0)."""
    _dev_tensor(V, "V")
    _need(V.dim() == 4 and V.dtype in _DT, "V must be [B, H, L, d], bfloat16 or float32")
    B, H, L, d = V.shape
    seq_len = L if seq_len is None else int(seq_len)
    if Vt is None:
        Vt = torch.empty((B, H, d, L), dtype=V.dtype, device=V.device)
    _dev_tensor(Vt, "Vt", V.dtype)
    _need(tuple(Vt.shape) == (B, H, d, L) and Vt.device == V.device, "Vt must be [B, H, d, L] on V's device")
    lib = load()
    check(lib.calibatt_transpose_v(_ptr(V), _ptr(Vt), B, H, L, seq_len, d, _DT[V.dtype], _stream(V)))
    return Vt


def calibatt_block_mass(Q, K, block, scale, lse_ws, mass, seq_len=None):
    for n, t in (("Q", Q), ("K", K)):
        _dev_tensor(t, n)
    _need(Q.dim() == 4 and K.shape == Q.shape and K.dtype == Q.dtype, "Q, K must be [B, H, L, d] alike")
    _need(Q.dtype in _DT, f"unsupported dtype {Q.dtype}")
    B, H, L, d = Q.shape
    seq_len = L if seq_len is None else int(seq_len)
    _need(block > 0 and L % block == 0, "L must be a multiple of block")
    nb = L // block
    _dev_tensor(lse_ws, "lse_ws", torch.float32)
    _dev_tensor(mass, "mass", torch.float32)
    _need(lse_ws.numel() == B * H * L, "lse_ws must have B*H*L entries")
    _need(mass.numel() == B * H * nb * nb, "mass must have B*H*nqb*nkb entries")
    lib = load()
    check(lib.calibatt_block_mass(_ptr(Q), _ptr(K), B, H, L, seq_len, d, _DT[Q.dtype], int(block),
                                  float(scale), _ptr(lse_ws), _ptr(mass), _stream(Q)))
    return mass


def calibatt_block_mass_ws_bytes(B, H, L, block):
    return int(load().calibatt_block_mass_ws_bytes(int(B), int(H), int(L), int(block)))


def calibatt_block_mass_single_pass(Q, K, block, scale, lse_ws, mass, seq_len=None, ws=None):
    """The pooled mass in one pass over the scores (per-(key block, query) log2
    partials in `ws`, a uint8 device tensor of calibatt_block_mass_ws_bytes bytes)."""
    for n, t in (("Q", Q), ("K", K)):
        _dev_tensor(t, n)
    _need(Q.dim() == 4 and K.shape == Q.shape and K.dtype == Q.dtype, "Q, K must be [B, H, L, d] alike")
    _need(Q.dtype in _DT, f"unsupported dtype {Q.dtype}")
    B, H, L, d = Q.shape
    seq_len = L if seq_len is None else int(seq_len)
    _need(block > 0 and L % block == 0, "L must be a multiple of block")
    nb = L // block
    _dev_tensor(lse_ws, "lse_ws", torch.float32)
    _dev_tensor(mass, "mass", torch.float32)
    _need(lse_ws.numel() == B * H * L, "lse_ws must have B*H*L entries")
    _need(mass.numel() == B * H * nb * nb, "mass must have B*H*nqb*nkb entries")
    need = calibatt_block_mass_ws_bytes(B, H, L, block)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
    _dev_tensor(ws, "ws", torch.uint8)
    lib = load()
    check(lib.calibatt_block_mass_single_pass(_ptr(Q), _ptr(K), B, H, L, seq_len, d, _DT[Q.dtype], int(block),
                                              float(scale), _ptr(lse_ws), _ptr(mass), _ptr(ws), ws.numel(),
                                              _stream(Q)))
    return mass


def calibatt_compile_ws_bytes(P, H, nqb, nkb):
    return int(load().calibatt_compile_ws_bytes(int(P), int(H), int(nqb), int(nkb)))


def _work_order_arg(work_order, rows):
    if work_order is not None:
        _dev_tensor(work_order, "work_order", torch.int32)
        _need(work_order.numel() == rows + PARTS + 1, f"work_order must have H*nqb+9 = {rows + PARTS + 1} entries")
    return _ptr(work_order)


def calibatt_compile_masks(mass, keep_topk, min_agree, nkb_valid=None, row_ptr=None, col_idx=None,
                           ws=None, work_order=None):
    """mass [P, H, nqb, nkb] float32 -> (row_ptr, col_idx) int32 device tensors; with
    work_order (an [H*nqb + 9] int32 tensor) the set's work order is written too."""
    _dev_tensor(mass, "mass", torch.float32)
    _need(mass.dim() == 4, "mass must be [P, H, nqb, nkb]")
    P, H, nqb, nkb = mass.shape
    nkb_valid = nkb if nkb_valid is None else int(nkb_valid)
    rows = H * nqb
    dev = mass.device
    if row_ptr is None:
        row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    _dev_tensor(row_ptr, "row_ptr", torch.int32)
    _need(row_ptr.numel() == rows + 1, "row_ptr must have H*nqb+1 entries")
    if col_idx is None:
        col_idx = torch.empty(max(1, rows * nkb_valid), dtype=torch.int32, device=dev)
    _dev_tensor(col_idx, "col_idx", torch.int32)
    need = calibatt_compile_ws_bytes(P, H, nqb, nkb)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _dev_tensor(ws, "ws", torch.uint8)
    nnz = ctypes.c_int64(0)
    lib = load()
    wo = _work_order_arg(work_order, rows)
    check(lib.calibatt_compile_masks(_ptr(mass), P, H, nqb, nkb, nkb_valid, int(keep_topk),
                                     int(min_agree), _ptr(row_ptr), _ptr(col_idx), col_idx.numel(), wo,
                                     ctypes.byref(nnz), _ptr(ws), ws.numel(), _stream(mass)))
    return row_ptr, col_idx[: nnz.value]


def _eps_fraction(eps):
    """epsilon as (num, den); a float is read as the decimal it prints as."""
    from fractions import Fraction
    e = Fraction(str(eps)) if isinstance(eps, float) else Fraction(eps)
    _need(0 <= e <= 1, "eps must lie in [0, 1]")
    _need(e.denominator < 2 ** 31, "eps needs a denominator below 2^31")
    return e.numerator, e.denominator


def calibatt_compile_masks_energy(mass, eps, min_agree, nkb_valid=None, row_ptr=None, col_idx=None, ws=None,
                                  work_order=None):
    """Energy-threshold compile: mass [P, H, nqb, nkb] float32 -> (row_ptr, col_idx) int32 device tensors."""
    _dev_tensor(mass, "mass", torch.float32)
    _need(mass.dim() == 4, "mass must be [P, H, nqb, nkb]")
    P, H, nqb, nkb = mass.shape
    nkb_valid = nkb if nkb_valid is None else int(nkb_valid)
    num, den = _eps_fraction(eps)
    rows = H * nqb
    dev = mass.device
    if row_ptr is None:
        row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    _dev_tensor(row_ptr, "row_ptr", torch.int32)
    _need(row_ptr.numel() == rows + 1, "row_ptr must have H*nqb+1 entries")
    if col_idx is None:
        col_idx = torch.empty(max(1, rows * nkb_valid), dtype=torch.int32, device=dev)
    _dev_tensor(col_idx, "col_idx", torch.int32)
    need = calibatt_compile_ws_bytes(P, H, nqb, nkb)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _dev_tensor(ws, "ws", torch.uint8)
    nnz = ctypes.c_int64(0)
    lib = load()
    wo = _work_order_arg(work_order, rows)
    check(lib.calibatt_compile_masks_energy(_ptr(mass), P, H, nqb, nkb, nkb_valid, num, den, int(min_agree),
                                            _ptr(row_ptr), _ptr(col_idx), col_idx.numel(), wo, ctypes.byref(nnz),
                                            _ptr(ws), ws.numel(), _stream(mass)))
    return row_ptr, col_idx[: nnz.value]


def calibatt_share_ws_bytes(T, H, nqb, nkb):
    return int(load().calibatt_share_ws_bytes(int(T), int(H), int(nqb), int(nkb)))


def calibatt_share_timesteps(row_ptr, col_idx, set_off, H, nqb, nkb, nkb_valid, tau, ws=None):
    """Bank of T sets (row_ptr [T, H*nqb+1], col_idx, set_off [T+1] int64, device) ->
    (cluster_of [T], iou [T, T], shared_row_ptr [C, H*nqb+1], shared_set_off [C+1], shared_col_idx)."""
    _dev_tensor(row_ptr, "row_ptr", torch.int32)
    _dev_tensor(col_idx, "col_idx", torch.int32)
    _dev_tensor(set_off, "set_off", torch.int64)
    _need(row_ptr.dim() == 2 and row_ptr.shape[1] == H * nqb + 1, "row_ptr must be [T, H*nqb+1]")
    T = row_ptr.shape[0]
    _need(set_off.numel() == T + 1, "set_off must have T+1 entries")
    dev = row_ptr.device
    iou = torch.empty((T, T), dtype=torch.float64, device=dev)
    cluster_of = torch.empty(T, dtype=torch.int32, device=dev)
    s_rp = torch.empty((T, H * nqb + 1), dtype=torch.int32, device=dev)
    s_off = torch.empty(T + 1, dtype=torch.int64, device=dev)
    s_ci = torch.empty(max(1, T * H * nqb * int(nkb_valid)), dtype=torch.int32, device=dev)
    need = calibatt_share_ws_bytes(T, H, nqb, nkb)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _dev_tensor(ws, "ws", torch.uint8)
    C = ctypes.c_int32(0)
    nnz = ctypes.c_int64(0)
    lib = load()
    check(lib.calibatt_share_timesteps(_ptr(row_ptr), _ptr(col_idx), _ptr(set_off), T, int(H), int(nqb), int(nkb),
                                       int(nkb_valid), float(tau), _ptr(iou), _ptr(cluster_of), _ptr(s_rp),
                                       _ptr(s_off), _ptr(s_ci), s_ci.numel(), ctypes.byref(C), ctypes.byref(nnz),
                                       _ptr(ws), ws.numel(), _stream(row_ptr)))
    c = C.value
    return cluster_of, iou, s_rp[:c], s_off[: c + 1], s_ci[: nnz.value]


def calibatt_skip_ws_bytes(T, H, nqb):
    return int(load().calibatt_skip_ws_bytes(int(T), int(H), int(nqb)))


def calibatt_encode_skip_lists(row_ptr, col_idx, set_off, H, nqb, nkb, merge_pct=100, ws=None):
    """Bank (row_ptr [T, H*nqb+1], col_idx, set_off [T+1] int64, device) ->
    (width, widest, counts [T*H*nqb], pairs [T*H*nqb, width, 2]) int32 device tensors."""
    from fractions import Fraction
    _dev_tensor(row_ptr, "row_ptr", torch.int32)
    _dev_tensor(col_idx, "col_idx", torch.int32)
    _dev_tensor(set_off, "set_off", torch.int64)
    _need(row_ptr.dim() == 2 and row_ptr.shape[1] == H * nqb + 1, "row_ptr must be [T, H*nqb+1]")
    p = Fraction(str(merge_pct)) if isinstance(merge_pct, float) else Fraction(merge_pct)
    T = row_ptr.shape[0]
    E = T * H * nqb
    dev = row_ptr.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    cap = int(nkb) // 2 + 1
    pairs = torch.empty(max(1, E * cap * 2), dtype=torch.int32, device=dev)
    need = calibatt_skip_ws_bytes(T, H, nqb)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _dev_tensor(ws, "ws", torch.uint8)
    w, widest = ctypes.c_int32(0), ctypes.c_int32(0)
    lib = load()
    check(lib.calibatt_encode_skip_lists(_ptr(row_ptr), _ptr(col_idx), _ptr(set_off), T, int(H), int(nqb), int(nkb),
                                         p.numerator, p.denominator, _ptr(counts), _ptr(pairs), cap,
                                         ctypes.byref(w), ctypes.byref(widest), _ptr(ws), ws.numel(), _stream(row_ptr)))
    return w.value, widest.value, counts, pairs[: E * w.value * 2].view(E, w.value, 2)


def calibatt_decode_skip_lists(counts, pairs, width, T, H, nqb, nnz_cap=None, ws=None):
    """-> (row_ptr [T, H*nqb+1], set_off [T+1] int64, col_idx) device tensors."""
    _dev_tensor(counts, "counts", torch.int32)
    _dev_tensor(pairs, "pairs", torch.int32)
    dev = counts.device
    rows = H * nqb
    rp = torch.empty((T, rows + 1), dtype=torch.int32, device=dev)
    off = torch.empty(T + 1, dtype=torch.int64, device=dev)
    need = calibatt_skip_ws_bytes(T, H, nqb)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _dev_tensor(ws, "ws", torch.uint8)
    nnz = ctypes.c_int64(0)
    lib = load()

    def call(ci, cap):
        return lib.calibatt_decode_skip_lists(_ptr(counts), _ptr(pairs), int(width), int(T), int(H), int(nqb),
                                              _ptr(rp), _ptr(off), _ptr(ci), cap, ctypes.byref(nnz), _ptr(ws),
                                              ws.numel(), _stream(counts))
    if nnz_cap is None:
        # size the column array from the library's own count (capacity protocol)
        probe = torch.empty(1, dtype=torch.int32, device=dev)
        st = call(probe, 0)
        if st == 0:
            return rp, off, probe[:0]
        _need(st == 6, f"decode count failed: {calibatt_status_string(st)}: {calibatt_last_error()}")
        nnz_cap = nnz.value
    ci = torch.empty(max(1, int(nnz_cap)), dtype=torch.int32, device=dev)
    check(call(ci, int(nnz_cap)))
    return rp, off, ci[: nnz.value]


def calibatt_similarity_ws_bytes(B, H, L):
    return int(load().calibatt_similarity_ws_bytes(int(B), int(H), int(L)))


def calibatt_spatial_similarity(Q, K, scale, grid, seq_len=None, sim=None, ws=None, lse=None):
    """Score per (b, h): mean cosine of the softmax rows of vertically adjacent
    tokens on the (frames, rows, cols) grid.  Returns sim [B, H] float64.
    `lse`: the [B*H*L] float32 log-sum-exp a block-mass call left for the same
    Q, K, scale and seq_len (skips recomputing it), or None."""
    for n, t in (("Q", Q), ("K", K)):
        _dev_tensor(t, n, torch.bfloat16)
    _need(Q.dim() == 4 and K.shape == Q.shape and K.device == Q.device, "Q, K must be [B, H, L, d] alike")
    B, H, L, d = Q.shape
    seq_len = L if seq_len is None else int(seq_len)
    F, R, C = (int(x) for x in grid)
    if sim is None:
        sim = torch.empty((B, H), dtype=torch.float64, device=Q.device)
    _dev_tensor(sim, "sim", torch.float64)
    _need(sim.numel() == B * H, "sim must have B*H entries")
    need = calibatt_similarity_ws_bytes(B, H, L)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
    _dev_tensor(ws, "ws", torch.uint8)
    if lse is not None:
        _dev_tensor(lse, "lse", torch.float32)
        _need(lse.numel() == B * H * L, "lse must have B*H*L entries")
    lib = load()
    check(lib.calibatt_spatial_similarity(_ptr(Q), _ptr(K), B, H, L, seq_len, d, BF16, float(scale), F, R, C,
                                          _ptr(lse), _ptr(sim), _ptr(ws), ws.numel(), _stream(Q)))
    return sim


def calibatt_select_repetitive_heads(sim, tau):
    """sim [P, H] float64 (device) -> ascending list of heads whose mean over P exceeds tau."""
    _dev_tensor(sim, "sim", torch.float64)
    _need(sim.dim() == 2, "sim must be [P, H]")
    P, H = sim.shape
    heads = np.zeros(H, dtype=np.int32)
    n = ctypes.c_int(0)
    lib = load()
    check(lib.calibatt_select_repetitive_heads(_ptr(sim), P, H, float(tau), heads.ctypes.data_as(ctypes.c_void_p),
                                               ctypes.byref(n), _stream(sim)))
    return [int(h) for h in heads[:n.value]]


def calibatt_anchor_ws_bytes(B, H, frames, grid_cols, k_anchor, d):
    return int(load().calibatt_anchor_ws_bytes(int(B), int(H), int(frames), int(grid_cols), int(k_anchor), int(d)))


def calibatt_anchor_parts(B, n_heads, grid, k_anchor, L, seq_len, d, num_cu):
    """Parts each anchor row is cut into (1, 2, 4 or 8); 0 for invalid arguments."""
    F, _, C = (int(x) for x in grid)
    return int(load().calibatt_anchor_parts(int(B), int(n_heads), F, C, int(k_anchor), int(L), int(seq_len), int(d),
                                            int(num_cu)))


def calibatt_anchor_attn_fwd(Q, K, V, O, heads, grid, k_anchor, scale, seq_len=None, queue_ws=None,
                             v_transposed=False, ws=None):
    """Anchor-row attention for the listed heads; other heads of O are left as they are."""
    B, H, L, d = _qkv(Q, K, V, O, v_transposed)
    _need(Q.dtype == torch.bfloat16, "anchor attention takes bfloat16 tensors")
    seq_len = L if seq_len is None else int(seq_len)
    F, R, C = (int(x) for x in grid)
    hl = np.ascontiguousarray(np.asarray(list(heads), dtype=np.int32))
    if queue_ws is None:
        queue_ws = new_queue(Q.device)
    _queue(queue_ws)
    need = calibatt_anchor_ws_bytes(B, H, F, C, k_anchor, d)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
    _dev_tensor(ws, "ws", torch.uint8)
    lib = load()
    check(lib.calibatt_anchor_attn_fwd(
        _ptr(Q), _ptr(K), _ptr(V), _ptr(O), hl.ctypes.data_as(ctypes.c_void_p), int(hl.size), F, R, C,
        int(k_anchor), float(scale), B, H, L, seq_len, d, BF16, _ptr(queue_ws),
        V_BHDL if v_transposed else V_BHLD, _ptr(ws), ws.numel(), _stream(Q)))
    return O


def calibatt_build_schedule(row_ptr, H, nqb, work_order=None):
    _dev_tensor(row_ptr, "row_ptr", torch.int32)
    _need(row_ptr.numel() == H * nqb + 1, "row_ptr must have H*nqb+1 entries")
    if work_order is None:
        work_order = torch.empty(H * nqb + PARTS + 1, dtype=torch.int32, device=row_ptr.device)
    _dev_tensor(work_order, "work_order", torch.int32)
    _need(work_order.numel() == H * nqb + PARTS + 1, "work_order must have H*nqb+9 entries")
    lib = load()
    check(lib.calibatt_build_schedule(_ptr(row_ptr), int(H), int(nqb), _ptr(work_order), _stream(row_ptr)))
    return work_order


def calibatt_validate_csr(row_ptr, col_idx, rows, nkb_valid):
    """Host arrays (numpy int32); raises CalibattError(CALIBATT_ERR_CSR) on a defect."""
    rp = np.ascontiguousarray(row_ptr, dtype=np.int32)
    ci = np.ascontiguousarray(col_idx, dtype=np.int32)
    if rp.size < rows + 1:
        raise ValueError("row_ptr shorter than rows + 1")
    lib = load()
    check(lib.calibatt_validate_csr(rp.ctypes.data_as(ctypes.c_void_p),
                                    ci.ctypes.data_as(ctypes.c_void_p) if ci.size else None,
                                    int(rows), int(nkb_valid), ci.size))


def calibatt_status_string(status):
    return load().calibatt_status_string(int(status)).decode()


def calibatt_last_error():
    return load().calibatt_last_error().decode()


def calibatt_version():
    return int(load().calibatt_version())


__all__ = [
    "CalibattError",
    "new_queue",
    "calibatt_transpose_v",
    "calibatt_sparse_attn_fwd",
    "calibatt_sparse_attn_fwd_noalloc",
    "calibatt_dense_attn_fwd",
    "calibatt_block_mass",
    "calibatt_compile_ws_bytes",
    "calibatt_compile_masks",
    "calibatt_build_schedule",
    "calibatt_validate_csr",
    "calibatt_status_string",
    "calibatt_last_error",
    "calibatt_version",
]
