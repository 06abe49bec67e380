/*
 * calibatt.h - C ABI of the MI355X (gfx950) calibrated block-sparse attention library.
 *
 * The method is CalibAtt ("Accelerating Text-to-Video Generation with
 * Calibrated Sparse Attention", arXiv 2603.05503).  Offline, calibration
 * prompts are run through the model, the post-softmax attention maps are
 * pooled to blocks, the top key blocks of every query block are kept per
 * prompt, and blocks that enough prompts agree on form a mask per (layer,
 * head, timestep).  At inference the kept blocks are computed densely and the
 * rest are skipped, i.e. their keys are absent from the softmax.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers unless the comment says (host).
 * - Q, K, V, O are [B, H, L, d] row-major and contiguous (d fastest).  L is
 *   the padded token count and must be a multiple of `block`; tokens
 *   t >= seq_len are padding: they are never keys, and their output rows are
 *   written as zero.  The attention entry points also accept V transposed,
 *   as V^T [B, H, d, L] (CALIBATT_V_BHDL); they read either layout as it
 *   lies and need no copy of it.
 * - One block is `block` tokens; query blocks and key blocks have the same
 *   size.  nqb = nkb = L / block; nkb_valid = ceil(seq_len / block).
 * - A mask set is CSR over rows r = h * nqb + qb (h-major): the kept key
 *   blocks of row r are col_idx[row_ptr[r] .. row_ptr[r+1]), ascending,
 *   unique, each < nkb_valid.  row_ptr has H*nqb+1 int32 entries, row_ptr[0]
 *   = 0.  One mask set serves every batch entry.
 * - Ownership: the caller allocates and frees every buffer.  The library keeps
 *   no pointer after a call returns and holds no global state besides a
 *   per-device property cache and a thread-local error message.
 * - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL is the
 *   default stream) and the call returns after enqueueing, except where a
 *   comment says it synchronises.
 * - Errors: argument checks run on the host before anything is enqueued; on
 *   an argument error nothing is written.  A failed HIP call returns
 *   CALIBATT_ERR_HIP.  calibatt_last_error() gives the detail.  A malformed
 *   CSR passed to a device entry point is undefined behaviour on the device:
 *   check untrusted lists with calibatt_validate_csr first.
 * - Supported shapes: d in {64, 128}; block in {64, 128}; bf16 or f32
 *   inputs; Q/K/V/O 16-byte aligned; B, H >= 1; 0 < seq_len <= L;
 *   B * H * L * d < 2^31.
 */
#ifndef CALIBATT_H
#define CALIBATT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CALIBATT_VERSION 303 /* major * 100 + minor */

typedef enum {
  CALIBATT_OK = 0,
  CALIBATT_ERR_NULL = 1,        /* a required pointer is NULL */
  CALIBATT_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  CALIBATT_ERR_DTYPE = 3,       /* unknown dtype code */
  CALIBATT_ERR_ALIGN = 4,       /* a pointer is not aligned as required */
  CALIBATT_ERR_CSR = 5,         /* a kept-block list is malformed */
  CALIBATT_ERR_CAPACITY = 6,    /* an output buffer is too small */
  CALIBATT_ERR_UNSUPPORTED = 7, /* a valid but unimplemented combination */
  CALIBATT_ERR_HIP = 8          /* the HIP runtime reported an error */
} calibatt_status;

typedef enum { CALIBATT_BF16 = 0, CALIBATT_F32 = 1 } calibatt_dtype;

/* Layout of the V argument of the attention entry points. */
typedef enum {
  CALIBATT_V_BHLD = 0, /* V [B, H, L, d], like Q and K */
  CALIBATT_V_BHDL = 1  /* V^T [B, H, d, L] (V[b,h,j,:] is column j) */
} calibatt_vlayout;

/*
 * Block-sparse attention forward (inference step).
 * Pages: abstract (selected connections computed densely, unselected ones
 * skipped) and Fig. 5(b) caption (block masks loaded, unset blocks not
 * computed).  For every batch entry b, head h and query token i < seq_len in
 * query block qb (row r = h*nqb + qb), with J_i the valid tokens of the kept
 * key blocks of row r:
 *     O[b,h,i,:] = sum_{j in J_i} softmax_j(scale * Q[b,h,i,:] . K[b,h,j,:]) V[b,h,j,:]
 * A row with no kept block, and every padded query row, is written as zero
 * (whatever the padded rows of Q, K and V hold).
 *
 *   Q, K        [B, H, L, d] inputs of dtype `dt` (device).
 *   V           input of dtype `dt` (device) in the layout `v_layout` names.
 *               With CALIBATT_V_BHDL its entries for keys >= seq_len must be
 *               finite (they are multiplied by zero probabilities); with
 *               CALIBATT_V_BHLD padded rows may hold anything.
 *   O           [B, H, L, d] output of dtype `dt` (device); fully written.
 *               It must not overlap Q, K or V (CALIBATT_ERR_SHAPE).
 *   row_ptr     [H*nqb + 1] int32 CSR row offsets (device).
 *   col_idx     [row_ptr[H*nqb]] int32 kept key blocks (device).
 *   block       tokens per block (64 or 128).
 *   scale       softmax scale applied to q.k (usually 1/sqrt(d)); finite
 *               and > 0, else CALIBATT_ERR_SHAPE.
 *   work_order  optional [H*nqb + 9] int32 from calibatt_build_schedule: a
 *               permutation of the rows split into 8 partition lists,
 *               followed by the 9 list offsets (0, ..., H*nqb).  NULL =
 *               partition p holds heads p, p+8, ... in natural order.  The
 *               result does not depend on it (each row is reduced by one
 *               group of waves in col_idx order).
 *   queue_ws    optional int32 workspace of >= 128 entries (device), 16-byte
 *               aligned.  Non-NULL selects the persistent launch: one grid
 *               that fills the GPU; workgroup i serves partition i % 8 (the
 *               XCD it runs on) from an atomic counter in queue_ws, then the
 *               other partitions.  The call resets the counters on `stream`
 *               itself.  NULL = one workgroup per row (block 128 bf16: per
 *               two rows).  Calls that share a queue_ws must not overlap in
 *               time.
 *   nnz         number of entries of col_idx (= row_ptr[H*nqb]); used only
 *               for the host-side size check.
 *   v_layout    CALIBATT_V_BHLD or CALIBATT_V_BHDL (see V).
 * The bf16 path computes q.k and p.v on bf16 matrix cores with float32
 * accumulation and a float32 softmax; probabilities are rounded to bf16
 * before the p.v product; O is rounded to bf16.  The f32 path is float32
 * throughout.
 */
calibatt_status calibatt_sparse_attn_fwd(const void* Q, const void* K, const void* V, void* O,
                                         const int32_t* row_ptr, const int32_t* col_idx,
                                         int block, float scale, int B, int H, int L,
                                         int seq_len, int d, calibatt_dtype dt,
                                         const int32_t* work_order, int32_t* queue_ws,
                                         int64_t nnz, calibatt_vlayout v_layout, void* stream);

/*
 * calibatt_sparse_attn_fwd for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments without queue_ws, same result bit for bit as
 * calibatt_sparse_attn_fwd with a queue_ws (the persistent launch, always).
 * The call allocates nothing: the queue counters live in a static device
 * array of the library, 512 bytes per GPU, held until the process ends; its
 * size does not grow with the problem, so every size calibatt_sparse_attn_fwd
 * accepts fits.  The call re-zeroes the counters on `stream` with a kernel
 * (no memset node).  All calls on one GPU share that array: calls that
 * overlap in time on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  Devices 0..63 (CALIBATT_ERR_UNSUPPORTED beyond).
 */
calibatt_status calibatt_sparse_attn_fwd_noalloc(const void* Q, const void* K, const void* V, void* O,
                                                 const int32_t* row_ptr, const int32_t* col_idx,
                                                 int block, float scale, int B, int H, int L,
                                                 int seq_len, int d, calibatt_dtype dt,
                                                 const int32_t* work_order, int64_t nnz,
                                                 calibatt_vlayout v_layout, void* stream);

/*
 * Dense attention forward: the same computation with every valid key block
 * kept (the pages' dense baseline, Table 1 and Table S6).  Arguments as above;
 * queue_ws (optional, >= 128 int32) selects the persistent launch with the
 * natural head partition.
 */
calibatt_status calibatt_dense_attn_fwd(const void* Q, const void* K, const void* V, void* O,
                                        int block, float scale, int B, int H, int L, int seq_len,
                                        int d, calibatt_dtype dt, int32_t* queue_ws,
                                        calibatt_vlayout v_layout, void* stream);

/*
 * V [B, H, L, d] -> V^T [B, H, d, L]: Vt[b,h,c,j] = V[b,h,j,c] for j <
 * seq_len and 0 for the padded keys j >= seq_len.  A layout change only: for
 * callers that keep V transposed (CALIBATT_V_BHDL); the attention entry
 * points read either layout themselves.
 *   V, Vt   inputs/outputs of dtype `dt` (device), 16-byte aligned, not
 *           overlapping.  L must be a multiple of 64; d in {64, 128}.
 */
calibatt_status calibatt_transpose_v(const void* V, void* Vt, int B, int H, int L, int seq_len, int d,
                                     calibatt_dtype dt, void* stream);

/*
 * Calibration pooling: post-softmax attention mass per (query block, key
 * block).  Pages: Fig. 2 caption (block-level view of post-softmax maps),
 * Table S5 caption (block energies on the calibration prompts).  With the
 * full softmax over the valid keys j < seq_len,
 *     mass[b,h,qb,kb] = sum_{i in qb, i < seq_len} sum_{j in kb, j < seq_len}
 *                       softmax_j(scale * Q[b,h,i,:] . K[b,h,j,:])
 * so each valid query contributes 1 to its row of blocks.
 *
 *   Q, K     [B, H, L, d] inputs of dtype `dt` (device).
 *   scale    softmax scale, finite and > 0 (else CALIBATT_ERR_SHAPE; the
 *            same holds for every entry point that takes a scale).
 *   lse_ws   [B, H, L] float32 workspace (device); on return it holds
 *            log(sum_{j < seq_len} exp(scale * q_i . k_j)) per query (natural
 *            log; padded rows hold -inf).
 *   mass     [B, H, nqb, nkb] float32 output (device); fully written.
 * Two passes are enqueued: row log-sum-exp, then tile sums of exp(s - lse).
 */
calibatt_status calibatt_block_mass(const void* Q, const void* K, int B, int H, int L, int seq_len,
                                    int d, calibatt_dtype dt, int block, float scale,
                                    float* lse_ws, float* mass, void* stream);

/*
 * The same pooling in one pass over the scores.  While the log-sum-exp is
 * accumulated, every (key block, query) pair's partial
 *     lp[b,h,kb,i] = log2 sum_{j in kb, j < seq_len} exp2(scale * log2(e) * q_i . k_j)
 * is stored in `ws`; then mass[b,h,qb,kb] = sum_{i in qb, i < seq_len}
 * exp2(lp[b,h,kb,i] - lse_i * log2(e)).  One matrix-core score product and
 * one exp per (query, key) instead of two.  Arguments as calibatt_block_mass,
 * plus:
 *   ws, ws_bytes  calibatt_block_mass_ws_bytes(B, H, L, block) bytes (device),
 *                 256-byte aligned: the partials as float32 [B, H, L/block, L]
 *                 (1.34 GB at B = 1, H = 40, L = 32,768, block 128).
 * The result equals calibatt_block_mass's up to float32 rounding (a few
 * units in the sixth significant digit); it is bitwise reproducible.
 */
calibatt_status calibatt_block_mass_single_pass(const void* Q, const void* K, int B, int H, int L, int seq_len,
                                                int d, calibatt_dtype dt, int block, float scale, float* lse_ws,
                                                float* mass, void* ws, size_t ws_bytes, void* stream);
size_t calibatt_block_mass_ws_bytes(int B, int H, int L, int block);

/*
 * Mask compile: per-prompt top-K key blocks -> cross-prompt agreement -> CSR.
 * Pages: Fig. 5(a) caption (top key blocks per query block, aggregated
 * across prompts into a mask dictionary), Fig. 3(b) caption (per-block keep
 * frequency across prompts, agreement threshold), abstract (patterns compiled
 * per layer, head and timestep).
 * For prompt p and row (h, qb) the key block kb < nkb_valid is kept when fewer
 * than keep_topk blocks precede it in the order (mass descending, kb
 * ascending; NaN last).  A block enters the CSR when at least min_agree
 * prompts keep it.  Rows with no agreed block stay empty.
 *
 *   mass       [P, H, nqb, nkb] float32 (device), e.g. calibatt_block_mass
 *              outputs of P prompts stacked.
 *   nkb_valid  key blocks eligible (<= nkb; ceil(seq_len / block)).
 *   keep_topk  K >= 0 (K >= nkb_valid keeps every eligible block).
 *   min_agree  0 <= min_agree <= P (ceil(rho * P) for agreement rho).
 *   row_ptr    [H*nqb + 1] int32 output (device).
 *   col_idx    [nnz_cap] int32 output (device).
 *   work_order [H*nqb + 9] int32 output (device), or NULL: the work order
 *              of the compiled set, as calibatt_build_schedule makes it,
 *              enqueued on `stream` after the compile; written on OK only.
 *   nnz_out    (host) int64: number of kept blocks, set on OK and on
 *              CALIBATT_ERR_CAPACITY (then col_idx is not written; call
 *              again with a larger buffer).  H*nqb*nkb_valid always suffices.
 *   ws         device workspace of calibatt_compile_ws_bytes(...) bytes,
 *              16-byte aligned.
 * Synchronises `stream` once (to read the kept count back to the host).
 */
calibatt_status calibatt_compile_masks(const float* mass, int P, int H, int nqb, int nkb,
                                       int nkb_valid, int keep_topk, int min_agree,
                                       int32_t* row_ptr, int32_t* col_idx, int64_t nnz_cap,
                                       int32_t* work_order, int64_t* nnz_out, void* ws, size_t ws_bytes,
                                       void* stream);

/*
 * Mask compile with the energy-threshold row rule instead of a fixed count.
 * Pages: Fig. S8 caption (an energy threshold epsilon per row, scheduled over
 * the normalised timestep; the schedule is the caller's: one epsilon per
 * call).  For prompt p and row (h, qb) the key block kb < nkb_valid is kept
 * when the mass of the blocks before it in the order (mass descending, kb
 * ascending; NaN last) is still short of (1 - epsilon) of the row's mass:
 * the shortest prefix of that order holding (1 - epsilon) of the mass.
 * Decided exactly: each mass becomes an integer number of 2^-40 units
 * (round half to even; NaN and negative values 0; values capped at 128, the
 * most a pooled row of 128 queries holds) and the test is
 * before * eps_den < (eps_den - eps_num) * total in 128-bit integers.
 * epsilon = 0 keeps every block with mass; epsilon = 1 keeps nothing.
 * Agreement, outputs, workspace and synchronisation as calibatt_compile_masks.
 *
 *   eps_num, eps_den  epsilon = eps_num / eps_den, 0 <= eps_num <= eps_den,
 *                     1 <= eps_den < 2^31 (a decimal 0.05 is 1 / 20).
 */
calibatt_status calibatt_compile_masks_energy(const float* mass, int P, int H, int nqb, int nkb,
                                              int nkb_valid, int64_t eps_num, int64_t eps_den,
                                              int min_agree, int32_t* row_ptr, int32_t* col_idx,
                                              int64_t nnz_cap, int32_t* work_order, int64_t* nnz_out,
                                              void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes calibatt_compile_masks(_energy) needs for these sizes (0 on bad sizes). */
size_t calibatt_compile_ws_bytes(int P, int H, int nqb, int nkb);

/*
 * Timestep sharing of a bank of compiled masks (one layer, T timesteps).
 * Pages: Fig. S11 caption (IoU between the skipped-block masks of two
 * timesteps, averaged over heads; late steps are alike), Table S3 caption
 * (timestep sharing clusters masks whose pair-wise IoU is at least tau).
 * The skipped set of (t, h) is every valid key block (kb < nkb_valid) of the
 * rows of head h that set t does not keep.  IoU(t1, t2) is the float64 mean
 * over heads of |S1 & S2| / |S1 | S2| (1 when both are empty), heads summed
 * in ascending order.  Clusters are greedy runs of consecutive timesteps: t
 * joins the current run when its IoU with every member is >= tau.  The
 * shared mask of a run keeps every block any member keeps, so no timestep
 * computes less than its own mask.
 *
 *   row_ptr         [T, H*nqb + 1] int32 (device): set t's row offsets from 0.
 *   col_idx         int32 (device): every set's columns, concatenated.
 *   set_off         [T + 1] int64 (device): set t's columns start at
 *                   col_idx + set_off[t].  The sets must be valid CSR over
 *                   nkb_valid key blocks (calibatt_validate_csr); columns
 *                   outside [0, nkb_valid) are ignored.
 *   T               1 <= T <= 1024 timesteps; nkb <= 1024.
 *   tau             the IoU threshold (not NaN; <= 0 gives one run, > 1
 *                   one run per timestep).
 *   iou             [T, T] float64 output (device).
 *   cluster_of      [T] int32 output (device): the run of each timestep.
 *   shared_row_ptr  [T, H*nqb + 1] int32 output (device): the first C rows
 *                   of offsets are written, one set per run, in the layout of
 *                   row_ptr.
 *   shared_set_off  [T + 1] int64 output (device): the first C + 1 written.
 *   shared_col_idx  [nnz_cap] int32 output (device), concatenated columns.
 *   n_clusters_out  (host) the run count C.
 *   nnz_out         (host) columns of all shared sets; set on OK and on
 *                   CALIBATT_ERR_CAPACITY (then shared_col_idx is not
 *                   written).  T*H*nqb*nkb_valid always suffices.
 *   ws              device workspace of calibatt_share_ws_bytes(...) bytes,
 *                   256-byte aligned.
 * Synchronises `stream` twice (to read C and the kept count).
 */
calibatt_status calibatt_share_timesteps(const int32_t* row_ptr, const int32_t* col_idx,
                                         const int64_t* set_off, int T, int H, int nqb, int nkb,
                                         int nkb_valid, double tau, double* iou, int32_t* cluster_of,
                                         int32_t* shared_row_ptr, int64_t* shared_set_off,
                                         int32_t* shared_col_idx, int64_t nnz_cap,
                                         int32_t* n_clusters_out, int64_t* nnz_out, void* ws,
                                         size_t ws_bytes, void* stream);

/* Workspace bytes calibatt_share_timesteps needs for these sizes (0 on bad sizes). */
size_t calibatt_share_ws_bytes(int T, int H, int nqb, int nkb);

/*
 * Interval-encoded skip lists of a bank of T compiled sets (one layer).
 * Pages: Fig. S10 caption (each row stores interval pairs for one (timestep,
 * head, query block) entry, padded past its data; per-layer trimming to the
 * widest row; merging outlier rows lowers the width), Fig. S9 caption (row
 * widths vary widely), Table S3 (merge percentages; merging fills a few
 * skipped blocks).  A row's intervals are its maximal runs of kept key
 * blocks, half-open [start, end), ascending.  The layer width is the
 * nearest-rank merge_num/merge_den-th percentile of the E = T*H*nqb row
 * widths (the smallest w with at least ceil(p/100 * E) rows no wider; 1 if
 * that is 0 while some row keeps blocks); p = 100 is plain trimming.  A
 * wider row fills its smallest gaps between consecutive intervals, ties to
 * the leftmost, until it has `width` intervals.
 *
 *   row_ptr, col_idx, set_off  the bank, as for calibatt_share_timesteps
 *                     (valid CSR, ascending columns, nkb <= 1024).
 *   merge_num/den     the percentile p in (0, 100], e.g. 95/1.
 *   counts            [E] int32 output (device): intervals of entry
 *                     e = t*H*nqb + r.
 *   pairs             [E, width, 2] int32 output (device): (start, end) of
 *                     each interval, (-1, -1) past counts[e]; rows of
 *                     `width` pairs, so width_cap >= width must hold.
 *   width_out         (host) the layer width; also set on
 *                     CALIBATT_ERR_CAPACITY (then pairs is not written).
 *   widest_out        (host) the widest row before merging.
 *   ws                calibatt_skip_ws_bytes(T, H, nqb) bytes, 256-byte
 *                     aligned.
 * Synchronises `stream` once (to read the width).
 */
calibatt_status calibatt_encode_skip_lists(const int32_t* row_ptr, const int32_t* col_idx,
                                           const int64_t* set_off, int T, int H, int nqb, int nkb,
                                           int64_t merge_num, int64_t merge_den, int32_t* counts,
                                           int32_t* pairs, int width_cap, int32_t* width_out,
                                           int32_t* widest_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Skip lists back to a bank of CSR sets (the kept blocks of every interval,
 * ascending), so the attention entry points run on the merged masks.
 *   counts, pairs, width  as written by calibatt_encode_skip_lists.
 *   row_ptr   [T, H*nqb + 1] int32 output (device), per-set offsets from 0.
 *   set_off   [T + 1] int64 output (device): set t starts at col_idx + set_off[t].
 *   col_idx   [nnz_cap] int32 output (device).
 *   nnz_out   (host) columns of all sets; set on OK and on CALIBATT_ERR_CAPACITY.
 *   ws        calibatt_skip_ws_bytes(T, H, nqb) bytes, 256-byte aligned.
 * Synchronises `stream` once (to read the count).
 */
calibatt_status calibatt_decode_skip_lists(const int32_t* counts, const int32_t* pairs, int width, int T,
                                           int H, int nqb, int32_t* row_ptr, int64_t* set_off,
                                           int32_t* col_idx, int64_t nnz_cap, int64_t* nnz_out, void* ws,
                                           size_t ws_bytes, void* stream);

/* Workspace bytes the skip-list encode and decode need (0 on bad sizes). */
size_t calibatt_skip_ws_bytes(int T, int H, int nqb);

/*
 * Spatial-repetition score per attention map (calibration).  Pages: Fig. 4
 * caption (a query frame's attention repeats from one spatial row to the
 * next), Fig. 6 caption (one spatial-similarity score per map), Fig. S13
 * caption (heads above tau = 0.87).  The pages give no formula; this is the
 * mean, over every token i = (f, y, x) with y < grid_rows - 1 and its
 * neighbour one spatial row down, i' = i + grid_cols, of the cosine of their
 * softmax rows over the valid keys:
 *     sim[b,h] = mean_i  sum_j p_ij p_i'j / sqrt(sum_j p_ij^2 sum_j p_i'j^2)
 * Tokens are n = (f*grid_rows + y)*grid_cols + x on a (frames, grid_rows,
 * grid_cols) grid that covers exactly seq_len tokens.
 *   Q, K     [B, H, L, d] bf16 (device); L a multiple of 128, d in {64, 128}.
 *   lse_in   [B, H, L] float32 (device) or NULL: the per-query log-sum-exp
 *            over the same Q, K, scale and seq_len, as calibatt_block_mass
 *            and calibatt_block_mass_single_pass leave in their lse_ws (the
 *            pooling of the same prompt); NULL computes it here.
 *   sim      [B, H] float64 output (device).
 *   ws       calibatt_similarity_ws_bytes(B, H, L) bytes (device), 256-byte
 *            aligned: per-query log-sum-exp and per-tile partial sums.
 * Softmax rows are formed in float32 from the bf16 matrix-core scores; each
 * workgroup adds its cosines in a fixed order in float64 and the partials
 * are added in tile order, so the result is bitwise reproducible.
 * grid_rows < 2 or a grid that does not cover seq_len: CALIBATT_ERR_SHAPE.
 */
calibatt_status calibatt_spatial_similarity(const void* Q, const void* K, int B, int H, int L, int seq_len,
                                            int d, calibatt_dtype dt, float scale, int frames, int grid_rows,
                                            int grid_cols, const float* lse_in, double* sim, void* ws,
                                            size_t ws_bytes, void* stream);
size_t calibatt_similarity_ws_bytes(int B, int H, int L);

/*
 * Heads flagged as spatially repetitive (Fig. 5(a) caption: a dictionary of
 * such heads; Fig. S13 caption: score above tau).  The score of head h is the
 * mean over the P calibration prompts, added in prompt order in float64; h is
 * selected when that mean is strictly greater than tau.
 *   sim      [P, H] float64 (device), e.g. P calls of
 *            calibatt_spatial_similarity with B = 1.
 *   heads    [H] int32 output (host): the selected heads, ascending.
 *   n_heads  int32 output (host): how many.
 * Synchronizes `stream` (the scores are read back to the host).
 */
calibatt_status calibatt_select_repetitive_heads(const double* sim, int P, int H, double tau, int32_t* heads,
                                                 int32_t* n_heads, void* stream);

/*
 * Anchor-row attention for spatially repetitive heads (inference).  Pages:
 * Fig. 5(b) caption (attention only for anchor rows of each frame, outputs
 * handed to the neighbouring rows), Table S4 (anchors attend to all keys;
 * 1 - k/30 of the query rows skipped at 30 rows per frame).  The rows of a
 * frame form k_anchor contiguous groups [floor(g*R/k), floor((g+1)*R/k))
 * (R = grid_rows), each anchored at its lower middle row
 * floor((lo + hi - 1)/2).  For each listed head h and token n = (f, y, x) <
 * seq_len, with a = the anchor row of y's group:
 *     O[b,h,n,:] = attention of query (f, a, x) over all valid keys
 * and O[b,h,n,:] = 0 for n >= seq_len.  Heads not listed are not written.
 *   Q, K, V, O  as in calibatt_dense_attn_fwd; bf16 only, block 128; scale
 *               finite and > 0; O must not overlap Q, K or V.
 *   heads       [n_heads] int32 (host): distinct heads in [0, H); at most 256.
 *   frames, grid_rows, grid_cols  the token grid (frames*grid_rows*grid_cols
 *               = seq_len); 1 <= k_anchor <= grid_rows.
 *   queue_ws    int32 workspace of >= 128 entries (device), required.
 *   v_layout    as in calibatt_sparse_attn_fwd.
 *   ws          calibatt_anchor_ws_bytes(B, H, frames, grid_cols, k_anchor,
 *               d) bytes (device), 256-byte aligned: the anchor outputs as
 *               [B, H, Lq, d] (Lq = frames * k_anchor * grid_cols rounded up
 *               to 128) and the row order (up to 8 entries per row).
 * The anchor queries run through the persistent dense kernel in a
 * split-query mode that reads each anchor query of Q in place (bf16 matrix
 * cores with float32 accumulation, float32 softmax, probabilities and O
 * rounded to bf16); a copy kernel then writes every token's row.  When the
 * anchor rows are too few to keep every wave group of the device busy, each
 * row is cut into 2, 4 or 8 parts over its key blocks; the parts' outputs
 * (bf16) and log-sum-exps go to the listed heads' rows of O first, a merge
 * kernel combines them into ws, and the copy then overwrites those rows.
 */
calibatt_status calibatt_anchor_attn_fwd(const void* Q, const void* K, const void* V, void* O,
                                         const int32_t* heads, int n_heads, int frames, int grid_rows,
                                         int grid_cols, int k_anchor, float scale, int B, int H, int L,
                                         int seq_len, int d, calibatt_dtype dt, int32_t* queue_ws,
                                         calibatt_vlayout v_layout, void* ws, size_t ws_bytes, void* stream);
size_t calibatt_anchor_ws_bytes(int B, int H, int frames, int grid_cols, int k_anchor, int d);

/*
 * Parts (1, 2, 4 or 8) calibatt_anchor_attn_fwd cuts each anchor row into,
 * for n_heads listed heads on a device with num_cu compute units (two wave
 * groups each, every group taking whole parts): the smallest S that
 * minimises ceil(rows*S / groups) * (ceil(n/S) + 4), n = ceil(seq_len/128)
 * key blocks and 4 blocks for a row switch, a larger S only when it saves
 * 2%, with S <= n and S*Lq*(2d+4) <= L*2d bytes.  0 for invalid arguments.
 * A host function (no device access).
 */
int calibatt_anchor_parts(int B, int n_heads, int frames, int grid_cols, int k_anchor, int L, int seq_len, int d,
                          int num_cu);

/*
 * Work order for calibatt_sparse_attn_fwd.  The pages do not describe a
 * scheduler; rows keep very different numbers of blocks (Fig. S9's
 * skip-list row lengths).  Heads (cost = kept blocks) are given, longest
 * first, to the least-loaded of 8 partitions (ties: lowest partition), one
 * partition per XCD so a head's K/V stays in one L2; a partition lists its
 * heads in that order and each head's rows by kept count descending, ties by
 * ascending qb.
 *   row_ptr     [H*nqb + 1] int32 (device).  H <= 1024, nqb <= 1024.
 *   work_order  [H*nqb + 9] int32 output (device): row indices h*nqb + qb of
 *               the 8 lists, then the 9 list offsets.
 */
calibatt_status calibatt_build_schedule(const int32_t* row_ptr, int H, int nqb,
                                        int32_t* work_order, void* stream);

/*
 * Host-side CSR check (no GPU use).  row_ptr (host) [rows + 1], col_idx
 * (host) [nnz].  Returns CALIBATT_OK, or CALIBATT_ERR_CSR naming the first
 * defect (row_ptr[0] != 0, decreasing offsets, row_ptr[rows] != nnz, a column
 * out of [0, nkb_valid), columns not strictly ascending).
 */
calibatt_status calibatt_validate_csr(const int32_t* row_ptr, const int32_t* col_idx, int rows,
                                      int nkb_valid, int64_t nnz);

/* Static text for a status code. */
const char* calibatt_status_string(calibatt_status s);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* calibatt_last_error(void);

/* CALIBATT_VERSION of the built library. */
int calibatt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CALIBATT_H */
