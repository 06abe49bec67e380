// Internal launch interface between the C ABI (api.hip) and the kernels.
// Arguments arrive here already validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace calibatt {

struct AttnArgs {
  const void* Q;
  const void* K;
  const void* V;               // V [B, H, L, d], or V^T [B, H, d, L] with v_transposed
  void* O;
  const int32_t* row_ptr;      // unused by the dense kernel
  const int32_t* col_idx;      // unused by the dense kernel
  const int32_t* work_order;   // [rows + kParts + 1] or null
  int32_t* queue;              // [kQueueInts] or null (one workgroup per row)
  int B, H, L, seq_len, d, block, nkb_valid;
  float scale;
  bool dtype_f32;
  bool v_transposed = false;
  int num_cu;
  // anchor-row launches only: rows index the q_valid anchor queries (padded
  // to Lq, a multiple of 128) of a (frames, grid_rows, grid_cols) token grid
  // with k_anchor anchors per frame; Q is read through the anchor map, O is
  // [B, H, Lq, d]
  int Lq = 0, q_valid = 0, grid_rows = 0, grid_cols = 0, k_anchor = 0;
  // rows split into 2^split_shift parts over their key blocks; O then has
  // ostride rows per head (the parts' rows and log-sum-exps)
  int split_shift = 0, ostride = 0;
};

hipError_t launch_attention(const AttnArgs& a, bool dense, hipStream_t st);
// Dense attention of the anchor queries (bf16, block 128; needs a work_order
// that lists the rows to run, and a queue).
hipError_t launch_anchor_attention(const AttnArgs& a, hipStream_t st);

struct TransposeArgs {
  const void* V;   // [B, H, L, d]
  void* Vt;        // [B, H, d, L]
  int B, H, L, seq_len, d;
  bool dtype_f32;
};

hipError_t launch_transpose_v(const TransposeArgs& a, hipStream_t st);

struct MassArgs {
  const void* Q;
  const void* K;
  float* lse;
  float* mass;
  int B, H, L, seq_len, d, block, nkb_valid;
  float scale;
};

hipError_t launch_block_mass(const MassArgs& a, hipStream_t st);
// The single-pass pooling: lpart is a [B, H, L/block, L] float32 workspace.
hipError_t launch_block_mass_single(const MassArgs& a, float* lpart, hipStream_t st);
// Pass 1 of the pooling alone: lse per query over the valid keys (block 128 tiles).
hipError_t launch_row_lse(const MassArgs& a, hipStream_t st);

// Heads handed to a kernel by value (kernel arguments), so that no device
// list has to be written first.
constexpr int kMaxListHeads = 256;
// anchor rows are cut into at most this many parts over their key blocks
constexpr int kMaxSplit = 8;
struct HeadList {
  int n;
  int32_t h[kMaxListHeads];
};

struct SimArgs {
  const void* Q;
  const void* K;
  const float* lse_in;   // [B, H, L] log-sum-exp given by the caller, or null
  float* lse;      // [B, H, L] (computed here when lse_in is null)
  double* part;    // [B, H, L/128]
  double* sim;     // [B, H]
  int B, H, L, seq_len, d;
  int frames, rows, cols;
  float scale;
};

hipError_t launch_spatial_similarity(const SimArgs& a, hipStream_t st);

struct AnchorArgs {
  const void* Q;
  const void* K;
  const void* V;   // [B, H, L, d], or V^T [B, H, d, L] with v_transposed
  bool v_transposed;
  void* O;
  void* Oa;        // [B, H, Lq, d]
  int32_t* order;  // [H*(Lq/128)*kMaxSplit + kParts + 1]
  int32_t* queue;
  HeadList heads;
  int B, H, L, seq_len, d;
  int rows, cols, k;   // grid rows and columns, anchors per frame
  int La, Lq;          // anchor queries, padded to a multiple of 128
  float scale;
  int num_cu;
};

hipError_t launch_anchor_fwd(const AnchorArgs& a, hipStream_t st);
// log2 of the parts each anchor row is cut into over its key blocks (rows:
// anchor rows of all listed heads and batch entries; groups: two per CU)
int anchor_split_shift(long long rows, int groups, int nkb, long long Lq, long long L, int d);

struct CompileArgs {
  const float* mass;
  int P, H, nqb, nkb, nkb_valid, keep_topk, min_agree;
  // per-prompt row rule: top keep_topk blocks, or (energy) the shortest
  // prefix holding (1 - eps_num/eps_den) of the row's mass
  bool energy = false;
  long long eps_num = 0, eps_den = 1;
  int32_t* row_ptr;
  int32_t* col_idx;
  uint8_t* keep_ws;   // [H*nqb*nkb]
  int32_t* count_ws;  // [H*nqb]
};

// Enqueues the per-row keep/agree pass and the row-offset scan.
hipError_t launch_compile_count(const CompileArgs& a, hipStream_t st);
// Enqueues the column fill (after the caller checked the kept count fits).
hipError_t launch_compile_fill(const CompileArgs& a, hipStream_t st);

hipError_t launch_schedule(const int32_t* row_ptr, int H, int nqb, int32_t* work_order,
                           hipStream_t st);

// Exclusive scan of n counts into offsets[0 .. n] (one workgroup).
hipError_t launch_row_offsets(const int32_t* counts, int n, int32_t* offsets, hipStream_t st);

struct ShareArgs {
  const int32_t* row_ptr;   // [T, rows + 1] per-set offsets
  const int32_t* col_idx;   // concatenated columns
  const int64_t* set_off;   // [T + 1]
  int T, H, nqb, nkb, nkb_valid, W;
  double tau;
  double* iou;              // [T, T]
  int32_t* cluster_of;      // [T]
  int32_t* shared_row_ptr;  // [C, rows + 1]
  int64_t* shared_set_off;  // [C + 1]
  int32_t* shared_col_idx;
  // workspace
  uint32_t* bits;           // [T, rows, W]
  uint32_t* shared_bits;    // [T, rows, W] (C <= T runs)
  int32_t* counts;          // [T * rows]
  int32_t* global_ptr;      // [T * rows + 1]
  int32_t* n_clusters;      // [1]
};

// Bitmasks, pair IoU, runs and the OR of each run (no host sync).
hipError_t launch_share_cluster(const ShareArgs& a, hipStream_t st);
// Row counts of the C shared sets and their global offsets.
hipError_t launch_share_count(const ShareArgs& a, int C, hipStream_t st);
// Per-set offsets, set starts and the column fill.
hipError_t launch_share_fill(const ShareArgs& a, int C, hipStream_t st);
// Global offsets over (set, row) -> per-set offsets from 0 and set starts.
hipError_t launch_local_offsets(const int32_t* global, int C, int rows, int32_t* local, int64_t* set_off,
                                hipStream_t st);

struct SkipArgs {
  const int32_t* row_ptr;   // [T, rows + 1] per-set offsets
  const int32_t* col_idx;
  const int64_t* set_off;   // [T + 1]
  int T, H, nqb;
  long long pct_num, pct_den;   // merge percentile, percent
  int32_t* counts;          // [E] output
  int32_t* pairs;           // [E, width, 2] output
  // workspace
  int32_t* widths;          // [E]
  int32_t* hist;            // [kMaxKeyBlocks / 2 + 1]
  int32_t* width_dev;       // [2]: layer width, widest row
};

struct SkipDecodeArgs {
  const int32_t* counts;
  const int32_t* pairs;
  int W, T, H, nqb;
  int32_t* row_ptr;         // [T, rows + 1] output
  int64_t* set_off;         // [T + 1] output
  int32_t* col_idx;         // output
  // workspace
  int32_t* kept;            // [E]
  int32_t* global_ptr;      // [E + 1]
};

// Row widths, their histogram and the layer width (no host sync).
hipError_t launch_skip_widths(const SkipArgs& a, hipStream_t st);
// The (merged) runs of every entry, after the caller checked the width fits.
hipError_t launch_skip_encode(const SkipArgs& a, hipStream_t st);
hipError_t launch_skip_decode_count(const SkipDecodeArgs& a, hipStream_t st);
hipError_t launch_skip_decode_fill(const SkipDecodeArgs& a, hipStream_t st);

constexpr int kMaxKeyBlocks = 1024;   // calibration and compile kernels keep a row in LDS
constexpr int kMaxHeads = 1024;       // the work-order kernel keeps all head costs in LDS
// Work partitions: MI355X has 8 XCDs and places workgroup i of a launch on XCD
// i % 8, so a persistent workgroup serves partition blockIdx.x % 8 first.
constexpr int kParts = 8;
constexpr int kQueueStride = 16;      // int32 between partition counters (64 bytes)
constexpr int kQueueInts = kParts * kQueueStride;

}  // namespace calibatt
