// Interval-encoded skip lists ("2D skip lists") for gfx950.
//
// Pages: Fig. S10 caption (each row of a layer's skip list stores interval
// pairs for one (timestep, head, query block) entry, padded past its data;
// per-layer trimming to the widest row; merging outlier rows lowers the
// layer's width), Fig. S9 caption (row widths vary widely), Table S3 (merge
// percentages; merging fills a few skipped blocks).  A row's intervals are
// its maximal runs of kept key blocks, half-open.  "Merge p%" sets the
// layer width to the nearest-rank p-th percentile of the row widths (the
// smallest w with at least ceil(p/100 * E) of the E rows no wider; 1 if that
// is 0 while some row keeps blocks); a wider row fills its smallest gaps,
// ties to the leftmost.  Padding pairs are (-1, -1).
//
// Kernels: row_widths (one thread per entry: interval count, and a histogram
// of the counts), pick_width (one thread: the percentile from the
// histogram), encode_rows (one wave per entry: runs from the row's columns
// with ballots into LDS, and for a row wider than the layer the rank of each
// gap among the row's gaps, then the merged runs), decode_counts / fill
// (CSR of every set back from the pairs, in the mask-bank layout).
#include "tiles.h"
#include "launch.h"

namespace calibatt {

constexpr int kSkipThreads = 256;
constexpr int kMaxRuns = kMaxKeyBlocks / 2;   // a row of nkb <= 1024 blocks has at most 512 runs
constexpr int kHistBins = kMaxRuns + 1;

__global__ void zero_i32_kernel(int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Row (entry e = t * rows + r) of the bank: columns and count.
struct BankRow {
  const int32_t* cols;
  int n;
};

__device__ __forceinline__ BankRow bank_row(const int32_t* row_ptr, const int32_t* col_idx, const int64_t* set_off,
                                            int rows, long long e) {
  const int t = (int)(e / rows), r = (int)(e - (long long)t * rows);
  const int32_t* rp = row_ptr + (size_t)t * (rows + 1);
  return BankRow{col_idx + set_off[t] + rp[r], rp[r + 1] - rp[r]};
}

__global__ __launch_bounds__(kSkipThreads) void row_widths_kernel(const int32_t* __restrict__ row_ptr,
                                                                  const int32_t* __restrict__ col_idx,
                                                                  const int64_t* __restrict__ set_off, int rows,
                                                                  long long E, int32_t* __restrict__ widths,
                                                                  int32_t* __restrict__ hist) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const BankRow row = bank_row(row_ptr, col_idx, set_off, rows, e);
  int w = 0;
  for (int j = 0; j < row.n; ++j) w += (j == 0 || row.cols[j] != row.cols[j - 1] + 1) ? 1 : 0;
  w = w < kMaxRuns ? w : kMaxRuns;   // valid lists never exceed it; keeps the histogram in range
  widths[e] = w;
  atomicAdd(hist + w, 1);
}

// out[0] = layer width, out[1] = widest row.
__global__ void pick_width_kernel(const int32_t* __restrict__ hist, long long E, long long pct_num, long long pct_den,
                                  int32_t* __restrict__ out) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  // need = ceil(pct_num / pct_den / 100 * E), in integers (pct <= 100, E < 2^31)
  const unsigned __int128 num = (unsigned __int128)(unsigned long long)pct_num * (unsigned long long)E;
  const unsigned __int128 den = (unsigned __int128)(unsigned long long)pct_den * 100u;
  const long long need = (long long)((num + den - 1) / den);
  long long cum = 0;
  int w = -1, widest = 0;
  for (int b = 0; b < kHistBins; ++b) {
    cum += hist[b];
    if (w < 0 && cum >= need) w = b;
    if (hist[b] > 0) widest = b;
  }
  if (w < 0) w = widest;
  if (w == 0 && widest > 0) w = 1;   // a row that keeps anything needs one interval
  out[0] = w;
  out[1] = widest;
}

// One wave per entry.  LDS per wave: run starts, run ends, gap-filled flags.
__global__ __launch_bounds__(kSkipThreads) void encode_rows_kernel(const int32_t* __restrict__ row_ptr,
                                                                   const int32_t* __restrict__ col_idx,
                                                                   const int64_t* __restrict__ set_off, int rows,
                                                                   long long E, const int32_t* __restrict__ width_p,
                                                                   int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ pairs) {
  constexpr int NW = kSkipThreads / 64;
  __shared__ int s_start[NW][kMaxRuns];
  __shared__ int s_end[NW][kMaxRuns];
  __shared__ uint8_t s_fill[NW][kMaxRuns];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const long long e = (long long)blockIdx.x * NW + wv;
  if (e >= E) return;   // whole waves leave together; no workgroup barrier below
  const int W = *width_p;
  const BankRow row = bank_row(row_ptr, col_idx, set_off, rows, e);
  int* S = s_start[wv];
  int* En = s_end[wv];
  uint8_t* F = s_fill[wv];
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  // runs of consecutive columns
  int n_start = 0, n_end = 0;
  for (int base = 0; base < row.n; base += 64) {
    const int j = base + lane;
    const bool in = j < row.n;
    const int c = in ? row.cols[j] : 0;
    const bool st = in && (j == 0 || row.cols[j - 1] + 1 != c);
    const bool en = in && (j == row.n - 1 || row.cols[j + 1] != c + 1);
    const unsigned long long bs = __ballot(st), be = __ballot(en);
    if (st) {
      const int k = n_start + __popcll(bs & below);
      if (k < kMaxRuns) S[k] = c;
    }
    if (en) {
      const int k = n_end + __popcll(be & below);
      if (k < kMaxRuns) En[k] = c + 1;
    }
    n_start += __popcll(bs);
    n_end += __popcll(be);
  }
  __builtin_amdgcn_wave_barrier();
  const int n = n_start < kMaxRuns ? n_start : kMaxRuns;
  int32_t* out = pairs + (size_t)e * W * 2;
  if (n <= W) {
    for (int i = lane; i < W; i += 64) {
      out[2 * i] = i < n ? S[i] : -1;
      out[2 * i + 1] = i < n ? En[i] : -1;
    }
    if (lane == 0) counts[e] = n;
    return;
  }
  // merge: fill the n - W gaps first in (length, position) order
  const int nfill = n - (W > 0 ? W : 1);
  for (int i = lane; i < n - 1; i += 64) {
    const int gi = S[i + 1] - En[i];
    int rank = 0;
    for (int k = 0; k < n - 1; ++k) {
      const int gk = S[k + 1] - En[k];
      rank += (gk < gi || (gk == gi && k < i)) ? 1 : 0;
    }
    F[i] = rank < nfill ? 1 : 0;
  }
  __builtin_amdgcn_wave_barrier();
  // run i opens an output interval when i == 0 or gap i-1 stays open; it
  // closes one when i == n-1 or gap i stays open
  int n_open = 0, n_close = 0;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    const bool in = i < n;
    const bool op = in && (i == 0 || F[i - 1] == 0);
    const bool cl = in && (i == n - 1 || F[i] == 0);
    const unsigned long long bo = __ballot(op), bc = __ballot(cl);
    if (op) out[2 * (n_open + __popcll(bo & below))] = S[i];
    if (cl) out[2 * (n_close + __popcll(bc & below)) + 1] = En[i];
    n_open += __popcll(bo);
    n_close += __popcll(bc);
  }
  for (int i = n_open + lane; i < W; i += 64) out[2 * i] = out[2 * i + 1] = -1;
  if (lane == 0) counts[e] = n_open;
}

__global__ __launch_bounds__(kSkipThreads) void decode_counts_kernel(const int32_t* __restrict__ counts,
                                                                     const int32_t* __restrict__ pairs, int W,
                                                                     long long E, int32_t* __restrict__ kept) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int c = counts[e] < W ? counts[e] : W;
  int s = 0;
  for (int i = 0; i < c; ++i) {
    const int len = pairs[((size_t)e * W + i) * 2 + 1] - pairs[((size_t)e * W + i) * 2];
    s += len > 0 ? len : 0;
  }
  kept[e] = s;
}

__global__ __launch_bounds__(kSkipThreads) void decode_fill_kernel(const int32_t* __restrict__ counts,
                                                                   const int32_t* __restrict__ pairs, int W,
                                                                   long long E, const int32_t* __restrict__ global,
                                                                   int32_t* __restrict__ col_idx) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int c = counts[e] < W ? counts[e] : W;
  int pos = global[e];
  for (int i = 0; i < c; ++i) {
    const int a = pairs[((size_t)e * W + i) * 2], b = pairs[((size_t)e * W + i) * 2 + 1];
    for (int k = a; k < b; ++k) col_idx[pos++] = k;
  }
}

static inline unsigned grid_for(long long n, int per) { return (unsigned)((n + per - 1) / per); }

hipError_t launch_skip_widths(const SkipArgs& a, hipStream_t st) {
  const long long E = (long long)a.T * a.H * a.nqb;
  const int rows = a.H * a.nqb;
  hipLaunchKernelGGL(zero_i32_kernel, dim3(grid_for(kHistBins, 256)), dim3(256), 0, st, a.hist, kHistBins);
  hipLaunchKernelGGL(row_widths_kernel, dim3(grid_for(E, kSkipThreads)), dim3(kSkipThreads), 0, st, a.row_ptr,
                     a.col_idx, a.set_off, rows, E, a.widths, a.hist);
  hipLaunchKernelGGL(pick_width_kernel, dim3(1), dim3(64), 0, st, (const int32_t*)a.hist, E, a.pct_num, a.pct_den,
                     a.width_dev);
  return hipGetLastError();
}

hipError_t launch_skip_encode(const SkipArgs& a, hipStream_t st) {
  const long long E = (long long)a.T * a.H * a.nqb;
  const int rows = a.H * a.nqb;
  hipLaunchKernelGGL(encode_rows_kernel, dim3(grid_for(E, kSkipThreads / 64)), dim3(kSkipThreads), 0, st,
                     a.row_ptr, a.col_idx, a.set_off, rows, E, (const int32_t*)a.width_dev, a.counts, a.pairs);
  return hipGetLastError();
}

hipError_t launch_skip_decode_count(const SkipDecodeArgs& a, hipStream_t st) {
  const long long E = (long long)a.T * a.H * a.nqb;
  hipLaunchKernelGGL(decode_counts_kernel, dim3(grid_for(E, kSkipThreads)), dim3(kSkipThreads), 0, st, a.counts,
                     a.pairs, a.W, E, a.kept);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_row_offsets(a.kept, (int)E, a.global_ptr, st);
}

hipError_t launch_skip_decode_fill(const SkipDecodeArgs& a, hipStream_t st) {
  const long long E = (long long)a.T * a.H * a.nqb;
  hipError_t e = launch_local_offsets(a.global_ptr, a.T, a.H * a.nqb, a.row_ptr, a.set_off, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_fill_kernel, dim3(grid_for(E, kSkipThreads)), dim3(kSkipThreads), 0, st, a.counts,
                     a.pairs, a.W, E, (const int32_t*)a.global_ptr, a.col_idx);
  return hipGetLastError();
}

}  // namespace calibatt
