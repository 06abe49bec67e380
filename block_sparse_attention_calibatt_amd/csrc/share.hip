// Timestep sharing of compiled masks for gfx950.
//
// Pages: Fig. S11 caption (the IoU of two timesteps' skipped-block masks,
// averaged over heads; later steps are alike), Table S3 caption (timestep
// sharing clusters masks whose pair-wise IoU is at least tau).  A head's
// skipped set is its valid key blocks (kb < nkb_valid) not kept.  IoU(t1, t2)
// is the float64 mean over heads of |S1 & S2| / |S1 | S2| (1 for two empty
// sets), the heads summed in ascending order.  Clusters are greedy runs of
// consecutive timesteps whose pair-wise IoU reaches tau; a cluster's shared
// mask keeps every block any member keeps.
//
// Kernels: csr_to_bits (one thread per (set, row): the row's kept blocks as
// a bitmask of W = ceil(nkb / 32) words), pair_iou (one workgroup per pair:
// per head, popcounts of the skipped sets' intersection and union, reduced
// in the workgroup), cluster_runs (one thread: the greedy runs), union_bits
// (one thread per (row, word): OR over each run), shared_counts,
// row_offsets (from compile.hip's scan), local_offsets and fill_bits (CSR of
// every shared set, in the bank layout: per-set row offsets from 0 and one
// concatenated column array).
#include "tiles.h"
#include "launch.h"

namespace calibatt {

constexpr int kShareThreads = 256;

// Valid-block bits of word j of a row (blocks 32j .. 32j+31 below nkb_valid).
__device__ __forceinline__ uint32_t valid_word(int j, int nkb_valid) {
  const int lo = 32 * j;
  if (nkb_valid >= lo + 32) return 0xffffffffu;
  if (nkb_valid <= lo) return 0u;
  return (1u << (nkb_valid - lo)) - 1u;
}

__global__ void zero_u32_kernel(uint32_t* __restrict__ p, long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

__global__ __launch_bounds__(kShareThreads) void csr_to_bits_kernel(const int32_t* __restrict__ row_ptr,
                                                                    const int32_t* __restrict__ col_idx,
                                                                    const int64_t* __restrict__ set_off, int T,
                                                                    int rows, int W, int nkb_valid,
                                                                    uint32_t* __restrict__ bits) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)T * rows) return;
  const int t = (int)(i / rows), r = (int)(i - (long long)t * rows);
  const int32_t* rp = row_ptr + (size_t)t * (rows + 1);
  const int32_t* ci = col_idx + set_off[t];
  uint32_t* out = bits + (size_t)i * W;
  for (int e = rp[r]; e < rp[r + 1]; ++e) {
    const int kb = ci[e];
    if (kb >= 0 && kb < nkb_valid) out[kb >> 5] |= 1u << (kb & 31);   // this thread owns the row
  }
}

__global__ __launch_bounds__(kShareThreads) void pair_iou_kernel(const uint32_t* __restrict__ bits, int T,
                                                                 int H, int nqb, int W, int nkb_valid,
                                                                 double* __restrict__ iou) {
  const int t1 = blockIdx.x, t2 = blockIdx.y;
  if (t2 < t1) return;
  if (t1 == t2) {
    if (threadIdx.x == 0) iou[(size_t)t1 * T + t1] = 1.0;
    return;
  }
  __shared__ int s_i[kShareThreads / 64], s_u[kShareThreads / 64];
  const size_t set_words = (size_t)H * nqb * W;
  const uint32_t* b1 = bits + (size_t)t1 * set_words;
  const uint32_t* b2 = bits + (size_t)t2 * set_words;
  const int head_words = nqb * W;
  double acc = 0.0;
  for (int h = 0; h < H; ++h) {
    int ni = 0, nu = 0;
    for (int w = threadIdx.x; w < head_words; w += kShareThreads) {
      const uint32_t v = valid_word(w % W, nkb_valid);
      const uint32_t s1 = ~b1[(size_t)h * head_words + w] & v;
      const uint32_t s2 = ~b2[(size_t)h * head_words + w] & v;
      ni += __popc(s1 & s2);
      nu += __popc(s1 | s2);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      ni += __shfl_xor(ni, off);
      nu += __shfl_xor(nu, off);
    }
    if ((threadIdx.x & 63) == 0) {
      s_i[threadIdx.x >> 6] = ni;
      s_u[threadIdx.x >> 6] = nu;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int ti = 0, tu = 0;
      for (int k = 0; k < kShareThreads / 64; ++k) ti += s_i[k], tu += s_u[k];
      acc += tu == 0 ? 1.0 : (double)ti / (double)tu;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double m = acc / (double)H;
    iou[(size_t)t1 * T + t2] = m;
    iou[(size_t)t2 * T + t1] = m;
  }
}

// One thread: runs of consecutive timesteps with pair-wise IoU >= tau.
__global__ void cluster_runs_kernel(const double* __restrict__ iou, int T, double tau,
                                    int32_t* __restrict__ cluster_of, int32_t* __restrict__ n_clusters) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int start = 0, c = 0;
  cluster_of[0] = 0;
  for (int t = 1; t < T; ++t) {
    bool joins = true;
    for (int u = start; u < t; ++u) joins = joins && (iou[(size_t)u * T + t] >= tau);
    if (!joins) {
      ++c;
      start = t;
    }
    cluster_of[t] = c;
  }
  *n_clusters = c + 1;
}

__global__ __launch_bounds__(kShareThreads) void union_bits_kernel(const uint32_t* __restrict__ bits,
                                                                   const int32_t* __restrict__ cluster_of, int T,
                                                                   long long row_words,
                                                                   uint32_t* __restrict__ shared) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= row_words) return;
  int cur = cluster_of[0];
  uint32_t acc = 0u;
  for (int t = 0; t < T; ++t) {
    const int c = cluster_of[t];
    if (c != cur) {
      shared[(size_t)cur * row_words + i] = acc;
      acc = 0u;
      cur = c;
    }
    acc |= bits[(size_t)t * row_words + i];
  }
  shared[(size_t)cur * row_words + i] = acc;
}

__global__ __launch_bounds__(kShareThreads) void shared_counts_kernel(const uint32_t* __restrict__ shared,
                                                                      long long n_rows, int W,
                                                                      int32_t* __restrict__ counts) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_rows) return;
  int n = 0;
  for (int j = 0; j < W; ++j) n += __popc(shared[(size_t)i * W + j]);
  counts[i] = n;
}

// Global offsets over (cluster, row) -> per-set offsets from 0 and set starts.
__global__ __launch_bounds__(kShareThreads) void local_offsets_kernel(const int32_t* __restrict__ global,
                                                                      int C, int rows,
                                                                      int32_t* __restrict__ local,
                                                                      int64_t* __restrict__ set_off) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)C * (rows + 1)) return;
  const int c = (int)(i / (rows + 1)), k = (int)(i - (long long)c * (rows + 1));
  const int32_t base = global[(size_t)c * rows];
  local[i] = global[(size_t)c * rows + k] - base;
  if (k == 0) set_off[c] = base;
  if (i == 0) set_off[C] = global[(size_t)C * rows];
}

__global__ __launch_bounds__(kShareThreads) void fill_bits_kernel(const uint32_t* __restrict__ shared,
                                                                  long long n_rows, int W,
                                                                  const int32_t* __restrict__ global,
                                                                  int32_t* __restrict__ col_idx) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_rows) return;
  int pos = global[i];
  for (int j = 0; j < W; ++j) {
    uint32_t v = shared[(size_t)i * W + j];
    while (v) {
      const int b = __ffs(v) - 1;
      col_idx[pos++] = 32 * j + b;
      v &= v - 1u;
    }
  }
}

static inline unsigned blocks_for(long long n) { return (unsigned)((n + kShareThreads - 1) / kShareThreads); }

hipError_t launch_share_cluster(const ShareArgs& a, hipStream_t st) {
  const int rows = a.H * a.nqb;
  const long long row_words = (long long)rows * a.W;
  const long long all_words = row_words * a.T;
  hipLaunchKernelGGL(zero_u32_kernel, dim3(blocks_for(all_words)), dim3(kShareThreads), 0, st, a.bits, all_words);
  hipLaunchKernelGGL(csr_to_bits_kernel, dim3(blocks_for((long long)a.T * rows)), dim3(kShareThreads), 0, st,
                     a.row_ptr, a.col_idx, a.set_off, a.T, rows, a.W, a.nkb_valid, a.bits);
  hipLaunchKernelGGL(pair_iou_kernel, dim3(a.T, a.T), dim3(kShareThreads), 0, st, (const uint32_t*)a.bits, a.T,
                     a.H, a.nqb, a.W, a.nkb_valid, a.iou);
  hipLaunchKernelGGL(cluster_runs_kernel, dim3(1), dim3(64), 0, st, (const double*)a.iou, a.T, a.tau,
                     a.cluster_of, a.n_clusters);
  hipLaunchKernelGGL(union_bits_kernel, dim3(blocks_for(row_words)), dim3(kShareThreads), 0, st,
                     (const uint32_t*)a.bits, (const int32_t*)a.cluster_of, a.T, row_words, a.shared_bits);
  return hipGetLastError();
}

hipError_t launch_share_count(const ShareArgs& a, int C, hipStream_t st) {
  const long long n_rows = (long long)C * a.H * a.nqb;
  hipLaunchKernelGGL(shared_counts_kernel, dim3(blocks_for(n_rows)), dim3(kShareThreads), 0, st,
                     (const uint32_t*)a.shared_bits, n_rows, a.W, a.counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_row_offsets(a.counts, (int)n_rows, a.global_ptr, st);
}

hipError_t launch_local_offsets(const int32_t* global, int C, int rows, int32_t* local, int64_t* set_off,
                                hipStream_t st) {
  hipLaunchKernelGGL(local_offsets_kernel, dim3(blocks_for((long long)C * (rows + 1))), dim3(kShareThreads), 0, st,
                     global, C, rows, local, set_off);
  return hipGetLastError();
}

hipError_t launch_share_fill(const ShareArgs& a, int C, hipStream_t st) {
  const int rows = a.H * a.nqb;
  const long long n_rows = (long long)C * rows;
  hipLaunchKernelGGL(local_offsets_kernel, dim3(blocks_for((long long)C * (rows + 1))), dim3(kShareThreads), 0, st,
                     (const int32_t*)a.global_ptr, C, rows, a.shared_row_ptr, a.shared_set_off);
  hipLaunchKernelGGL(fill_bits_kernel, dim3(blocks_for(n_rows)), dim3(kShareThreads), 0, st,
                     (const uint32_t*)a.shared_bits, n_rows, a.W, (const int32_t*)a.global_ptr, a.shared_col_idx);
  return hipGetLastError();
}

}  // namespace calibatt
