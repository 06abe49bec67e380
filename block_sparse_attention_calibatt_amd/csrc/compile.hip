// Mask compile and work order for gfx950.
//
// Per-prompt keep rule (Fig. 5(a) caption: the top key blocks of each query
// block are kept): key block kb < nkb_valid of row (h, qb) is kept for prompt
// p when fewer than K blocks precede it in the total order (mass descending,
// kb ascending, NaN last).  The rank is counted exactly by comparing against
// every block of the row held in LDS, so ties resolve the same way on every
// run.  Agreement (Fig. 3(b) caption): a block enters the compiled list when
// at least min_agree prompts keep it.  Lists are CSR rows r = h*nqb + qb with
// ascending columns (the abstract compiles one pattern per layer, head and
// timestep).
//
// Energy rule (Fig. S8 caption: an energy threshold epsilon per row): the
// variant of the top-K rule.  Block kb is kept for prompt p when the mass of
// the blocks before it in the same order is still short of (1 - eps) of the
// row's mass, decided in exact integers: masses in units of 2^-40 (round half
// to even; NaN and negative values 0; capped at 128, the most a pooled
// 128-query row holds), compared as before * den < (den - num) * total in
// 128-bit products.
//
// Kernels: keep_agree (one workgroup per row: per-prompt ranks, counts,
// agreed flags, kept count), row_offsets (one workgroup: exclusive scan of
// the kept counts), fill_columns (one workgroup per row: ordered compaction
// of the agreed flags), lpt_schedule (one workgroup per head: the head's
// partition, then each row's rank by kept count descending, index ascending).
#include "tiles.h"
#include "launch.h"

namespace calibatt {

// True when (a, ia) precedes (b, ib): non-NaN first, larger mass first, smaller index first.
__device__ __forceinline__ bool precedes(float a, int ia, float b, int ib) {
  const bool na = a != a, nb = b != b;
  if (na != nb) return nb;
  if (!na && a != b) return a > b;
  return ia < ib;
}

constexpr int kRowThreads = 256;
constexpr int kPerThread = kMaxKeyBlocks / kRowThreads;

__global__ __launch_bounds__(kRowThreads) void keep_agree_kernel(
    const float* __restrict__ mass, int P, int rows, int nkb, int nkb_valid, int K, int min_agree,
    uint8_t* __restrict__ keep, int32_t* __restrict__ counts) {
  __shared__ float m[kMaxKeyBlocks];
  __shared__ int wsum[kRowThreads / 64];
  const int r = blockIdx.x;
  int cnt[kPerThread];
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) cnt[j] = 0;
  for (int p = 0; p < P; ++p) {
    __syncthreads();
    const float* src = mass + ((size_t)p * rows + r) * nkb;
    for (int kb = threadIdx.x; kb < nkb_valid; kb += kRowThreads) m[kb] = src[kb];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int kb = threadIdx.x + j * kRowThreads;
      if (kb < nkb_valid) {
        const float x = m[kb];
        int rank = 0;
        for (int o = 0; o < nkb_valid; ++o) rank += precedes(m[o], o, x, kb) ? 1 : 0;
        cnt[j] += rank < K ? 1 : 0;
      }
    }
  }
  int kept = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int kb = threadIdx.x + j * kRowThreads;
    if (kb < nkb) {
      const bool on = kb < nkb_valid && cnt[j] >= min_agree;
      keep[(size_t)r * nkb + kb] = on ? 1 : 0;
      kept += on ? 1 : 0;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) kept += __shfl_xor(kept, off);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = kept;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int i = 0; i < kRowThreads / 64; ++i) t += wsum[i];
    counts[r] = t;
  }
}

// Block mass in units of 2^-40 (see the energy rule above).
__device__ __forceinline__ unsigned long long mass_fixed(float x) {
  double d = (double)x;
  if (!(d > 0.0)) return 0ull;   // NaN, zero, negative
  if (d > 128.0) d = 128.0;
  return (unsigned long long)rint(d * 1099511627776.0);   // * 2^40, exact; rint: half to even
}

__global__ __launch_bounds__(kRowThreads) void keep_energy_kernel(
    const float* __restrict__ mass, int P, int rows, int nkb, int nkb_valid, long long eps_num,
    long long eps_den, int min_agree, uint8_t* __restrict__ keep, int32_t* __restrict__ counts) {
  __shared__ float m[kMaxKeyBlocks];
  __shared__ unsigned long long fx[kMaxKeyBlocks];
  __shared__ unsigned long long wtot[kRowThreads / 64];
  __shared__ int wsum[kRowThreads / 64];
  const int r = blockIdx.x;
  const unsigned __int128 den = (unsigned long long)eps_den;
  const unsigned __int128 keepw = (unsigned long long)(eps_den - eps_num);
  int cnt[kPerThread];
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) cnt[j] = 0;
  for (int p = 0; p < P; ++p) {
    __syncthreads();
    const float* src = mass + ((size_t)p * rows + r) * nkb;
    unsigned long long part = 0;
    for (int kb = threadIdx.x; kb < nkb_valid; kb += kRowThreads) {
      const float x = src[kb];
      m[kb] = x;
      fx[kb] = mass_fixed(x);
      part += fx[kb];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    if ((threadIdx.x & 63) == 0) wtot[threadIdx.x >> 6] = part;
    __syncthreads();
    unsigned long long total = 0;
#pragma unroll
    for (int i = 0; i < kRowThreads / 64; ++i) total += wtot[i];
    const unsigned __int128 target = keepw * total;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int kb = threadIdx.x + j * kRowThreads;
      if (kb < nkb_valid) {
        const float x = m[kb];
        unsigned long long before = 0;
        for (int o = 0; o < nkb_valid; ++o) before += precedes(m[o], o, x, kb) ? fx[o] : 0ull;
        cnt[j] += ((unsigned __int128)before * den < target) ? 1 : 0;
      }
    }
  }
  int kept = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int kb = threadIdx.x + j * kRowThreads;
    if (kb < nkb) {
      const bool on = kb < nkb_valid && cnt[j] >= min_agree;
      keep[(size_t)r * nkb + kb] = on ? 1 : 0;
      kept += on ? 1 : 0;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) kept += __shfl_xor(kept, off);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = kept;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int i = 0; i < kRowThreads / 64; ++i) t += wsum[i];
    counts[r] = t;
  }
}

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void row_offsets_kernel(const int32_t* __restrict__ counts,
                                                                   int rows,
                                                                   int32_t* __restrict__ row_ptr) {
  __shared__ int part[kScanThreads];
  const int per = (rows + kScanThreads - 1) / kScanThreads;
  const int lo = threadIdx.x * per;
  const int hi = min(lo + per, rows);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += counts[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int run = part[threadIdx.x] - s;   // exclusive prefix of this thread's chunk
  if (threadIdx.x == 0) row_ptr[0] = 0;
  for (int i = lo; i < hi; ++i) {
    run += counts[i];
    row_ptr[i + 1] = run;
  }
}

__global__ __launch_bounds__(kRowThreads) void fill_columns_kernel(const uint8_t* __restrict__ keep,
                                                                   int nkb,
                                                                   const int32_t* __restrict__ row_ptr,
                                                                   int32_t* __restrict__ col_idx) {
  __shared__ int pre[kRowThreads];
  const int r = blockIdx.x;
  // thread t owns the contiguous key blocks [t*kPerThread, t*kPerThread + kPerThread)
  const int kb0 = threadIdx.x * kPerThread;
  bool on[kPerThread];
  int n = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int kb = kb0 + j;
    on[j] = kb < nkb && keep[(size_t)r * nkb + kb] != 0;
    n += on[j] ? 1 : 0;
  }
  pre[threadIdx.x] = n;
  __syncthreads();
  for (int off = 1; off < kRowThreads; off <<= 1) {
    const int v = threadIdx.x >= off ? pre[threadIdx.x - off] : 0;
    __syncthreads();
    pre[threadIdx.x] += v;
    __syncthreads();
  }
  int pos = row_ptr[r] + pre[threadIdx.x] - n;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (on[j]) col_idx[pos++] = kb0 + j;
}

// Work order: heads go to kParts partitions longest first (greedy, ties to
// the lowest partition); a partition lists its heads in that order and each
// head's rows by kept count descending, ties by query block.  Output: the
// concatenated lists, then the kParts+1 list offsets.  Every workgroup (one
// per head) recomputes the small head assignment itself, so no scratch
// memory is needed.
__global__ __launch_bounds__(kRowThreads) void lpt_schedule_kernel(const int32_t* __restrict__ row_ptr,
                                                                   int H, int nqb,
                                                                   int32_t* __restrict__ out) {
  __shared__ int hcost[kMaxHeads];
  __shared__ int hsorted[kMaxHeads];
  __shared__ int cost[kMaxKeyBlocks];
  __shared__ int s_off[kParts + 1];
  __shared__ int s_start;
  const int h = blockIdx.x;
  const int rows = H * nqb;
  for (int i = threadIdx.x; i < H; i += kRowThreads) hcost[i] = row_ptr[(i + 1) * nqb] - row_ptr[i * nqb];
  __syncthreads();
  for (int i = threadIdx.x; i < H; i += kRowThreads) {
    const int ci = hcost[i];
    int rank = 0;
    for (int o = 0; o < H; ++o) rank += (hcost[o] > ci || (hcost[o] == ci && o < i)) ? 1 : 0;
    hsorted[rank] = i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    long long load[kParts];
    int cnt[kParts];
    for (int p = 0; p < kParts; ++p) load[p] = 0, cnt[p] = 0;
    int mine = 0, pos = 0;
    for (int k = 0; k < H; ++k) {
      const int hh = hsorted[k];
      int p = 0;
      for (int i = 1; i < kParts; ++i)
        if (load[i] < load[p]) p = i;
      if (hh == h) mine = p, pos = cnt[p];
      load[p] += hcost[hh];
      cnt[p] += 1;
    }
    int off = 0;
    for (int p = 0; p < kParts; ++p) {
      s_off[p] = off;
      off += cnt[p] * nqb;
    }
    s_off[kParts] = off;
    s_start = s_off[mine] + pos * nqb;
  }
  const int r0 = h * nqb;
  for (int qb = threadIdx.x; qb < nqb; qb += kRowThreads) cost[qb] = row_ptr[r0 + qb + 1] - row_ptr[r0 + qb];
  __syncthreads();
  for (int qb = threadIdx.x; qb < nqb; qb += kRowThreads) {
    const int cq = cost[qb];
    int rank = 0;
    for (int o = 0; o < nqb; ++o) {
      const int co = cost[o];
      rank += (co > cq || (co == cq && o < qb)) ? 1 : 0;
    }
    out[s_start + rank] = r0 + qb;
  }
  if (h == 0 && threadIdx.x <= kParts) out[rows + threadIdx.x] = s_off[threadIdx.x];
}

hipError_t launch_compile_count(const CompileArgs& a, hipStream_t st) {
  const int rows = a.H * a.nqb;
  if (a.energy)
    hipLaunchKernelGGL(keep_energy_kernel, dim3(rows), dim3(kRowThreads), 0, st, a.mass, a.P, rows, a.nkb,
                       a.nkb_valid, a.eps_num, a.eps_den, a.min_agree, a.keep_ws, a.count_ws);
  else
    hipLaunchKernelGGL(keep_agree_kernel, dim3(rows), dim3(kRowThreads), 0, st, a.mass, a.P, rows,
                       a.nkb, a.nkb_valid, a.keep_topk, a.min_agree, a.keep_ws, a.count_ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(row_offsets_kernel, dim3(1), dim3(kScanThreads), 0, st, (const int32_t*)a.count_ws,
                     rows, a.row_ptr);
  return hipGetLastError();
}

hipError_t launch_row_offsets(const int32_t* counts, int n, int32_t* offsets, hipStream_t st) {
  hipLaunchKernelGGL(row_offsets_kernel, dim3(1), dim3(kScanThreads), 0, st, counts, n, offsets);
  return hipGetLastError();
}

hipError_t launch_compile_fill(const CompileArgs& a, hipStream_t st) {
  const int rows = a.H * a.nqb;
  hipLaunchKernelGGL(fill_columns_kernel, dim3(rows), dim3(kRowThreads), 0, st,
                     (const uint8_t*)a.keep_ws, a.nkb, (const int32_t*)a.row_ptr, a.col_idx);
  return hipGetLastError();
}

hipError_t launch_schedule(const int32_t* row_ptr, int H, int nqb, int32_t* work_order,
                           hipStream_t st) {
  hipLaunchKernelGGL(lpt_schedule_kernel, dim3(H), dim3(kRowThreads), 0, st, row_ptr, H, nqb, work_order);
  return hipGetLastError();
}

}  // namespace calibatt
