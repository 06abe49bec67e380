// Block-sparse (and dense) flash-style attention forward for gfx950.
//
// Computes, per batch entry b, head h and query block qb (row r = h*nqb+qb),
// attention of the block's queries over the valid keys of the row's kept key
// blocks only; skipped blocks are absent from the softmax (CalibAtt abstract;
// Fig. 5(b) caption).  The dense kernel is the same code with every valid key
// block kept.
//
// bf16 kernel: one workgroup per query block of BLK tokens, BLK/32 waves,
// each wave owning 32 queries.  Per kept key block: K tile -> LDS, V tile ->
// transposed LDS, S^T = K Q^T on the matrix cores (Q held in registers),
// online softmax in float32 with exp2 and the scale folded into one FMA,
// P rounded to bf16, O^T += V^T P^T on the matrix cores.  The key blocks of a
// row are reduced in col_idx order by that one workgroup, so the result does
// not depend on the order rows are scheduled in.
//
// Scheduling: with a queue pointer the grid is persistent and workgroups pop
// row indices from an atomic counter; the optional work_order permutes rows
// (longest first) so the tail of the launch holds the short rows.
#include "tiles.h"
#include "launch.h"

namespace calibatt {

template <int D, int BLK, bool DENSE>
__global__ __launch_bounds__(BLK * 2) void attn_fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const int32_t* __restrict__ work_order, int32_t* __restrict__ queue, int items, int H, int L,
    int seq_len, int nkb_valid, float c2) {
  constexpr int NT = BLK * 2;
  constexpr int KT = BLK / 32;   // 32-key slices per block
  constexpr int DS = D / 16;     // k-steps of Q K^T
  constexpr int DT = D / 32;     // 32-row d tiles of O^T
  constexpr int CH = D / 8;      // 16-byte chunks per K row
  constexpr int CHV = BLK / 8;   // 16-byte chunks per Vt row
  __shared__ u32x4 ldsK[BLK * CH];
  __shared__ u32x4 ldsV[D * CHV];
  __shared__ int s_item;

  const int nqb = L / BLK;
  const int rows = H * nqb;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 5, c = lane & 31;

  int item = blockIdx.x;
  for (;;) {
    if (queue) {
      if (threadIdx.x == 0) s_item = atomicAdd(queue, 1);
      __syncthreads();
      item = s_item;
      __syncthreads();
    }
    if (item >= items) break;
    const int b = item / rows, ri = item - b * rows;
    const int r = work_order ? work_order[ri] : ri;
    const int h = r / nqb, qb = r - h * nqb;
    const size_t base = ((size_t)b * H + h) * (size_t)L * D;
    const bf16* Qb = Q + base;
    const bf16* Kb = K + base;
    const bf16* Vb = V + base;
    const int q = qb * BLK + 32 * w + c;   // this lane's query

    bf16x8 qreg[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qreg[s] = *reinterpret_cast<const bf16x8*>(Qb + (size_t)q * D + 16 * s + 8 * g);

    f32x16 oacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
    float m_run = kNegInf, l_run = 0.f;

    const int beg = DENSE ? 0 : row_ptr[r];
    const int end = DENSE ? nkb_valid : row_ptr[r + 1];
    for (int it = beg; it < end; ++it) {
      const int kb = DENSE ? it : col_idx[it];
      const size_t koff = (size_t)kb * BLK * D;
      __syncthreads();
      load_k_tile<D, BLK, NT>(Kb + koff, ldsK);
      load_v_tile_t<D, BLK, NT>(Vb + koff, ldsV);
      __syncthreads();

      f32x16 sacc[KT];
      qk_tile<D, BLK>(ldsK, qreg, sacc, g, c);

      const int k0 = kb * BLK;
      if (k0 + BLK > seq_len) {
#pragma unroll
        for (int mt = 0; mt < KT; ++mt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            if (k0 + 32 * mt + slice_key(rr, g) >= seq_len) sacc[mt][rr] = kNegInf;
      }

      float mx = kNegInf;
#pragma unroll
      for (int mt = 0; mt < KT; ++mt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, sacc[mt][rr]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2((m_run - m_use) * c2);
      const float mc = m_use * c2;
      m_run = m_new;

      float psum = 0.f;
      bf16x8 pb[BLK / 16];
#pragma unroll
      for (int mt = 0; mt < KT; ++mt) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = fast_exp2(fmaf(sacc[mt][8 * half + e], c2, -mc));
            psum += p;
            v[e] = (bf16)p;
          }
          pb[2 * mt + half] = v;
        }
      }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int t = 0; t < DT; ++t) oacc[t] *= alpha;

#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const int row = 32 * t + c;
#pragma unroll
        for (int ks = 0; ks < BLK / 16; ++ks) {
          const u32x4 a = ldsV[chunk_index<CHV>(row, 2 * ks + g)];
          oacc[t] = mfma_bf16(__builtin_bit_cast(bf16x8, a), pb[ks], oacc[t]);
        }
      }
    }

    const float l_tot = pair_sum(l_run);
    const float inv = (q < seq_len && l_tot > 0.f) ? 1.f / l_tot : 0.f;
    bf16* Ob = O + base + (size_t)q * D;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * t + 8 * rq + 4 * g;
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (bf16)(oacc[t][4 * rq + e] * inv);
        *reinterpret_cast<bf16x4*>(Ob + d0) = o;
      }
    }
    if (!queue) break;
  }
}

// float32 path: 32-key slices, fp32 matrix cores (32x32x2), P kept in float32.
// Lane (g, c) holds, for slice accumulator register r, key 2r + g (rows of
// the K slice are fed in that order), which is the B layout of P^T.
template <int D, int BLK, bool DENSE>
__global__ __launch_bounds__(BLK * 2) void attn_fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const int32_t* __restrict__ work_order, int32_t* __restrict__ queue, int items, int H, int L,
    int seq_len, int nkb_valid, float c2) {
  constexpr int NT = BLK * 2;
  constexpr int KP = D + 1;   // padded K row (floats)
  constexpr int DT = D / 32;
  __shared__ float ldsK[32 * KP];
  __shared__ float ldsV[32 * D];
  __shared__ int s_item;

  const int nqb = L / BLK;
  const int rows = H * nqb;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 5, c = lane & 31;
  // slice row fed by lane column c: key 2*(i without bit 2) + bit 2
  const int krow = ((c >> 3) << 3) | ((c & 3) << 1) | ((c >> 2) & 1);

  int item = blockIdx.x;
  for (;;) {
    if (queue) {
      if (threadIdx.x == 0) s_item = atomicAdd(queue, 1);
      __syncthreads();
      item = s_item;
      __syncthreads();
    }
    if (item >= items) break;
    const int b = item / rows, ri = item - b * rows;
    const int r = work_order ? work_order[ri] : ri;
    const int h = r / nqb, qb = r - h * nqb;
    const size_t base = ((size_t)b * H + h) * (size_t)L * D;
    const int q = qb * BLK + 32 * w + c;

    float qreg[D / 2];
#pragma unroll
    for (int s = 0; s < D / 2; ++s) qreg[s] = Q[base + (size_t)q * D + 2 * s + g];

    f32x16 oacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
    float m_run = kNegInf, l_run = 0.f;

    const int beg = DENSE ? 0 : row_ptr[r];
    const int end = DENSE ? nkb_valid : row_ptr[r + 1];
    for (int it = beg; it < end; ++it) {
      const int kb = DENSE ? it : col_idx[it];
      for (int sl = 0; sl < BLK / 32; ++sl) {
        const int k0 = kb * BLK + 32 * sl;
        __syncthreads();
        for (int i = threadIdx.x; i < 32 * D; i += NT) {
          const int kr = i / D, dd = i % D;
          ldsK[kr * KP + dd] = K[base + (size_t)(k0 + kr) * D + dd];
          ldsV[kr * D + dd] = V[base + (size_t)(k0 + kr) * D + dd];
        }
        __syncthreads();
        f32x16 sacc = {};
#pragma unroll
        for (int s = 0; s < D / 2; ++s)
          sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(ldsK[krow * KP + 2 * s + g], qreg[s], sacc, 0, 0, 0);
        if (k0 + 32 > seq_len) {
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            if (k0 + 2 * rr + g >= seq_len) sacc[rr] = kNegInf;
        }
        float mx = kNegInf;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, sacc[rr]);
        mx = pair_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = fast_exp2((m_run - m_use) * c2);
        const float mc = m_use * c2;
        m_run = m_new;
        float psum = 0.f;
        float p[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          p[rr] = fast_exp2(fmaf(sacc[rr], c2, -mc));
          psum += p[rr];
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          oacc[t] *= alpha;
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            oacc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(ldsV[(2 * rr + g) * D + 32 * t + c], p[rr],
                                                           oacc[t], 0, 0, 0);
        }
      }
    }
    const float l_tot = pair_sum(l_run);
    const float inv = (q < seq_len && l_tot > 0.f) ? 1.f / l_tot : 0.f;
    float* Ob = O + base + (size_t)q * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) Ob[32 * t + 8 * (rr >> 2) + 4 * g + (rr & 3)] = oacc[t][rr] * inv;
    if (!queue) break;
  }
}

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

template <typename Kern>
static hipError_t occupancy(Kern k, int threads, int* blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, k, threads, 0);
}

template <int D, int BLK, bool DENSE>
static hipError_t launch_typed(const AttnArgs& a, hipStream_t st) {
  const int threads = BLK * 2;
  const int items = a.B * a.H * (a.L / BLK);
  const float c2 = a.scale * kLog2e;
  if (items == 0) return hipSuccess;
  int grid = items;
  if (a.queue) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(64), 0, st, a.queue, 16, 0);
    int per_cu = 1;
    hipError_t e = a.dtype_f32
        ? occupancy(attn_fwd_f32_kernel<D, BLK, DENSE>, threads, &per_cu)
        : occupancy(attn_fwd_bf16_kernel<D, BLK, DENSE>, threads, &per_cu);
    if (e != hipSuccess) return e;
    const long long cap = (long long)a.num_cu * (per_cu > 0 ? per_cu : 1);
    grid = (int)(cap < items ? cap : items);
  }
  if (a.dtype_f32) {
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D, BLK, DENSE>), dim3(grid), dim3(threads), 0, st,
                       (const float*)a.Q, (const float*)a.K, (const float*)a.V, (float*)a.O,
                       a.row_ptr, a.col_idx, a.work_order, a.queue, items, a.H, a.L, a.seq_len,
                       a.nkb_valid, c2);
  } else {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, BLK, DENSE>), dim3(grid), dim3(threads), 0, st,
                       (const bf16*)a.Q, (const bf16*)a.K, (const bf16*)a.V, (bf16*)a.O, a.row_ptr,
                       a.col_idx, a.work_order, a.queue, items, a.H, a.L, a.seq_len, a.nkb_valid, c2);
  }
  return hipGetLastError();
}

template <bool DENSE>
static hipError_t dispatch(const AttnArgs& a, hipStream_t st) {
  if (a.d == 128 && a.block == 128) return launch_typed<128, 128, DENSE>(a, st);
  if (a.d == 128 && a.block == 64) return launch_typed<128, 64, DENSE>(a, st);
  if (a.d == 64 && a.block == 128) return launch_typed<64, 128, DENSE>(a, st);
  return launch_typed<64, 64, DENSE>(a, st);
}

hipError_t launch_attention(const AttnArgs& a, bool dense, hipStream_t st) {
  return dense ? dispatch<true>(a, st) : dispatch<false>(a, st);
}

}  // namespace calibatt
