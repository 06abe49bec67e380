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
// Scheduling: with a queue pointer the grid is persistent; each workgroup
// pops rows from the atomic counter of its XCD's partition of the work order
// (heads spread over partitions, rows longest first), then helps the other
// partitions.  Keeping a head's rows on one XCD keeps its K/V in that XCD's
// L2; longest-first puts the short rows at the tail of the launch.
#include "tiles.h"
#include "launch.h"

namespace calibatt {

// Pipeline geometry of the bf16 kernel.  Keys are consumed in sub-tiles of
// 64 (a 128-token kept block is two sub-tiles).  Two LDS buffers each hold a
// K sub-tile (rows of 16-byte chunks, XOR-swizzled) and a transposed V
// sub-tile.  While sub-tile j is computed from one buffer, sub-tile j+1 is in
// flight: K goes straight from HBM into the other buffer by buffer-to-LDS
// DMA (no registers), V comes into registers in 8-key x 4-d blocks (8 loads
// of 8 bytes per thread) and is transposed with byte permutes and written
// after the compute of sub-tile j.
template <int D, int BLK>
struct Pipe {
  static constexpr int NT = BLK * 2;        // threads: BLK/32 waves of 64
  static constexpr int NW = BLK / 32;
  static constexpr int BN = 64;             // keys per sub-tile
  static constexpr int SPB = BLK / BN;      // sub-tiles per kept block
  static constexpr int CH = D / 8;          // 16-byte chunks per K row
  static constexpr int CHV = BN / 8;        // 16-byte chunks per Vt row
  static constexpr int KROWS_PER_LOAD = 64 / CH;            // rows one wave DMA covers
  static constexpr int KLOADS = BN / KROWS_PER_LOAD / NW;   // DMA instructions per wave
  static constexpr int DQ = D / 4;          // 4-wide d groups
  static constexpr int VBLK = (BN / 8) * DQ;                // 8x4 V blocks per sub-tile
  static constexpr int VPER = (VBLK + NT - 1) / NT;
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Per-lane byte offsets of the K DMA (one per DMA instruction), relative to the sub-tile start.
template <int D, int BLK>
__device__ __forceinline__ void k_dma_offsets(int w, int lane, int* koff) {
  using P = Pipe<D, BLK>;
#pragma unroll
  for (int i = 0; i < P::KLOADS; ++i) {
    const int row = (w * P::KLOADS + i) * P::KROWS_PER_LOAD + lane / P::CH;
    const int chunk = (lane % P::CH) ^ swz<P::CH>(row);
    koff[i] = (row * D + chunk * 8) * 2;
  }
}

// K sub-tile starting at key k0 -> swizzled LDS buffer, by DMA.
template <int D, int BLK>
__device__ __forceinline__ void k_dma(__amdgpu_buffer_rsrc_t rk, int k0, u32x4* ldsK, int w, const int* koff) {
  using P = Pipe<D, BLK>;
#pragma unroll
  for (int i = 0; i < P::KLOADS; ++i) {
    const int r0 = (w * P::KLOADS + i) * P::KROWS_PER_LOAD;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(ldsK + r0 * P::CH), 16, koff[i], k0 * D * 2, 0, 0);
  }
}

template <int D, int BLK>
__device__ __forceinline__ void v_load(__amdgpu_buffer_rsrc_t rv, int k0, int voff, u32x2* st) {
  using P = Pipe<D, BLK>;
#pragma unroll
  for (int j = 0; j < P::VPER; ++j) {
    const int vb = threadIdx.x + j * P::NT;
    if (P::VBLK % P::NT == 0 || vb < P::VBLK) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        st[8 * j + i] = __builtin_amdgcn_raw_buffer_load_b64(
            rv, voff + j * (P::NT / P::DQ) * 8 * D * 2 + i * D * 2, k0 * D * 2, 0);
    }
  }
}

template <int D, int BLK>
__device__ __forceinline__ void v_store(const u32x2* st, u32x4* ldsV) {
  using P = Pipe<D, BLK>;
#pragma unroll
  for (int j = 0; j < P::VPER; ++j) {
    const int vb = threadIdx.x + j * P::NT;
    if (P::VBLK % P::NT == 0 || vb < P::VBLK) {
      const int dq = vb % P::DQ, kg = vb / P::DQ;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t x = st[8 * j + 2 * q][e >> 1], y = st[8 * j + 2 * q + 1][e >> 1];
          o[q] = __builtin_amdgcn_perm(y, x, (e & 1) ? 0x07060302u : 0x05040100u);
        }
        ldsV[chunk_index<P::CHV>(dq * 4 + e, kg)] = o;
      }
    }
  }
}

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Where a workgroup's next row comes from.  With a work order, rows are
// grouped into kParts partition lists (offsets after the rows); without one,
// partition p holds heads p, p + kParts, ... in natural order.
struct RowSource {
  const int32_t* order;
  int rows, nqb, H, B;
  __device__ __forceinline__ int part_len(int p) const {
    if (order) return order[rows + p + 1] - order[rows + p];
    return ((H - p + kParts - 1) / kParts) * nqb;
  }
  __device__ __forceinline__ int part_row(int p, int k) const {
    if (order) return order[order[rows + p] + k];
    return (p + kParts * (k / nqb)) * nqb + k % nqb;
  }
};

// Persistent scheduling: serve partition blockIdx.x % kParts (the XCD this
// workgroup runs on) until its counter passes its length, then move to the
// next partition; every workgroup visits every partition once, so the grid
// always drains.  Without a queue, workgroup i takes row i of the order.
template <typename Body>
__device__ __forceinline__ void for_each_row(const RowSource& src, int32_t* queue, int* s_item, Body body) {
  if (queue) {
    int p = blockIdx.x % kParts;
    for (int tries = 0; tries < kParts;) {
      if (threadIdx.x == 0) *s_item = atomicAdd(queue + p * kQueueStride, 1);
      __syncthreads();
      const int k = *s_item;
      __syncthreads();
      const int len = src.part_len(p);
      if (k >= src.B * len) {
        p = (p + 1) % kParts;
        ++tries;
        continue;
      }
      const int b = k / len;
      body(b, src.part_row(p, k - b * len));
    }
  } else {
    const int item = blockIdx.x;
    const int b = item / src.rows, j = item - b * src.rows;
    body(b, src.order ? src.order[j] : j);
  }
}

constexpr float kLazyLog2 = 8.f;

template <int I>
struct Buf {
  static constexpr int value = I;
};

template <int D, int BLK, bool DENSE>
__global__ __launch_bounds__(BLK * 2, 2) void attn_fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const int32_t* __restrict__ work_order, int32_t* __restrict__ queue, int items, int H, int L,
    int seq_len, int nkb_valid, float c2) {
  using P = Pipe<D, BLK>;
  constexpr int DS = D / 16;     // k-steps of Q K^T
  constexpr int DT = D / 32;     // 32-row d tiles of O^T
  // two buffers as separate LDS objects, so loads into one never alias reads of the other
  __shared__ u32x4 ldsK0[P::BN * P::CH];
  __shared__ u32x4 ldsK1[P::BN * P::CH];
  __shared__ u32x4 ldsV0[D * P::CHV];
  __shared__ u32x4 ldsV1[D * P::CHV];
  __shared__ int s_item;

  const int nqb = L / BLK;
  const int rows = H * nqb;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 5, c = lane & 31;
  const int prow = qk_row_perm(c);
  const uint32_t slab_bytes = (uint32_t)L * D * 2;
  const float lazy_thr = kLazyLog2 / c2;   // in raw score units

  int koff[P::KLOADS];
  k_dma_offsets<D, BLK>(w, lane, koff);
  const int voff = (((threadIdx.x / P::DQ) * 8) * D + (threadIdx.x % P::DQ) * 4) * 2;

  const RowSource src{work_order, rows, nqb, H, items / rows};
  for_each_row(src, queue, &s_item, [&](int b, int r) {
    const int h = r / nqb, qb = r - h * nqb;
    const size_t base = ((size_t)b * H + h) * (size_t)L * D;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + base, slab_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + base, slab_bytes);
    const int q = qb * BLK + 32 * w + c;   // this lane's query

    bf16x8 qreg[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qreg[s] = *reinterpret_cast<const bf16x8*>(Q + base + (size_t)q * D + 16 * s + 8 * g);

    f32x16 oacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
    float m_run = kNegInf, l_run = 0.f;

    const int beg = DENSE ? 0 : row_ptr[r];
    const int nsub = ((DENSE ? nkb_valid : row_ptr[r + 1]) - beg) * P::SPB;
    auto key0 = [&](int j) -> int {
      const int kb = DENSE ? j / P::SPB : col_idx[beg + j / P::SPB];
      return kb * BLK + (j % P::SPB) * P::BN;
    };

    u32x2 st[8 * P::VPER];
    if (nsub > 0) {
      const int k0 = key0(0);
      k_dma<D, BLK>(rk, k0, ldsK0, w, koff);
      v_load<D, BLK>(rv, k0, voff, st);
      v_store<D, BLK>(st, ldsV0);
    }
    wait_vm();
    __syncthreads();

    // one sub-tile: compute from buffer B while sub-tile j+1 streams into buffer 1-B
    auto step = [&](int j, auto bufc) {
      constexpr int B = decltype(bufc)::value;
      u32x4* const kcur = B == 0 ? ldsK0 : ldsK1;
      u32x4* const vcur = B == 0 ? ldsV0 : ldsV1;
      u32x4* const knext = B == 0 ? ldsK1 : ldsK0;
      u32x4* const vnext = B == 0 ? ldsV1 : ldsV0;
      const int k0 = key0(j);
      const bool more = j + 1 < nsub;
      if (more) {
        const int k1 = key0(j + 1);
        k_dma<D, BLK>(rk, k1, knext, w, koff);
        v_load<D, BLK>(rv, k1, voff, st);
      }

      // S^T for 64 keys x 32 queries: two 32x32 accumulators
      f32x16 sacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int row = 32 * mt + prow;
        u32x4 a[DS];
#pragma unroll
        for (int s = 0; s < DS; ++s) a[s] = kcur[chunk_index<P::CH>(row, 2 * s + g)];
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < DS; ++s) acc = mfma_bf16(__builtin_bit_cast(bf16x8, a[s]), qreg[s], acc);
        sacc[mt] = acc;
      }
      if (k0 + P::BN > seq_len) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            if (k0 + 32 * mt + slice_key(rr, g) >= seq_len) sacc[mt][rr] = kNegInf;
      }

      float mx = kNegInf;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, sacc[mt][rr]);
      mx = pair_max(mx);
      // Lazy rescale: the reference maximum moves only when a score passes it
      // by more than kLazyLog2 in log2 units, so probabilities stay below
      // 2^kLazyLog2 and O and l are rescaled a few times per row instead of
      // on most sub-tiles.  O = acc / l is the same for any reference.
      if (__any(mx > m_run + lazy_thr)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2((m_run - m_new) * c2);
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
        m_run = m_new;
      }
      const float mc = (m_run == kNegInf ? 0.f : m_run) * c2;

      bf16x8 pb[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (bf16)fast_exp2(fmaf(sacc[ks >> 1][8 * (ks & 1) + e], c2, -mc));
        pb[ks] = v;
      }
      // row sum of the rounded probabilities, the same values the P*V product uses
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      const bf16x2 one2 = {(bf16)1.f, (bf16)1.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pr = {pb[ks][e], pb[ks][e + 1]};
          l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, l_run, false);
        }

#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const int row = 32 * t + c;
        u32x4 a[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) a[ks] = vcur[chunk_index<P::CHV>(row, 2 * ks + g)];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) oacc[t] = mfma_bf16(__builtin_bit_cast(bf16x8, a[ks]), pb[ks], oacc[t]);
      }
      if (more) v_store<D, BLK>(st, vnext);
      wait_vm();
      __syncthreads();
    };

    for (int j = 0; j < nsub; j += 2) {
      step(j, Buf<0>{});
      if (j + 1 < nsub) step(j + 1, Buf<1>{});
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
  });
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

  const RowSource src{work_order, rows, nqb, H, items / rows};
  for_each_row(src, queue, &s_item, [&](int b, int r) {
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
  });
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
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(kQueueInts), 0, st, a.queue, kQueueInts, 0);
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
