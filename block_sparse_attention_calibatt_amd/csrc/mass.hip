// Calibration pooling for gfx950: post-softmax attention mass per
// (query block, key block), over the full (dense) map of one prompt.
//
// The pages pool post-softmax maps to block level (Fig. 2 caption) and call
// the pooled values block energies (Table S5 caption).  With the softmax over
// all valid keys, tile (qb, kb) receives sum_{i in qb} sum_{j in kb} p_ij.
//
// Pass 1 (row_lse_kernel): per query, log-sum-exp of scale*q.k over the
// valid keys, by the same online max/sum as the attention forward (no P*V).
// Pass 2 (block_pool_kernel): recompute S per key block on the matrix cores,
// p = exp(s - lse) in float32, sum each wave's 32x BLK sub-tile with a fixed
// butterfly, keep one partial per wave per key block in LDS, and add the
// partials of the block's waves in wave order at the end.  The reduction
// order is fixed, so the mass is bitwise reproducible.
//
// Single pass (row_lse_kernel<.., true> + mass_from_partials_kernel): pass 1
// also stores, per (key block, query), the block's log2 partial
// lp = log2 sum_{j in kb} exp2(c s_ij), i.e. the reference plus the log of
// the tile's sum against it, so a later move of the lazy reference does not
// touch it.  The mass is then sum_{i in qb} exp2(lp_i,kb - lse2_i): one score
// product and one exp per (query, key) instead of two, for a [B, H, nkb, L]
// float32 workspace.
#include "tiles.h"
#include "launch.h"

namespace calibatt {

// Pass 1 keeps its reference until a tile's per-lane sum passes this bound
// (or is not finite); the row sum stays far inside float32's range.
constexpr float kLseCap = 1048576.f;

template <int D, int BLK, bool PARTIALS = false>
__global__ __launch_bounds__(BLK * 2) void row_lse_kernel(const bf16* __restrict__ Q,
                                                          const bf16* __restrict__ K,
                                                          float* __restrict__ lse, int H, int L,
                                                          int seq_len, int nkb_valid, float c2,
                                                          float* __restrict__ lpart = nullptr) {
  constexpr int KT = BLK / 32;
  constexpr int DS = D / 16;
  __shared__ u32x4 ldsK[BLK * D / 8];
  const int nqb = L / BLK;
  const int item = blockIdx.x;
  const int bh = item / nqb, qb = item - bh * nqb;
  const size_t base = (size_t)bh * L * D;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 5, c = lane & 31;
  const int q = qb * BLK + 32 * w + c;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + base, (uint32_t)L * D * 2);

  bf16x8 qreg[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s)
    qreg[s] = *reinterpret_cast<const bf16x8*>(Q + base + (size_t)q * D + 16 * s + 8 * g);

  // m_run: the reference (raw score units), valid once `fresh` is false
  float m_run = 0.f, l_run = 0.f;
  bool fresh = true;
  for (int kb = 0; kb < nkb_valid; ++kb) {
    __syncthreads();
    dma_k_tile<D, BLK>(rk, kb * BLK, ldsK, wu, lane);
    wait_vm_all();
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
    // lazy reference (scaled units): set from the first tile's maximum and
    // moved to the running maximum only when a tile's sum passes kLseCap or
    // is not finite, so most tiles need no maximum
    auto tile_sum = [&](float mc) __attribute__((always_inline)) {
      float ps = 0.f;
#pragma unroll
      for (int mt = 0; mt < KT; ++mt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) ps += fast_exp2(fmaf(sacc[mt][rr], c2, -mc));
      return ps;
    };
    float psum = fresh ? 0.f : tile_sum(m_run * c2);
    if (__any(fresh || !(psum <= kLseCap))) {
      float mx = kNegInf;
#pragma unroll
      for (int mt = 0; mt < KT; ++mt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, sacc[mt][rr]);
      mx = pair_max(mx);
      const float m_new = fresh ? mx : fmaxf(m_run, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      l_run *= fresh ? 0.f : fast_exp2((m_run - m_use) * c2);
      m_run = m_use;
      fresh = m_new == kNegInf;
      psum = tile_sum(m_run * c2);
    }
    l_run += psum;
    if constexpr (PARTIALS) {
      // the block's log2 partial for this query: [bh][kb][q], coalesced over q
      const float tot = pair_sum(psum);
      if (g == 0) lpart[((size_t)bh * nqb + kb) * L + q] = fresh ? kNegInf : m_run * c2 + __log2f(tot);
    }
  }
  const float l_tot = pair_sum(l_run);
  if (g == 0) {
    float v = kNegInf;
    if (q < seq_len && l_tot > 0.f) v = (m_run * c2 + __log2f(l_tot)) * kLn2;
    lse[(size_t)bh * L + q] = v;
  }
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void block_pool_kernel(const bf16* __restrict__ Q,
                                                             const bf16* __restrict__ K,
                                                             const float* __restrict__ lse,
                                                             float* __restrict__ mass, int H, int L,
                                                             int seq_len, int nkb_valid, float c2) {
  constexpr int NT = BLK * 2;
  constexpr int NW = BLK / 32;
  constexpr int KT = BLK / 32;
  constexpr int DS = D / 16;
  __shared__ u32x4 ldsK[BLK * D / 8];
  __shared__ float part[NW][kMaxKeyBlocks];
  const int nqb = L / BLK;
  const int nkb = nqb;
  const int item = blockIdx.x;
  const int bh = item / nqb, qb = item - bh * nqb;
  const size_t base = (size_t)bh * L * D;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 5, c = lane & 31;
  const int q = qb * BLK + 32 * w + c;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + base, (uint32_t)L * D * 2);
  const bool qvalid = q < seq_len;
  const float lse2 = qvalid ? lse[(size_t)bh * L + q] * kLog2e : 0.f;

  bf16x8 qreg[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s)
    qreg[s] = *reinterpret_cast<const bf16x8*>(Q + base + (size_t)q * D + 16 * s + 8 * g);

  for (int kb = 0; kb < nkb_valid; ++kb) {
    __syncthreads();
    dma_k_tile<D, BLK>(rk, kb * BLK, ldsK, wu, lane);
    wait_vm_all();
    __syncthreads();
    f32x16 sacc[KT];
    qk_tile<D, BLK>(ldsK, qreg, sacc, g, c);
    const int k0 = kb * BLK;
    float psum = 0.f;
    if (qvalid) {
      if (k0 + BLK > seq_len) {   // the tile holding the padded keys
#pragma unroll
        for (int mt = 0; mt < KT; ++mt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const bool kvalid = k0 + 32 * mt + slice_key(rr, g) < seq_len;
            psum += kvalid ? fast_exp2(fmaf(sacc[mt][rr], c2, -lse2)) : 0.f;
          }
      } else {
#pragma unroll
        for (int mt = 0; mt < KT; ++mt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) psum += fast_exp2(fmaf(sacc[mt][rr], c2, -lse2));
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) psum += __shfl_xor(psum, off);
    if (lane == 0) part[w][kb] = psum;
  }
  __syncthreads();
  float* out = mass + ((size_t)bh * nqb + qb) * nkb;
  for (int kb = threadIdx.x; kb < nkb; kb += NT) {
    float s = 0.f;
    if (kb < nkb_valid) {
#pragma unroll
      for (int i = 0; i < NW; ++i) s += part[i][kb];
    }
    out[kb] = s;
  }
}

// mass[bh, qb, kb] = sum over the block's valid queries of exp2(lp - lse2),
// for every key block: threads 0..BLK-1 take the queries of one key block,
// the rest those of the next; sums by a fixed butterfly, then in wave order.
template <int BLK>
__global__ __launch_bounds__(256) void mass_from_partials_kernel(const float* __restrict__ lpart,
                                                                 const float* __restrict__ lse,
                                                                 float* __restrict__ mass, int L, int seq_len,
                                                                 int nkb_valid) {
  constexpr int PER = 256 / BLK;   // key blocks per step
  constexpr int WPB = BLK / 64;    // waves per key block
  __shared__ float part[4];
  const int nqb = L / BLK;
  const int nkb = nqb;
  const int item = blockIdx.x;
  const int bh = item / nqb, qb = item - bh * nqb;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int sub = threadIdx.x / BLK, t = threadIdx.x % BLK;
  const int q = qb * BLK + t;
  const bool qvalid = q < seq_len;
  const float lse2 = qvalid ? lse[(size_t)bh * L + q] * kLog2e : 0.f;
  float* out = mass + ((size_t)bh * nqb + qb) * nkb;
  for (int kb0 = 0; kb0 < nkb; kb0 += PER) {
    const int kb = kb0 + sub;
    float v = 0.f;
    if (qvalid && kb < nkb_valid) v = fast_exp2(lpart[((size_t)bh * nqb + kb) * L + q] - lse2);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    __syncthreads();
    if (lane == 0) part[w] = v;
    __syncthreads();
    if (t == 0 && kb < nkb) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < WPB; ++i) s += part[sub * WPB + i];
      out[kb] = s;
    }
  }
}

template <int D, int BLK>
static hipError_t launch_mass_single_typed(const MassArgs& a, float* lpart, hipStream_t st) {
  const int items = a.B * a.H * (a.L / BLK);
  const float c2 = a.scale * kLog2e;
  hipLaunchKernelGGL((row_lse_kernel<D, BLK, true>), dim3(items), dim3(BLK * 2), 0, st, (const bf16*)a.Q,
                     (const bf16*)a.K, a.lse, a.H, a.L, a.seq_len, a.nkb_valid, c2, lpart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((mass_from_partials_kernel<BLK>), dim3(items), dim3(256), 0, st, (const float*)lpart,
                     (const float*)a.lse, a.mass, a.L, a.seq_len, a.nkb_valid);
  return hipGetLastError();
}

hipError_t launch_block_mass_single(const MassArgs& a, float* lpart, hipStream_t st) {
  if (a.d == 128 && a.block == 128) return launch_mass_single_typed<128, 128>(a, lpart, st);
  if (a.d == 128 && a.block == 64) return launch_mass_single_typed<128, 64>(a, lpart, st);
  if (a.d == 64 && a.block == 128) return launch_mass_single_typed<64, 128>(a, lpart, st);
  return launch_mass_single_typed<64, 64>(a, lpart, st);
}

template <int D, int BLK>
static hipError_t launch_mass_typed(const MassArgs& a, hipStream_t st) {
  const int items = a.B * a.H * (a.L / BLK);
  const float c2 = a.scale * kLog2e;
  hipLaunchKernelGGL((row_lse_kernel<D, BLK>), dim3(items), dim3(BLK * 2), 0, st, (const bf16*)a.Q,
                     (const bf16*)a.K, a.lse, a.H, a.L, a.seq_len, a.nkb_valid, c2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((block_pool_kernel<D, BLK>), dim3(items), dim3(BLK * 2), 0, st,
                     (const bf16*)a.Q, (const bf16*)a.K, (const float*)a.lse, a.mass, a.H, a.L,
                     a.seq_len, a.nkb_valid, c2);
  return hipGetLastError();
}

hipError_t launch_row_lse(const MassArgs& a, hipStream_t st) {
  const int items = a.B * a.H * (a.L / 128);
  const float c2 = a.scale * kLog2e;
  if (a.d == 128)
    hipLaunchKernelGGL((row_lse_kernel<128, 128>), dim3(items), dim3(256), 0, st, (const bf16*)a.Q,
                       (const bf16*)a.K, a.lse, a.H, a.L, a.seq_len, a.nkb_valid, c2);
  else
    hipLaunchKernelGGL((row_lse_kernel<64, 128>), dim3(items), dim3(256), 0, st, (const bf16*)a.Q,
                       (const bf16*)a.K, a.lse, a.H, a.L, a.seq_len, a.nkb_valid, c2);
  return hipGetLastError();
}

hipError_t launch_block_mass(const MassArgs& a, hipStream_t st) {
  if (a.d == 128 && a.block == 128) return launch_mass_typed<128, 128>(a, st);
  if (a.d == 128 && a.block == 64) return launch_mass_typed<128, 64>(a, st);
  if (a.d == 64 && a.block == 128) return launch_mass_typed<64, 128>(a, st);
  return launch_mass_typed<64, 64>(a, st);
}

}  // namespace calibatt
