// Block-sparse (and dense) flash-style attention forward for gfx950.
//
// Computes, per batch entry b, head h and query block qb (row r = h*nqb+qb),
// attention of the block's queries over the valid keys of the row's kept key
// blocks only; skipped blocks are absent from the softmax (CalibAtt abstract;
// Fig. 5(b) caption).  The dense kernel is the same code with every valid key
// block kept.
//
// V is read transposed, as V^T [B, H, d, L]: the P*V product contracts over
// keys, and the matrix cores want the contracted index contiguous in each
// lane's operand, so a V^T tile can go from HBM to LDS by DMA unchanged.
// transpose_v_kernel makes V^T from V [B, H, L, d] when the caller has only
// the latter (one HBM-bound pass over V).
//
// bf16 kernel: one workgroup per query block of BLK tokens, BLK/32 waves of
// 32 queries each, two workgroups per CU.  Per 64-key sub-tile of a kept key
// block: K tile and V^T tile -> LDS by DMA (the next sub-tile's DMA runs
// while this one is computed), S^T = K Q^T on the matrix cores (Q held in
// registers), online softmax in float32 with exp2 and the scale folded into
// one FMA, P rounded to bf16, O^T += V^T P^T on the matrix cores.  The key
// blocks of a row are reduced in col_idx order by that one workgroup, so the
// result does not depend on the order rows are scheduled in.
//
// Scheduling: with a queue pointer the grid is persistent; each workgroup
// pops rows from the atomic counter of its XCD's partition of the work order
// (heads spread over partitions, rows longest first), then helps the other
// partitions.  Keeping a head's rows on one XCD keeps its K/V in that XCD's
// L2; longest-first puts the short rows at the tail of the launch.
#include "tiles.h"
#include "launch.h"

namespace calibatt {

// s_waitcnt immediate (gfx9 encoding) for vmcnt(N) with expcnt and lgkmcnt
// left unconstrained.  Written with the builtin rather than inline asm so that
// the compiler's own wait insertion knows which DMA has landed.
template <int N>
constexpr int vmcnt_imm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  return (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
}

__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>()); }

// Workgroup barrier for the DMA pipeline.  Every wave first waits (s_waitcnt
// vmcnt) for its own DMA writes that the next reads need; once it has, they
// are in LDS, so the barrier itself needs no wait for memory traffic.  The
// empty asm statements keep the compiler from moving LDS accesses across it;
// LDS reads and writes of the wave itself complete in order.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

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
      const int k = __builtin_amdgcn_readfirstlane(*s_item);
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

// Lazy rescale: the reference of a query's probabilities moves (to the
// running maximum) only when a sub-tile's probabilities sum past kSumCap, so
// O and l are rescaled a few times per row, and the row maxima are computed
// only then.  Probabilities stay at most kSumCap; O = acc / l is the same for
// any reference.
constexpr float kSumCap = 4096.f;

template <int I>
struct Cst {
  static constexpr int value = I;
};

// Geometry of the 32-queries-per-wave bf16 kernel: BLK/32 waves, each owning
// 32 queries, keys in sub-tiles of 64 (a kept block of 128 is two), two LDS
// stages that each hold a K sub-tile (64 rows of D/8 16-byte units) and a
// V^T sub-tile (D rows of 8 units), both filled by DMA.
template <int D, int BLK>
struct Geo {
  static constexpr int NW = BLK / 32;
  static constexpr int NT = NW * 64;
  static constexpr int BN = 64;
  static constexpr int SPB = BLK / BN;
  static constexpr int CH = D / 8;
  static constexpr int DS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int KS = BN / 16;
  static constexpr int KUNITS = BN * CH;
  static constexpr int VUNITS = D * 8;
  static constexpr int KPER = KUNITS / 64 / NW;
  static constexpr int VPER = VUNITS / 64 / NW;
  // DMA instruction m of a tile writes LDS units 64m .. 64m+63; the lane's
  // source offset within them depends on m modulo 4 only (the swizzles use
  // row bits 0..4), and wave w issues m = w, w + NW, ...
  static constexpr int PAT = 4 / NW;
};

// K DMA instruction i (0 .. KPER-1) of wave w for the K sub-tile at key k0
// (keys k0 .. k0+63, rows of D/8 units) into its swizzled LDS tile.
template <int D, int BLK>
__device__ __forceinline__ void k_dma_one(int i, __amdgpu_buffer_rsrc_t rk, int k0, u32x4* kt, int w,
                                          const int* kpat) {
  using G = Geo<D, BLK>;
  const int m = w + G::NW * i;
  const int voff = kpat[i % G::PAT];
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kt + 64 * m), 16, voff, k0 * D * 2 + m * 1024, 0, 0);
}

// V^T DMA instruction i (0 .. VPER-1) of wave w for the V^T sub-tile at key
// k0 (D rows of 128 contiguous bytes of V^T; instruction m covers rows
// 8m .. 8m+7) into its swizzled LDS tile.
template <int D, int BLK>
__device__ __forceinline__ void v_dma_one(int i, __amdgpu_buffer_rsrc_t rv, int k0, int L, u32x4* vt, int w,
                                          const int* vpat) {
  using G = Geo<D, BLK>;
  const int m = w + G::NW * i;
  const int voff = vpat[i % G::PAT];
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vt + 64 * m), 16, voff, k0 * 2 + m * 16 * L, 0, 0);
}

// DMA instruction i (0 .. KPER+VPER-1) of this wave for the sub-tile at key
// k0, into a stage that holds the K tile followed by the V^T tile.
template <int D, int BLK>
__device__ __forceinline__ void tile_dma(int i, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int k0,
                                         int L, u32x4* stage, int w, const int* kpat, const int* vpat) {
  using G = Geo<D, BLK>;
  if (i < G::KPER)
    k_dma_one<D, BLK>(i, rk, k0, stage, w, kpat);
  else
    v_dma_one<D, BLK>(i - G::KPER, rv, k0, L, stage + G::KUNITS, w, vpat);
}

// bf16 kernel, 32 queries per wave.  Sub-tile j of a row is computed from
// stage j%2 while the DMA of sub-tile j+1 fills the other stage:
//   S^T = K Q^T (Q in registers) on the matrix cores, the two 32-key halves
//   interleaved, with this wave's DMA instructions for sub-tile j+1 spread
//   between the products (issued in one burst right after the barrier they
//   queue behind the other waves' and stall the wave); tail keys masked;
//   P = exp2(S c2 - mc) rounded to bf16 and its row sums; the lazy rescale;
//   O^T += V^T P^T on the matrix cores; wait for the DMA, barrier.
// The key-block indices of a row are read two blocks ahead, so their scalar
// loads have returned when a DMA needs them.  Past the row's last sub-tile
// the DMA loads that sub-tile again into the free stage, so every step has
// the same shape.  Two waves per SIMD (two workgroups per CU) let one wave's
// softmax run beside the other's products; at d = 128 with 64-token blocks
// the registers allow only one.
template <int D, int BLK, bool DENSE>
__global__ __launch_bounds__(BLK * 2, (D == 128 && BLK == 64) ? 1 : 2) void attn_fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ Vt,
    bf16* __restrict__ O, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const int32_t* __restrict__ work_order, int32_t* __restrict__ queue, int items, int H, int L,
    int seq_len, int nkb_valid, float c2) {
  using G = Geo<D, BLK>;
  constexpr int DS = G::DS, DT = G::DT, KS = G::KS, CH = G::CH;
  // the two stages are separate LDS objects, so the DMA into one never
  // aliases the operand reads of the other
  __shared__ u32x4 st0[G::KUNITS + G::VUNITS];
  __shared__ u32x4 st1[G::KUNITS + G::VUNITS];
  __shared__ int s_item;

  const int nqb = L / BLK;
  const int rows = H * nqb;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, c = lane & 31;
  const int prow = qk_row_perm(c);
  const uint32_t slab_bytes = (uint32_t)L * D * 2;

  int kpat[G::PAT], vpat[G::PAT];
#pragma unroll
  for (int i = 0; i < G::PAT; ++i) {
    const int m = w + G::NW * i;
    const int krow = m * (64 / CH) + lane / CH;
    kpat[i] = (lane / CH) * D * 2 + (((lane % CH) ^ swz<CH>(krow)) * 16);
    const int vrow = m * 8 + lane / 8;
    vpat[i] = (lane / 8) * L * 2 + (((lane % 8) ^ swz<8>(vrow)) * 16);
  }
  // operand reads: K row 32*mt + prow, unit 2s+g; V^T row 32*t + c, unit
  // 2ks+g.  The swizzles see row bits 0..4 only, so the unit is the lane's
  // constant XOR the k-step.
  // The byte offsets of the DS + KS operand reads are kept in registers for
  // the whole kernel, so that a read costs no address arithmetic: the stage
  // and the 32-row tile are added as the instruction's immediate offset.
  const int kx = g ^ swz<CH>(prow);
  const int vx = g ^ swz<8>(c);
  int koffs[DS], voffs[KS];
#pragma unroll
  for (int s = 0; s < DS; ++s) koffs[s] = (prow * CH + ((2 * s) ^ kx)) * 16;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) voffs[ks] = (G::KUNITS + c * 8 + ((2 * ks) ^ vx)) * 16;
#pragma unroll
  for (int s = 0; s < DS; ++s) asm volatile("" : "+v"(koffs[s]));
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(voffs[ks]));
  auto kread = [&](const u32x4* t, int mt, int s) __attribute__((always_inline)) {
    return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(t) + mt * 32 * CH * 16 + koffs[s]);
  };
  auto vread = [&](const u32x4* t, int dt, int ks) __attribute__((always_inline)) {
    return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(t) + dt * 32 * 8 * 16 + voffs[ks]);
  };

  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one2 = {(bf16)1.f, (bf16)1.f};

  const RowSource src{work_order, rows, nqb, H, items / rows};
  for_each_row(src, queue, &s_item, [&](int b, int r) {
    const int h = r / nqb, qb = r - h * nqb;
    const size_t base = ((size_t)b * H + h) * (size_t)L * D;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + base, slab_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vt + base, slab_bytes);
    const int q = qb * BLK + 32 * w + c;   // this lane's query

    const int beg = DENSE ? 0 : row_ptr[r];
    const int nblk = (DENSE ? nkb_valid : row_ptr[r + 1]) - beg;
    const int nsub = nblk * G::SPB;
    // key blocks: kb0 holds the current sub-tile's, kb1 the next block's,
    // kb2 the one after (its load is in flight for a whole block)
    auto blk = [&](int i) __attribute__((always_inline)) -> int {
      i = i < nblk ? i : nblk - 1;
      return DENSE ? i : col_idx[beg + i];
    };
    int kb0 = 0, kb1 = 0, kb2 = 0;
    if (nsub > 0) {
      kb0 = blk(0);
      kb1 = blk(1);
      kb2 = blk(2);
#pragma unroll
      for (int i = 0; i < G::KPER + G::VPER; ++i) tile_dma<D, BLK>(i, rk, rv, kb0 * BLK, L, st0, w, kpat, vpat);
    }

    bf16x8 qreg[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qreg[s] = *reinterpret_cast<const bf16x8*>(Q + base + (size_t)q * D + 16 * s + 8 * g);

    f32x16 oacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
    float mc = kNegInf, l_run = 0.f;   // reference of P (log2 units) and row sum
    wait_vm();
    lds_barrier();

    // sub-tile j (part p of its block kb0): S from stage B, DMA of sub-tile
    // j+1 (clamped to the last) into the other stage
    auto step = [&](int j, auto bufc, int p) __attribute__((always_inline)) {
      constexpr int B = decltype(bufc)::value;
      constexpr int NDMA = G::KPER + G::VPER;
      const u32x4* const cur = B == 0 ? st0 : st1;
      u32x4* const nxt = B == 0 ? st1 : st0;
      const int k0 = kb0 * BLK + p * G::BN;
      const int kd = j + 1 >= nsub ? k0 : (p + 1 < G::SPB ? k0 + G::BN : kb1 * BLK);

      // slot s: operand reads two slots ahead, the products of both 32-key
      // halves at k-step s, then this slot's share of the DMA
      f32x16 sacc[2];
      {
        u32x4 ra[3][2];
        ra[0][0] = kread(cur, 0, 0);
        ra[0][1] = kread(cur, 1, 0);
        if (DS > 1) {
          ra[1][0] = kread(cur, 0, 1);
          ra[1][1] = kread(cur, 1, 1);
        }
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          if (s + 2 < DS) {
            ra[(s + 2) % 3][0] = kread(cur, 0, s + 2);
            ra[(s + 2) % 3][1] = kread(cur, 1, s + 2);
          }
          sacc[0] = mfma_bf16(__builtin_bit_cast(bf16x8, ra[s % 3][0]), qreg[s], s == 0 ? f32x16{} : sacc[0]);
          sacc[1] = mfma_bf16(__builtin_bit_cast(bf16x8, ra[s % 3][1]), qreg[s], s == 0 ? f32x16{} : sacc[1]);
#pragma unroll
          for (int i = s * NDMA / DS; i < (s + 1) * NDMA / DS; ++i)
            tile_dma<D, BLK>(i, rk, rv, kd, L, nxt, w, kpat, vpat);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (k0 + G::BN > seq_len) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            if (k0 + 32 * mt + slice_key(rr, g) >= seq_len) sacc[mt][rr] = kNegInf;
      }

      // P = exp2(S c2 - mc) against the current reference, and its row sums
      // (of the rounded values, the ones P*V uses) in two chains
      bf16x8 pb[KS];
      float ls[2];
      auto probs = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          bf16x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (bf16)fast_exp2(fmaf(sacc[ks >> 1][8 * (ks & 1) + e], c2, -mc));
          pb[ks] = v;
        }
        ls[0] = ls[1] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const bf16x2 pr = {pb[ks][e], pb[ks][e + 1]};
            ls[(e >> 1) & 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, ls[(e >> 1) & 1], false);
          }
      };
      probs();
      // The reference moves only when a lane's sum passes kSumCap (or is not
      // finite: the first sub-tile, whose reference is -inf): then to the row
      // maximum, with O and l rescaled and P recomputed.  Every probability
      // stays at most kSumCap, and O = acc / l does not depend on the
      // reference.
      if (__any(!(ls[0] + ls[1] <= kSumCap))) {
        float mx = kNegInf;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, sacc[mt][rr]);
        float mc_new = fmaxf(mc, pair_max(mx) * c2);
        if (mc_new == kNegInf) mc_new = 0.f;   // every key so far masked
        const float alpha = fast_exp2(mc - mc_new);
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
        mc = mc_new;
        probs();
      }
      l_run += ls[0] + ls[1];

#pragma unroll
      for (int t = 0; t < DT; ++t) {
        u32x4 a[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a[ks] = vread(cur, t, ks);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) oacc[t] = mfma_bf16(__builtin_bit_cast(bf16x8, a[ks]), pb[ks], oacc[t]);
      }
      wait_vm();
      lds_barrier();
    };

    // after the last sub-tile of a block the window moves on one block
    int nb = 3;   // next block index to load
    auto shift = [&]() __attribute__((always_inline)) {
      kb0 = kb1;
      kb1 = kb2;
      kb2 = blk(nb++);
    };
    for (int j = 0; j < nsub; j += 2) {
      step(j, Cst<0>{}, 0);
      if (G::SPB == 1) shift();
      if (j + 1 < nsub) step(j + 1, Cst<1>{}, G::SPB == 1 ? 0 : 1);
      shift();
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

// bf16 kernel for 128-token blocks in ping-pong form.  One workgroup of 8
// waves per CU serves one row: wave group A (waves 0-3) takes the even
// 64-key sub-tiles of the row and group B (waves 4-7) the odd ones, each
// wave the same 32 queries as its partner w ^ 4, which shares its SIMD.
// Each group keeps its own reference, row sums and O; at the end of the row
// B hands its state to A through LDS and A writes the combined result (a
// fixed split, so the result does not depend on scheduling).
//
// Time is cut into barrier-separated phases t = 0 .. n+1 (n sub-tiles).  In
// phase t the group of parity t does only matrix-core work and the other
// only vector work, so the two waves of a SIMD always hold complementary
// work:
//   matrix phase  S(t) = K(t) Q^T, with this wave's share of the DMA of
//                 K(t+2) and V^T(t) spread between the products; then
//                 O^T += V^T(t-2) P(t-2)^T
//   vector phase  P(t-1) = exp2(S(t-1) c2 - mc) rounded to bf16, its row
//                 sums and the lazy rescale; then wait for this wave's DMA
//                 of the phase before
// A DMA issued in phase t has landed by the end of phase t+1, so K(x) is
// issued two phases before S(x) reads it and V^T(x) two phases before
// P*V(x).  K and V^T rotate through three LDS stages each.
//
// SPLITQ: the rows are the anchor queries of the spatial-repetition heads:
// query m < q_valid of head h is token anchor_token(m) of Q (read in place),
// O is [B, H, Lq, d] with Lq a multiple of 128, rows h*(Lq/128) + qb; keys
// still run over K and V^T of length L with seq_len valid.
template <int D, bool DENSE, bool SPLITQ = false>
__global__ __launch_bounds__(512) void attn_fwd_pp_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ Vt,
    bf16* __restrict__ O, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const int32_t* __restrict__ work_order, int32_t* __restrict__ queue, int items, int H, int L,
    int seq_len, int nkb_valid, float c2, int Lq, int q_valid, int grid_rows, int grid_cols, int k_anchor) {
  constexpr int BLK = 128;
  using G = Geo<D, BLK>;   // one wave group: NW = 4 waves of 32 queries
  constexpr int DS = G::DS, DT = G::DT, KS = G::KS, CH = G::CH;
  constexpr int NDMA = G::KPER + G::VPER;
  static_assert(G::KUNITS == G::VUNITS, "K and V^T stages have one size");
  static_assert(DT * 2 * 8192 <= 4 * G::KUNITS * 16, "group B's O fits in K0, K1, K2 and V0");
  constexpr int OBJ = G::KUNITS * 16;   // bytes of one stage
  __shared__ u32x4 ks0[G::KUNITS], ks1[G::KUNITS], ks2[G::KUNITS];
  __shared__ u32x4 vs0[G::VUNITS], vs1[G::VUNITS], vs2[G::VUNITS];
  __shared__ int s_next[8];   // the next row: b, r (-1: none), first list entry, blocks, kb0, kb1, kb2
  __shared__ int s_fstate[2];   // the fetching wave's queue state: partition, partitions tried
  __shared__ float s_ml[G::NW * 64 * 2];   // group B's reference and row sum, per lane
  u32x4* const kst[3] = {ks0, ks1, ks2};
  u32x4* const vst[3] = {vs0, vs1, vs2};

  const int nqb = (SPLITQ ? Lq : L) / BLK;
  const int rows = H * nqb;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wv >> 2;   // 0: even sub-tiles, 1: odd
  const int w = wv & 3;      // query slice of the block
  const int g = lane >> 5, c = lane & 31;
  const int prow = qk_row_perm(c);
  const uint32_t slab_bytes = (uint32_t)L * D * 2;

  int kpat[G::PAT], vpat[G::PAT];
#pragma unroll
  for (int i = 0; i < G::PAT; ++i) {
    const int m = w + G::NW * i;
    const int krow = m * (64 / CH) + lane / CH;
    kpat[i] = (lane / CH) * D * 2 + (((lane % CH) ^ swz<CH>(krow)) * 16);
    const int vrow = m * 8 + lane / 8;
    vpat[i] = (lane / 8) * L * 2 + (((lane % 8) ^ swz<8>(vrow)) * 16);
  }
  // operand read offsets, kept in registers (see the 4-wave kernel)
  const int kx = g ^ swz<CH>(prow);
  const int vx = g ^ swz<8>(c);
  int koffs[DS], voffs[KS];
#pragma unroll
  for (int s = 0; s < DS; ++s) koffs[s] = (prow * CH + ((2 * s) ^ kx)) * 16;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) voffs[ks] = (c * 8 + ((2 * ks) ^ vx)) * 16;
#pragma unroll
  for (int s = 0; s < DS; ++s) asm volatile("" : "+v"(koffs[s]));
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(voffs[ks]));
  auto kread = [&](const u32x4* t, int mt, int s) __attribute__((always_inline)) {
    return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(t) + mt * 32 * CH * 16 + koffs[s]);
  };
  auto vread = [&](const u32x4* t, int dt, int ks) __attribute__((always_inline)) {
    return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(t) + dt * 32 * 8 * 16 + voffs[ks]);
  };

  // the V^T stages start as zeros, so that a product with zero
  // probabilities never meets a non-finite LDS value
  for (int u = threadIdx.x; u < G::VUNITS; u += 512) vs0[u] = vs1[u] = vs2[u] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();

  const RowSource src{work_order, rows, nqb, H, items / rows};
  // Rows come from the same per-XCD queues as in for_each_row, but wave 4
  // fetches the next row while group A merges the current one: the queue
  // pop, its work-order entry, the row's list bounds and first three key
  // blocks (a chain of dependent loads) land in LDS before the row starts.
  // The queue state lives in LDS too, so that no register is held through
  // the phase loop for it.
  if (threadIdx.x == 0) {
    s_fstate[0] = blockIdx.x % kParts;
    s_fstate[1] = 0;
  }
  __syncthreads();
  auto fetch_next = [&]() __attribute__((always_inline)) {
    int p_f = __builtin_amdgcn_readfirstlane(s_fstate[0]);
    int tries_f = __builtin_amdgcn_readfirstlane(s_fstate[1]);
    int b_ = 0, r_ = -1;
    if (!queue) {   // one workgroup per row: row blockIdx.x of the order, once
      if (tries_f == 0) {
        tries_f = kParts;
        const int item = blockIdx.x;
        b_ = item / src.rows;
        const int j = item - b_ * src.rows;
        r_ = src.order ? src.order[j] : j;
      }
    }
    while (queue && tries_f < kParts) {
      int k = 0;
      if (lane == 0) k = atomicAdd(queue + p_f * kQueueStride, 1);
      k = __builtin_amdgcn_readfirstlane(k);
      const int len = src.part_len(p_f);
      if (k >= src.B * len) {
        p_f = (p_f + 1) % kParts;
        ++tries_f;
        continue;
      }
      b_ = k / len;
      r_ = src.part_row(p_f, k - b_ * len);
      break;
    }
    int beg_ = 0, nblk_ = 0, k0_ = 0, k1_ = 0, k2_ = 0;
    if (r_ >= 0) {
      beg_ = DENSE ? 0 : row_ptr[r_];
      nblk_ = (DENSE ? nkb_valid : row_ptr[r_ + 1]) - beg_;
      if (nblk_ > 0) {
        auto bl = [&](int i) __attribute__((always_inline)) -> int {
          i = i < nblk_ ? i : nblk_ - 1;
          return DENSE ? i : col_idx[beg_ + i];
        };
        k0_ = bl(0);
        k1_ = bl(1);
        k2_ = bl(2);
      }
    }
    if (lane == 0) {
      s_fstate[0] = p_f;
      s_fstate[1] = tries_f;
      s_next[0] = b_;
      s_next[1] = r_;
      s_next[2] = beg_;
      s_next[3] = nblk_;
      s_next[4] = k0_;
      s_next[5] = k1_;
      s_next[6] = k2_;
    }
  };
  auto body = [&](int b, int r, int beg, int nblk, int pk0, int pk1, int pk2) {
    const int h = r / nqb, qb = r - h * nqb;
    const size_t base = ((size_t)b * H + h) * (size_t)L * D;
    const size_t qbase = SPLITQ ? ((size_t)b * H + h) * (size_t)Lq * D : base;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + base, slab_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vt + base, slab_bytes);
    const int q = qb * BLK + 32 * w + c;   // this lane's query

    const int n = nblk * 2;   // sub-tiles
    // key blocks around phase t (block b = t/2): kbm = b-1, kb0 = b, kb1 =
    // b+1; kb2 (b+2) is loaded a block ahead
    int kbm = 0, kb0 = 0, kb1 = 0, kb2 = 0;
    // Inside the phase loop the indices come from two vector registers that
    // hold 64 consecutive entries of the row's list each (lane l: entry
    // 64*chunk + l), read with readlane: a scalar memory load there would
    // make the next LDS wait also wait for it.  The next chunk is loaded 64
    // blocks before it is read.
    auto idx_chunk = [&](int cix) __attribute__((always_inline)) -> int {
      int j = 64 * cix + lane;
      j = j < nblk ? j : nblk - 1;
      return DENSE ? j : col_idx[beg + j];
    };
    int cbase = 0, ck_cur = 0, ck_nxt = 0;
    if (n > 0) {
      kb0 = pk0;
      kb1 = pk1;
      kb2 = pk2;
      if (!DENSE) {
        ck_cur = idx_chunk(0);
        ck_nxt = idx_chunk(1);
      }
      // K(0) by group A, K(1) by group B
#pragma unroll
      for (int i = 0; i < G::KPER; ++i)
        k_dma_one<D, BLK>(i, rk, kb0 * BLK + grp * G::BN, grp == 0 ? ks0 : ks1, w, kpat);
    }

    // Q is scaled by c2 (the softmax scale in log2 units) on loading and
    // rounded to bf16, so that the products give scores in log2 units and,
    // with the accumulators started at -ref, exp2 needs no vector arithmetic
    // before it
    // the token this lane's query reads (anchor rows: through the anchor
    // map; padding rows past q_valid read token 0 and are never written)
    const int qsrc = SPLITQ ? (q < q_valid ? anchor_token(q, grid_rows, grid_cols, k_anchor) : 0) : q;
    bf16x8 qreg[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const bf16x8 qv = *reinterpret_cast<const bf16x8*>(Q + base + (size_t)qsrc * D + 16 * s + 8 * g);
#pragma unroll
      for (int e = 0; e < 8; ++e) qreg[s][e] = (bf16)((float)qv[e] * c2);
    }

    f32x16 oacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
    // this group's reference (log2 units) and row sum; fresh until the
    // reference has been set from the maximum of a sub-tile with valid keys
    float ref = 0.f, l_run = 0.f;
    bool fresh = true;
    f32x16 cneg = {};   // -ref in every accumulator register
    f32x16 sacc[2];
    bf16x8 pb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) pb[ks] = bf16x8{};   // P*V of phases 0 and 1 adds nothing
    bool rescale = false;   // O *= alpha is due before the next P*V
    float alpha = 1.f;
    wait_vm();
    lds_barrier();

    // after a phase of odd t the next phase is in the next block
    auto shift = [&](int t) __attribute__((always_inline)) {
      kbm = kb0;
      kb0 = kb1;
      kb1 = kb2;
      int j = (t + 1) / 2 + 2;
      j = j < nblk ? j : nblk - 1;
      if (DENSE) {
        kb2 = j;
      } else {
        const bool adv = (j >> 6) != cbase;   // j moves on by at most one per call
        if (adv) {
          ++cbase;
          ck_cur = ck_nxt;
        }
        kb2 = __builtin_amdgcn_readlane(ck_cur, j & 63);
        if (adv) ck_nxt = idx_chunk(cbase + 1);
      }
    };
    // matrix phase t, with TM = t % 6 fixing the stages.  S(t) and
    // P*V(t-2) run as one sequence of slots, each one pair of products and
    // the operand reads of the slot PF ahead, so the P*V operands are in
    // flight while the last scores are computed.  Every phase up to n+1 has
    // this one shape: in phases 0 and 1 P is zero, so P*V adds nothing (the
    // V^T stages always hold finite values: zeroed at the start, later only
    // V^T tiles); in phases n and n+1 the scores come from a stale K stage
    // and are never used; the DMA keys are clamped to the row.
    auto mphase = [&](int t, auto tmc) __attribute__((always_inline)) {
      constexpr int TM = decltype(tmc)::value;
      constexpr int KST = TM % 3, KDST = (TM + 2) % 3, VST = (TM + 1) % 3, VDST = TM % 3;
      // the wave index, re-read in every phase so that the DMA destinations
      // (one per stage and instruction) are formed where they are used
      // instead of all being kept in scalar registers
      int wq;
      asm volatile("s_mov_b32 %0, %1" : "=s"(wq) : "s"(w));
      const int kd = kb1 * BLK + (TM & 1) * G::BN;   // K(t+2), clamped by blk()
      const int vd = kb0 * BLK + (TM & 1) * G::BN;   // V^T(t)
      const u32x4* const kc = kst[KST];
      const u32x4* const vc = vst[VST];
      auto dma_share = [&](int s) __attribute__((always_inline)) {
#pragma unroll
        for (int i = s * NDMA / DS; i < (s + 1) * NDMA / DS; ++i) {
          if (i < G::KPER)
            k_dma_one<D, BLK>(i, rk, kd, kst[KDST], wq, kpat);
          else
            v_dma_one<D, BLK>(i - G::KPER, rv, vd, L, vst[VDST], wq, vpat);
        }
      };
      // O moves to the reference P(t-2) was computed against
      auto apply_rescale = [&]() __attribute__((always_inline)) {
        if (rescale) {
#pragma unroll
          for (int tt = 0; tt < DT; ++tt) oacc[tt] *= alpha;
          rescale = false;
        }
      };
      if (t < n + 2) {
        apply_rescale();
        constexpr int NSL = DS + DT * KS / 2;   // slots: DS of scores, then P*V
        constexpr int PF = 2;                   // operand reads run PF slots ahead
        // operand h of slot sl: K row tile h at k-step sl, or the V^T tile of
        // P*V product 2 (sl - DS) + h (ks = i / DT, dt = i % DT)
        auto rd = [&](int sl, int h) __attribute__((always_inline)) -> u32x4 {
          if (sl < DS) return kread(kc, h, sl);
          const int i = 2 * (sl - DS) + h;
          return vread(vc, i % DT, i / DT);
        };
        u32x4 ra[PF + 1][2];
#pragma unroll
        for (int sl = 0; sl < PF; ++sl) {
          ra[sl][0] = rd(sl, 0);
          ra[sl][1] = rd(sl, 1);
        }
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) {
          if (sl + PF < NSL) {
            ra[(sl + PF) % (PF + 1)][0] = rd(sl + PF, 0);
            ra[(sl + PF) % (PF + 1)][1] = rd(sl + PF, 1);
          }
          const bf16x8 a0 = __builtin_bit_cast(bf16x8, ra[sl % (PF + 1)][0]);
          const bf16x8 a1 = __builtin_bit_cast(bf16x8, ra[sl % (PF + 1)][1]);
          if (sl < DS) {
            sacc[0] = mfma_bf16(a0, qreg[sl], sl == 0 ? cneg : sacc[0]);
            sacc[1] = mfma_bf16(a1, qreg[sl], sl == 0 ? cneg : sacc[1]);
            dma_share(sl);
          } else {
            const int i0 = 2 * (sl - DS), i1 = i0 + 1;
            oacc[i0 % DT] = mfma_bf16(a0, pb[i0 / DT], oacc[i0 % DT]);
            oacc[i1 % DT] = mfma_bf16(a1, pb[i1 / DT], oacc[i1 % DT]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      lds_barrier();
      if (TM & 1) shift(t);
    };
    // vector phase t: P(t-1); then this wave's DMA of the phase before, which
    // the next phase reads, must have landed
    auto vphase = [&](int t, auto tmc) __attribute__((always_inline)) {
      constexpr int TM = decltype(tmc)::value;
      {
        const int x = t - 1;
        if (x >= 0 && x < n) {
          const int k0 = (TM & 1) ? kb0 * BLK : kbm * BLK + G::BN;
          if (k0 + G::BN > seq_len) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
              for (int rr = 0; rr < 16; ++rr)
                if (k0 + 32 * mt + slice_key(rr, g) >= seq_len) sacc[mt][rr] = kNegInf;
          }
          // P rounded to bf16 for the products; its row sums in fp32 from
          // the unrounded values, in four chains (plain adds run beside the
          // other wave's matrix products far better than dot2 does)
          float ls[2];
          auto probs = [&]() __attribute__((always_inline)) {
            float ch[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              bf16x8 v;
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float pe = fast_exp2(sacc[ks >> 1][8 * (ks & 1) + e]);
                v[e] = (bf16)pe;
                ch[e & 3] += pe;
              }
              pb[ks] = v;
            }
            ls[0] = ch[0] + ch[1];
            ls[1] = ch[2] + ch[3];
          };
          probs();
          // the reference moves to the row maximum on the first sub-tile
          // with valid keys, and later only when a lane's sum passes kSumCap
          const bool redo = (fresh && k0 < seq_len) || __any(!(ls[0] + ls[1] <= kSumCap));
          if (redo) {
            float mx = kNegInf;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
              for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, sacc[mt][rr]);
            mx = pair_max(mx);   // relative to ref; finite (a valid key is in range)
            const float delta = fresh ? mx : fmaxf(mx, 0.f);
            if (!fresh) {
              alpha = fast_exp2(-delta);
              l_run *= alpha;
              rescale = true;
            }
            fresh = false;
            ref += delta;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
              for (int rr = 0; rr < 16; ++rr) {
                sacc[mt][rr] -= delta;
                cneg[rr] = -ref;
              }
          }
          if (redo) probs();
          l_run += ls[0] + ls[1];
        }
        wait_vm();
      }
      lds_barrier();
      if (TM & 1) shift(t);
    };

    // each wave alternates matrix and vector phases, six to a loop turn with
    // no phase skipped (a phase past the row's work only meets the barrier),
    // so on every path a matrix phase follows the vector phase that waited
    // for its DMA.  Both groups meet T + 1 barriers: group A runs phases
    // 0 .. T-1 and one empty one, group B an empty vector phase 0 and then
    // phases 1 .. T.
    const int T = ((n + 2 + 5) / 6) * 6;
    auto run = [&](auto gc) __attribute__((always_inline)) {
      constexpr int GR = decltype(gc)::value;
      if (GR == 1) vphase(0, Cst<0>{});
      for (int t = GR; t < T + GR; t += 6) {
        mphase(t, Cst<GR % 6>{});
        vphase(t + 1, Cst<(GR + 1) % 6>{});
        mphase(t + 2, Cst<(GR + 2) % 6>{});
        vphase(t + 3, Cst<(GR + 3) % 6>{});
        mphase(t + 4, Cst<(GR + 4) % 6>{});
        vphase(t + 5, Cst<(GR + 5) % 6>{});
      }
      if (GR == 0) lds_barrier();
    };
    if (n > 0) {
      if (grp == 0)
        run(Cst<0>{});
      else
        run(Cst<1>{});
    }

    // group B hands O, ref and l to group A: O in 8-float chunks u = 0 ..
    // 2*DT-1 of every lane, chunk u in stage object (u * 8 KiB) / OBJ of
    // K0, K1, K2, V0 (never V1 or V2: the P*V of the next row's phases 0
    // and 1 reads those with zero probabilities, so they may only hold V^T
    // tiles or zeros), ref and l in s_ml
    char* const objs[4] = {(char*)ks0, (char*)ks1, (char*)ks2, (char*)vs0};
    auto chunk = [&](int u) __attribute__((always_inline)) -> float* {
      return reinterpret_cast<float*>(objs[(u * 8192) / OBJ] + (u * 8192) % OBJ) + (w * 64 + lane) * 8;
    };
    float* const ml = s_ml + (w * 64 + lane) * 2;
    if (grp == 1) {
#pragma unroll
      for (int u = 0; u < 2 * DT; ++u) {
        f32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = oacc[u >> 1][8 * (u & 1) + e];
          hi[e] = oacc[u >> 1][8 * (u & 1) + 4 + e];
        }
        reinterpret_cast<f32x4*>(chunk(u))[0] = lo;
        reinterpret_cast<f32x4*>(chunk(u))[1] = hi;
      }
      ml[0] = fresh ? kNegInf : ref;
      ml[1] = l_run;
    }
    lds_barrier();
    if (grp == 0) {
      // a group that saw no valid key (fresh) holds nothing and is left out
      const float mca = fresh ? kNegInf : ref;
      const float mcb = ml[0], lb = ml[1];
      float m = fmaxf(mca, mcb);
      if (m == kNegInf) m = 0.f;
      const float aa = fast_exp2(mca - m), ab = fast_exp2(mcb - m);
      const float l_tot = pair_sum(l_run * aa + lb * ab);
      const float inv = (q < (SPLITQ ? q_valid : seq_len) && l_tot > 0.f) ? 1.f / l_tot : 0.f;
      const float fa = aa * inv, fb = ab * inv;
      bf16* Ob = O + qbase + (size_t)q * D;
#pragma unroll
      for (int u = 0; u < 2 * DT; ++u) {
        const f32x4 lo = reinterpret_cast<const f32x4*>(chunk(u))[0];
        const f32x4 hi = reinterpret_cast<const f32x4*>(chunk(u))[1];
        const int t = u >> 1;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int rq = 2 * (u & 1) + half;   // register quad: rows 4*rq .. 4*rq+3 of the tile
          const f32x4 ob = half ? hi : lo;
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (bf16)(oacc[t][4 * rq + e] * fa + ob[e] * fb);
          *reinterpret_cast<bf16x4*>(Ob + 32 * t + 8 * rq + 4 * g) = o;
        }
      }
    } else if (wv == 4) {
      // group B is idle while A merges: fetch the next row
      fetch_next();
    }
    // the stages are free again for the next row's DMA
    lds_barrier();
  };
  if (wv == 4) fetch_next();
  __syncthreads();
  for (;;) {
    const int nb = __builtin_amdgcn_readfirstlane(s_next[0]);
    const int nr = __builtin_amdgcn_readfirstlane(s_next[1]);
    const int nbeg = __builtin_amdgcn_readfirstlane(s_next[2]);
    const int nn = __builtin_amdgcn_readfirstlane(s_next[3]);
    const int n0 = __builtin_amdgcn_readfirstlane(s_next[4]);
    const int n1 = __builtin_amdgcn_readfirstlane(s_next[5]);
    const int n2 = __builtin_amdgcn_readfirstlane(s_next[6]);
    // every wave has read the entry before wave 4 may write the next one
    // (it does so only in the row's merge, many barriers later)
    __syncthreads();
    if (nr < 0) break;
    body(nb, nr, nbeg, nn, n0, n1, n2);
  }
}

// float32 path: 32-key slices, fp32 matrix cores (32x32x2), P kept in float32.
// Lane (g, c) holds, for slice accumulator register r, key 2r + g (rows of
// the K slice are fed in that order), which is the B layout of P^T.
template <int D, int BLK, bool DENSE>
__global__ __launch_bounds__(BLK * 2) void attn_fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ Vt,
    float* __restrict__ O, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const int32_t* __restrict__ work_order, int32_t* __restrict__ queue, int items, int H, int L,
    int seq_len, int nkb_valid, float c2) {
  constexpr int NT = BLK * 2;
  constexpr int KP = D + 1;   // padded K and V rows (floats)
  constexpr int DT = D / 32;
  __shared__ float ldsK[32 * KP];
  __shared__ float ldsV[32 * KP];
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
          const int vk = i % 32, vd = i / 32;   // V^T row vd, 32 consecutive keys
          ldsV[vk * KP + vd] = Vt[base + (size_t)vd * L + k0 + vk];
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
            oacc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(ldsV[(2 * rr + g) * KP + 32 * t + c], p[rr],
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

// V [B, H, L, d] -> V^T [B, H, d, L], keys at or past seq_len written as 0
// (so that the zero probabilities of masked keys never meet a non-finite V).
// One workgroup per 64 keys of one head; elements are moved as raw bits.
template <typename T, int D>
__global__ __launch_bounds__(256) void transpose_v_kernel(const T* __restrict__ V, T* __restrict__ Vt, int L,
                                                           int seq_len) {
  constexpr int KB = 64;
  constexpr int VEC = 16 / sizeof(T);      // elements per 16-byte access
  constexpr int RS = D + 4 / sizeof(T);    // padded LDS row (elements): rows shift by one bank
  __shared__ T tile[KB * RS];
  const int tiles_per_head = L / KB;
  const int bh = blockIdx.x / tiles_per_head;
  const int k0 = (blockIdx.x - bh * tiles_per_head) * KB;
  const T* src = V + (size_t)bh * L * D + (size_t)k0 * D;
  T* dst = Vt + (size_t)bh * D * L + k0;
  for (int i = threadIdx.x; i < KB * D / VEC; i += 256) {
    const int kr = i / (D / VEC), dv = (i % (D / VEC)) * VEC;
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + (size_t)kr * D + dv);
#pragma unroll
    for (int x = 0; x < VEC; ++x) tile[kr * RS + dv + x] = reinterpret_cast<const T*>(&v)[x];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < D * KB / VEC; i += 256) {
    const int d = i / (KB / VEC), kk = (i % (KB / VEC)) * VEC;
    u32x4 v;
#pragma unroll
    for (int x = 0; x < VEC; ++x)
      reinterpret_cast<T*>(&v)[x] = (k0 + kk + x < seq_len) ? tile[(kk + x) * RS + d] : T(0);
    *reinterpret_cast<u32x4*>(dst + (size_t)d * L + kk) = v;
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

template <int D, bool DENSE, bool SPLITQ = false>
static hipError_t launch_pp(const AttnArgs& a, hipStream_t st) {
  const int Lq = SPLITQ ? a.Lq : a.L;
  const int items = a.B * a.H * (Lq / 128);
  const float c2 = a.scale * kLog2e;
  if (items == 0) return hipSuccess;
  int grid = items;
  if (a.queue) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(kQueueInts), 0, st, a.queue, kQueueInts, 0);
    int per_cu = 1;
    hipError_t e = occupancy(attn_fwd_pp_kernel<D, DENSE, SPLITQ>, 512, &per_cu);
    if (e != hipSuccess) return e;
    const long long cap = (long long)a.num_cu * (per_cu > 0 ? per_cu : 1);
    grid = (int)(cap < items ? cap : items);
  }
  hipLaunchKernelGGL((attn_fwd_pp_kernel<D, DENSE, SPLITQ>), dim3(grid), dim3(512), 0, st, (const bf16*)a.Q,
                     (const bf16*)a.K, (const bf16*)a.Vt, (bf16*)a.O, a.row_ptr, a.col_idx, a.work_order, a.queue,
                     items, a.H, a.L, a.seq_len, a.nkb_valid, c2, Lq, SPLITQ ? a.q_valid : a.seq_len,
                     a.grid_rows, a.grid_cols, a.k_anchor);
  return hipGetLastError();
}

hipError_t launch_anchor_attention(const AttnArgs& a, hipStream_t st) {
  if (a.dtype_f32 || a.block != 128 || !a.work_order || !a.queue) return hipErrorInvalidValue;
  if (a.d == 128) return launch_pp<128, true, true>(a, st);
  return launch_pp<64, true, true>(a, st);
}

template <int D, int BLK, bool DENSE>
static hipError_t launch_typed(const AttnArgs& a, hipStream_t st) {
  if (BLK == 128 && !a.dtype_f32) return launch_pp<D, DENSE>(a, st);
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
                       (const float*)a.Q, (const float*)a.K, (const float*)a.Vt, (float*)a.O,
                       a.row_ptr, a.col_idx, a.work_order, a.queue, items, a.H, a.L, a.seq_len,
                       a.nkb_valid, c2);
  } else {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, BLK, DENSE>), dim3(grid), dim3(threads), 0, st,
                       (const bf16*)a.Q, (const bf16*)a.K, (const bf16*)a.Vt, (bf16*)a.O, a.row_ptr,
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

template <typename T>
static hipError_t transpose_typed(const TransposeArgs& a, hipStream_t st) {
  const int grid = a.B * a.H * (a.L / 64);
  if (grid == 0) return hipSuccess;
  if (a.d == 128)
    hipLaunchKernelGGL((transpose_v_kernel<T, 128>), dim3(grid), dim3(256), 0, st, (const T*)a.V, (T*)a.Vt, a.L,
                       a.seq_len);
  else
    hipLaunchKernelGGL((transpose_v_kernel<T, 64>), dim3(grid), dim3(256), 0, st, (const T*)a.V, (T*)a.Vt, a.L,
                       a.seq_len);
  return hipGetLastError();
}

hipError_t launch_transpose_v(const TransposeArgs& a, hipStream_t st) {
  return a.dtype_f32 ? transpose_typed<uint32_t>(a, st) : transpose_typed<uint16_t>(a, st);
}

}  // namespace calibatt
