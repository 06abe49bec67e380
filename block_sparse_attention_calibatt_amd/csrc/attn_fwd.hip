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
// stages that each hold a K sub-tile (64 rows of D/8 16-byte units) and a V
// sub-tile (64 rows of D/8 units in natural layout, or D rows of 8 units of
// V^T), both filled by DMA.
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

// V DMA instruction i (0 .. VPER-1) of wave w for the V sub-tile at key k0
// into its swizzled LDS tile: natural layout, instruction m covering key rows
// m*(64/CH) ..; or (VT) D rows of 128 contiguous bytes of V^T, instruction m
// covering rows 8m .. 8m+7.
template <int D, int BLK, bool VT>
__device__ __forceinline__ void v_dma_one(int i, __amdgpu_buffer_rsrc_t rv, int k0, int L, u32x4* vt, int w,
                                          const int* vpat) {
  using G = Geo<D, BLK>;
  const int m = w + G::NW * i;
  const int voff = vpat[i % G::PAT];
  const int soff = VT ? k0 * 2 + m * 16 * L : k0 * D * 2 + m * 1024;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vt + 64 * m), 16, voff, soff, 0, 0);
}

// DMA instruction i (0 .. KPER+VPER-1) of this wave for the sub-tile at key
// k0, into a stage that holds the K tile followed by the V tile.
template <int D, int BLK, bool VT>
__device__ __forceinline__ void tile_dma(int i, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int k0,
                                         int L, u32x4* stage, int w, const int* kpat, const int* vpat) {
  using G = Geo<D, BLK>;
  if (i < G::KPER)
    k_dma_one<D, BLK>(i, rk, k0, stage, w, kpat);
  else
    v_dma_one<D, BLK, VT>(i - G::KPER, rv, k0, L, stage + G::KUNITS, w, vpat);
}

// bf16 kernel, 32 queries per wave.  Sub-tile j of a row is computed from
// stage j%2 while the DMA of sub-tile j+1 fills the other stage:
//   S^T = K Q^T (Q in registers) on the matrix cores, the two 32-key halves
//   interleaved, with this wave's DMA instructions for sub-tile j+1 spread
//   between the products (issued in one burst right after the barrier they
//   queue behind the other waves' and stall the wave); tail keys masked;
//   P = exp2(S c2 - mc) rounded to bf16 and its row sums; the lazy rescale;
//   O^T += V^T P^T on the matrix cores (the V^T operand by transposed LDS
//   reads of the natural-layout tile, or with VT plain reads of a V^T
//   tile); wait for the DMA, barrier.
// The key-block indices of a row are read two blocks ahead, so their scalar
// loads have returned when a DMA needs them.  Past the row's last sub-tile
// the DMA loads that sub-tile again into the free stage, so every step has
// the same shape.  Two waves per SIMD (two workgroups per CU) let one wave's
// softmax run beside the other's products; at d = 128 with 64-token blocks
// the registers allow only one.
template <int D, int BLK, bool DENSE, bool VT>
__global__ __launch_bounds__(BLK * 2, (D == 128 && BLK == 64) ? 1 : 2) void attn_fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
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
  constexpr int RB = D * 2;
  // K and V rows past seq_len read as zero (buffer range check)
  const uint32_t k_bytes = (uint32_t)seq_len * RB;
  const uint32_t v_bytes = VT ? (uint32_t)L * RB : (uint32_t)seq_len * RB;

  int kpat[G::PAT], vpat[G::PAT];
#pragma unroll
  for (int i = 0; i < G::PAT; ++i) {
    const int m = w + G::NW * i;
    const int krow = m * (64 / CH) + lane / CH;
    kpat[i] = (lane / CH) * RB + (((lane % CH) ^ swz<CH>(krow)) * 16);
    if (VT) {
      const int vrow = m * 8 + lane / 8;
      vpat[i] = (lane / 8) * L * 2 + (((lane % 8) ^ swz<8>(vrow)) * 16);
    } else {
      const int vrow = m * (64 / CH) + lane / CH;
      vpat[i] = (lane / CH) * RB + (((lane % CH) ^ vswz<D>(vrow)) * 16);
    }
  }
  // operand reads: K row 32*mt + prow, unit 2s+g.  V (natural layout): lane
  // 16G + 4jj + mm reads 8 bytes of key row 16ks + 8g + 4h + jj at d = 32t +
  // 16(G%2) + 4mm and the transposed read hands lane (g, c) its 4 keys at d =
  // 32t + c; V^T: row 32*t + c, unit 2ks+g.  The swizzles see row bits 0..4
  // only, so the unit is the lane's constant XOR the k-step.
  // The byte offsets of the operand reads are kept in registers for the
  // whole kernel, so that a read costs no address arithmetic: the stage and
  // the 32-row tile are added as the instruction's immediate offset.
  constexpr int NV = VT ? KS : DT;
  const int kx = g ^ swz<CH>(prow);
  int koffs[DS], voffs[NV];
#pragma unroll
  for (int s = 0; s < DS; ++s) koffs[s] = (prow * CH + ((2 * s) ^ kx)) * 16;
  if (VT) {
    const int vx = g ^ swz<8>(c);
#pragma unroll
    for (int ks = 0; ks < NV; ++ks) voffs[ks] = (G::KUNITS + c * 8 + ((2 * ks) ^ vx)) * 16;
  } else {
    const int jj = (lane >> 2) & 3, mm = lane & 3;
#pragma unroll
    for (int t = 0; t < NV; ++t)
      voffs[t] = G::KUNITS * 16 + (8 * g + jj) * RB +
                 (((4 * t + 2 * (c >> 4) + (mm >> 1)) ^ vswz<D>(jj)) * 16) + (mm & 1) * 8;
  }
#pragma unroll
  for (int s = 0; s < DS; ++s) asm volatile("" : "+v"(koffs[s]));
#pragma unroll
  for (int i = 0; i < NV; ++i) asm volatile("" : "+v"(voffs[i]));
  auto kread = [&](const u32x4* t, int mt, int s) __attribute__((always_inline)) {
    return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(t) + mt * 32 * CH * 16 + koffs[s]);
  };
  auto vread = [&](const u32x4* t, int dt, int ks) __attribute__((always_inline)) -> u32x4 {
    if (VT) return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(t) + dt * 32 * 8 * 16 + voffs[ks]);
    const char* p = reinterpret_cast<const char*>(t) + voffs[dt] + 16 * ks * RB;
    const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr16(p));
    const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr16(p + 4 * RB));
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };

  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one2 = {(bf16)1.f, (bf16)1.f};

  const RowSource src{work_order, rows, nqb, H, items / rows};
  for_each_row(src, queue, &s_item, [&](int b, int r) {
    const int h = r / nqb, qb = r - h * nqb;
    const size_t base = ((size_t)b * H + h) * (size_t)L * D;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + base, k_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + base, v_bytes);
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
      for (int i = 0; i < G::KPER + G::VPER; ++i) tile_dma<D, BLK, VT>(i, rk, rv, kb0 * BLK, L, st0, w, kpat, vpat);
    }

    // a padded query is taken as zero (its output is zeroed; a non-finite
    // value would also move the wave's shared rescale decisions)
    bf16x8 qreg[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qreg[s] = q < seq_len ? *reinterpret_cast<const bf16x8*>(Q + base + (size_t)q * D + 16 * s + 8 * g) : bf16x8{};

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
            tile_dma<D, BLK, VT>(i, rk, rv, kd, L, nxt, w, kpat, vpat);
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

    // padded query rows (and rows that saw no key) are written as zero,
    // whatever their accumulators hold
    const float l_tot = pair_sum(l_run);
    const bool valid = q < seq_len && l_tot > 0.f;
    const float inv = valid ? 1.f / l_tot : 0.f;
    bf16* Ob = O + base + (size_t)q * D;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * t + 8 * rq + 4 * g;
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = valid ? (bf16)(oacc[t][4 * rq + e] * inv) : (bf16)0.f;
        *reinterpret_cast<bf16x4*>(Ob + d0) = o;
      }
    }
  });
}

// Geometry of the 128-token-block kernel: keys in 64-key sub-tiles; a K
// stage holds one sub-tile as 64 rows of D/8 16-byte units, a V stage the
// same sub-tile of V (64 rows, natural layout) or of V^T (D rows of 8 units).
// Each wave group owns four stages: K0, K1, V0, V1.  The stages are four LDS
// objects, each holding both groups' stage of that name, so that the DMA
// into one stage and the operand reads of another are accesses to different
// objects, which the compiler can tell apart (it would otherwise wait for
// every DMA in flight before each read).  (Two objects of two stages each
// would do the same, but put every read of one matrix phase past the 64 KiB
// reach of the LDS instructions' immediate offset, which costs an address
// add per read or two.)
template <int D>
struct PPGeo {
  static constexpr int CH = D / 8;
  static constexpr int DS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int KS = 4;
  static constexpr int UNITS = 64 * CH;
  static constexpr int STAGE = UNITS * 16;
  static constexpr int NDMA = UNITS / 64 / 4;   // DMA instructions per wave per stage (4 waves)
  static constexpr int RB = D * 2;              // bytes of one K or V row
};

// bf16 kernel for 128-token blocks.  One workgroup of 8 waves per CU, in two
// groups of 4 (A: waves 0-3, B: waves 4-7; wave w and w+4 share a SIMD).  Each
// group serves rows on its own: its 4 waves own 32 queries each of the row's
// 128 and walk the row's 64-key sub-tiles in list order, so one group reduces
// a whole row and the result does not depend on scheduling.
//
// Time is cut into barrier-separated phases, and the groups alternate: in a
// phase one group does only matrix-core work and the other only vector work,
// so the two waves of a SIMD always hold complementary work.  A group's
// sub-tiles form one stream across its rows; cycle x of the stream is
//   matrix phase  S(x) = K(x) Q^T (Q in registers, pre-scaled), with this
//                 wave's share of the DMA of K(x+1) and V(x) spread between
//                 the products; then O^T += V^T(x-1) P(x-1)^T
//   vector phase  P(x) = exp2(S(x) - ref) rounded to bf16, its row sums and
//                 the lazy rescale; then wait for this wave's DMA
// so a DMA issued in a matrix phase has landed by the end of the next phase.
// At a row boundary the stream does not stop: the matrix phase that computes
// the last scores of a row loads the next row's Q after them and its first K
// tile, the next matrix phase computes the new row's first scores beside the
// old row's last P*V, and the vector phase after it writes the old row's O.
//
// V is read in its natural layout by default: a V tile goes to LDS by DMA as
// it lies (padded keys read as zero through the buffer's range check), and
// the transposed-read LDS instruction forms the P*V operand, whose
// contracted index (keys) must be contiguous in each lane.  With VT the
// kernel reads V^T [B, H, d, L] tiles instead, with plain 16-byte reads.
//
// Rows come from per-XCD partitions of the work order through atomic
// counters.  Wave 0 of a group fetches the group's next row one dependent
// load per vector phase (counter, work-order entry, list bounds, first key
// blocks) while the current row runs, and finishes the chain at once if the
// row is about to end; the result sits in LDS for the group.
//
// SPLITQ: the rows are the anchor queries of the spatial-repetition heads:
// query m < q_valid of head h is token anchor_token(m) of Q (read in place),
// O is [B, H, Lq, d] with Lq a multiple of 128, rows h*(Lq/128) + qb; keys
// still run over K and V of length L with seq_len valid.  With split_shift
// = s > 0 each row is cut into S = 2^s parts over its key blocks (part p:
// blocks [p*n/S, (p+1)*n/S) of the n = nkb_valid), work-order entries are
// row*S + p, and O is [B, H, ostride, d]: part p's normalised output rows
// from row p*Lq, then S*Lq floats of the parts' log-sum-exps (log2 units)
// for a merge pass.
template <int D, bool DENSE, bool SPLITQ, bool VT>
__global__ __launch_bounds__(512) void attn_fwd_pp_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const int32_t* __restrict__ work_order, int32_t* __restrict__ queue, int items, int H, int L,
    int seq_len, int nkb_valid, float c2, int Lq, int q_valid, int grid_rows, int grid_cols, int k_anchor,
    int split_shift, int ostride) {
  constexpr int BLK = 128;
  using G = PPGeo<D>;
  constexpr int CH = G::CH, DS = G::DS, DT = G::DT, KS = G::KS, NDMA = G::NDMA;
  constexpr int STAGE = G::STAGE, RB = G::RB;
  __shared__ u32x4 lk0[2 * G::UNITS], lk1[2 * G::UNITS], lv0[2 * G::UNITS], lv1[2 * G::UNITS];
  __shared__ u32x4 s_ost[4 * 32 * 8];   // O staging: per wave of a group 32 rows x 64 columns
  // per group: next row b, r (-1: none), list start, blocks; then kb0, kb1
  __shared__ i32x4 s_desc[2][2];
  __shared__ int s_fin[2];            // phase in which each group finished
  __shared__ i32x2 s_prev[2];         // per group: batch and row of the row whose O is due

  const int nqb = (SPLITQ ? Lq : L) / BLK;
  // SPLITQ: a work-order entry is row * 2^split_shift + part, the part
  // running over its share of the key blocks
  const int rows = (H * nqb) << (SPLITQ ? split_shift : 0);
  const int qlim = SPLITQ ? q_valid : seq_len;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wv >> 2;   // wave group
  const int w = wv & 3;      // 32-query slice of the row
  const int g = lane >> 5, c = lane & 31;
  const int prow = qk_row_perm(c);
  // K and V rows past seq_len read as zero (buffer range check)
  const uint32_t k_bytes = (uint32_t)seq_len * RB;
  const uint32_t v_bytes = VT ? (uint32_t)L * RB : (uint32_t)seq_len * RB;
  char* const kst[2] = {reinterpret_cast<char*>(lk0), reinterpret_cast<char*>(lk1)};
  char* const vst[2] = {reinterpret_cast<char*>(lv0), reinterpret_cast<char*>(lv1)};
  const int gbase = grp * STAGE;   // the group's half of each stage object

  // K stage layout (the group's half of a stage object): wave w's 1/4 holds
  // the 16-byte key chunks CPW*w .. CPW*w + CPW-1 of all 64 keys (the d
  // range of its own k-steps KPW*w ..), in NDMA row groups of RPI keys; in a
  // row group key k's CPW units sit at k*CPW, ordered by chunk XOR kswz(k),
  // so that 16 lanes reading one chunk of 16 consecutive keys meet 16
  // distinct bank groups.  Each wave fetches its own quarter, one row group
  // per DMA instruction, and starts its scores at its own k-steps: at the
  // end of a vector phase its own DMA has landed, so it can read the next
  // matrix phase's first operands before the barrier.
  constexpr int CPW = CH / 4, RPI = 64 / CPW, KPW = CPW / 2;
  auto kswz = [](int k) { return (k / (16 / CPW)) % CPW; };
  // DMA lane patterns: a K instruction writes one row group (lane l: key
  // l / CPW, unit l % CPW); a V instruction m writes LDS units 64m .. 64m+63
  // (this wave issues m = w, w+4, ...), its swizzle seeing only the lane.
  int kpat, vpat;
  {
    kpat = (lane / CPW) * RB + (((lane % CPW) ^ kswz(lane / CPW)) * 16);
    if (VT) {
      const int vrow = w * 8 + lane / 8;
      vpat = (lane / 8) * L * 2 + (((lane % 8) ^ swz<8>(vrow)) * 16);
    } else {
      const int vrow = w * (64 / CH) + lane / CH;
      vpat = (lane / CH) * RB + (((lane % CH) ^ vswz<D>(vrow)) * 16);
    }
  }
  // operand read offsets, kept in registers: the stage and tile are added as
  // the instruction's immediate offset.  K: row 32*mt + prow, unit 2s+g.
  // V (natural): lane 16G + 4jj + mm reads 8 bytes of row 16ks + 8g + 4h +
  // jj at d = 32t + 16(G%2) + 4mm; the transposed read hands lane (g, c) the
  // 4 keys of its half at d = 32t + c.  V^T: row 32t + c, unit 2ks + g.
  constexpr int NV = VT ? KS : DT;
  int koffs[DS], voffs[NV];
  {
    // score slot sl takes k-step (sl + KPW*w) mod DS: chunk 2s + g of key
    // prow (+ 32 mt, an immediate)
    const int kr = prow % RPI;
#pragma unroll
    for (int sl = 0; sl < DS; ++sl) {
      const int ch = 2 * ((sl + KPW * w) % DS) + g;
      koffs[sl] = gbase + ((ch / CPW) * NDMA + prow / RPI) * 1024 + (kr * CPW + ((ch % CPW) ^ kswz(kr))) * 16;
    }
    if (VT) {
      const int vx = g ^ swz<8>(c);
#pragma unroll
      for (int ks = 0; ks < NV; ++ks) voffs[ks] = gbase + (c * 8 + ((2 * ks) ^ vx)) * 16;
    } else {
      const int jj = (lane >> 2) & 3, mm = lane & 3;
#pragma unroll
      for (int t = 0; t < NV; ++t)
        voffs[t] = gbase + (8 * g + jj) * RB +
                   (((4 * t + 2 * (c >> 4) + (mm >> 1)) ^ vswz<D>(jj)) * 16) + (mm & 1) * 8;
    }
  }
#pragma unroll
  for (int s = 0; s < DS; ++s) asm volatile("" : "+v"(koffs[s]));
#pragma unroll
  for (int i = 0; i < NV; ++i) asm volatile("" : "+v"(voffs[i]));
  auto kread = [&](int st, int mt, int sl) __attribute__((always_inline)) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(kst[st] + koffs[sl] + mt * (32 / RPI) * 1024);
  };
  // A operand of P*V product (t, ks) from V stage st
  auto vop = [&](int st, int t, int ks) __attribute__((always_inline)) -> u32x4 {
    if (VT) return *reinterpret_cast<const u32x4*>(vst[st] + voffs[ks] + t * 32 * 8 * 16);
    const char* p = vst[st] + voffs[t] + 16 * ks * RB;
    const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr16(p));
    const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr16(p + 4 * RB));
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };

  // every stage starts as zeros: the first P*V of a group multiplies zero
  // probabilities with a V stage no tile has been loaded into yet
  for (int u = threadIdx.x; u < 2 * G::UNITS; u += 512) lk0[u] = lk1[u] = lv0[u] = lv1[u] = u32x4{0u, 0u, 0u, 0u};
  if (threadIdx.x < 2) s_fin[threadIdx.x] = 0x7fffffff;
  __syncthreads();

  // Arguments only the rare paths use (row fetch, row switch, O store) sit
  // in the lanes of one vector register: lane 2i and 2i+1 the low and high
  // word of pointer i of (Q, K, V, O, row_ptr, col_idx, work_order, queue),
  // lane 16 H, lane 17 items, lane 18 c2, lane 19 the batch entries, lanes
  // 20-28 the work order's partition offsets.  They are read with readlane where
  // needed; the register is re-declared live in every phase, so that the
  // compiler cannot hoist those reads out of the phase loop and hold their
  // results (or values derived from them) in scalar registers throughout.
  uint32_t argv = 0;
  {
    const void* const ptrs[8] = {Q, K, V, O, row_ptr, col_idx, work_order, queue};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      argv = lane == 2 * i ? (uint32_t)(uintptr_t)ptrs[i] : argv;
      argv = lane == 2 * i + 1 ? (uint32_t)((uintptr_t)ptrs[i] >> 32) : argv;
    }
    argv = lane == 16 ? (uint32_t)H : argv;
    argv = lane == 17 ? (uint32_t)items : argv;
    argv = lane == 18 ? __float_as_uint(c2) : argv;
    argv = lane == 19 ? (uint32_t)(items / rows) : argv;
    // lanes 20 .. 20+kParts: the partition offsets of the work order
    if (work_order && lane >= 20 && lane <= 20 + kParts) argv = (uint32_t)work_order[rows + lane - 20];
    // lanes 29-30: m = floor(2^40 / nqb) + 1 (low, high word), for row /
    // nqb without a division
    const uint64_t m = (1ull << 40) / (uint32_t)nqb + 1u;
    argv = lane == 29 ? (uint32_t)m : argv;
    argv = lane == 30 ? (uint32_t)(m >> 32) : argv;
    // lanes 31-32 (SPLITQ): the part shift, and the output rows per head
    if (SPLITQ) {
      argv = lane == 31 ? (uint32_t)split_shift : argv;
      argv = lane == 32 ? (uint32_t)ostride : argv;
    }
  }
  auto argw = [&](int i) __attribute__((always_inline)) -> uint32_t {
    return (uint32_t)__builtin_amdgcn_readlane((int)argv, i);
  };
  // (each half goes through uint32_t, so that a low word with bit 31 set is
  // not sign-extended into the high word)
  auto ap = [&](int i) __attribute__((always_inline)) -> uintptr_t {
    return (uintptr_t)argw(2 * i) | ((uintptr_t)argw(2 * i + 1) << 32);
  };
  auto nheads = [&]() __attribute__((always_inline)) -> int { return (int)argw(16); };
  // r / nqb for a row index r < H * nqb: (r * m) >> 40 with m =
  // floor(2^40 / nqb) + 1 is exact while r * nqb < 2^40; the host accepts
  // only B*H*L*d < 2^31 with d >= 64, so r < 2^18 and nqb < 2^18
  auto head_of = [&](int r) __attribute__((always_inline)) -> int {
    const uint64_t m = (uint64_t)argw(29) | ((uint64_t)argw(30) << 32);
    return (int)(((uint64_t)(uint32_t)r * m) >> 40);
  };
  // row and part of a work-order entry
  auto row_of = [&](int e) __attribute__((always_inline)) -> int { return SPLITQ ? e >> argw(31) : e; };
  auto part_of = [&](int e) __attribute__((always_inline)) -> int {
    return SPLITQ ? e & ((1 << argw(31)) - 1) : 0;
  };
  // first element of entry e's output rows: O is [B, H, nqb*BLK, D], or with
  // SPLITQ [B, H, ostride, D] holding part p's rows from row p*Lq
  auto o_row = [&](int b, int e) __attribute__((always_inline)) -> size_t {
    const int r = row_of(e);
    const int h = head_of(r), qb = r - h * nqb;
    if (SPLITQ)
      return (((size_t)b * nheads() + h) * (size_t)argw(32) + (size_t)part_of(e) * Lq + (size_t)qb * BLK) * D;
    return (((size_t)b * nheads() + h) * (size_t)nqb + qb) * (size_t)BLK * D;
  };

  // ---- row fetch (wave 0 of each group) ----
  // f_step: 0 done (the group's descriptor holds the next row or none),
  // 1 counter pop due, 2 pop in flight, 3 work-order entry in flight, 4 list
  // bounds in flight.  The descriptor's fields go to LDS as they become
  // known (no other wave reads it before the chain has ended and a barrier
  // has passed), and the row's first two key blocks reach it by DMA, so the
  // chain ends with the bounds step.  The partition and the partitions
  // tried live in lanes 0-1 of fstv between calls, so that no scalar
  // register holds them through the phase loop.
  int f_step = 1;
  int f_val = 0;   // result of the load in flight
  int f_pop = 0;   // result of the queue pop in flight
  int fstv = lane == 0 ? (int)(blockIdx.x % kParts) : 0;   // partition to serve first; none tried
  auto write_desc = [&](int b, int r, int beg, int n, int k0, int k1) __attribute__((always_inline)) {
    if (lane == 0) {
      s_desc[grp][0] = i32x4{b, r, beg, n};
      s_desc[grp][1] = i32x4{k0, k1, 0, 0};
    }
  };
  // an empty row is written as zeros by the fetching wave
  auto zero_row = [&](int b, int r) __attribute__((always_inline)) {
    g_u32x4* const dst = (g_u32x4*)((g_bf16*)ap(3) + o_row(b, r));
    for (int i = lane; i < BLK * D / 8; i += 64) dst[i] = u32x4{0u, 0u, 0u, 0u};
  };
  // take the result of the link in flight and issue the next; with finish,
  // run the chain to its end
  auto fetch = [&](bool finish) __attribute__((always_inline)) {
    const g_i32* const rp_ = (const g_i32*)ap(4);
    const g_i32* const wo_ = (const g_i32*)ap(6);
    g_i32* const qu_ = (g_i32*)ap(7);
    const int rows_ = nheads() * nqb;
    for (;;) {
      // The step's load: lanes 0-1 read ld[lane < lcap ? lane : 0]; the
      // queue pop is an atomic into f_pop.  One load site keeps the result
      // in one register: with a load per step the compiler copies each
      // result into a shared register, which waits for the load on the spot.
      const g_i32* ld = nullptr;
      int lcap = 0;
      bool pop = false;
      int r_known = -1;   // the row is known: its list bounds are next
      if (f_step == 1) {
        if (!qu_) {   // no queue: workgroup i serves rows 2i and 2i+1 of the order, one per group
          asm volatile("" : "+v"(fstv));
          const int item = 2 * blockIdx.x + grp;
          if (__builtin_amdgcn_readlane(fstv, 1) == 0 && item < (int)argw(17)) {
            fstv = lane == 1 ? 1 : fstv;
            const int b = item / rows_;
            const int jr = item - b * rows_;
            if (lane == 0) s_desc[grp][0][0] = b;
            if (wo_) {
              ld = wo_ + jr;
              lcap = 1;
              f_step = 3;
            } else {
              r_known = jr;
            }
          } else {
            write_desc(0, -1, 0, 0, 0, 0);
            f_step = 0;
          }
        } else {
          pop = true;
          f_step = 2;
        }
      } else if (f_step == 2) {
        asm volatile("" : "+v"(fstv));
        const int k = __builtin_amdgcn_readfirstlane(f_pop);
        int p = __builtin_amdgcn_readlane(fstv, 0);
        const int len = wo_ ? (int)argw(21 + p) - (int)argw(20 + p) : ((nheads() - p + kParts - 1) / kParts) * nqb;
        const int nb_ = (int)argw(19);   // batch entries
        if (k >= nb_ * len) {
          // this partition is drained: try the next one
          const int tries = __builtin_amdgcn_readlane(fstv, 1) + 1;
          p = (p + 1) % kParts;
          fstv = lane == 0 ? p : fstv;
          fstv = lane == 1 ? tries : fstv;
          if (tries >= kParts) {
            write_desc(0, -1, 0, 0, 0, 0);
            f_step = 0;
          } else {
            pop = true;
          }
        } else {
          const int b = nb_ > 1 ? k / len : 0;
          const int jr = k - b * len;
          if (lane == 0) s_desc[grp][0][0] = b;
          if (wo_) {
            ld = wo_ + (int)argw(20 + p) + jr;
            lcap = 1;
            f_step = 3;
          } else {
            const int hh = head_of(jr);
            r_known = (p + kParts * hh) * nqb + (jr - hh * nqb);
          }
        }
      } else if (f_step == 3) {
        r_known = __builtin_amdgcn_readfirstlane(f_val);
      } else if (f_step == 4) {
        const int beg = __builtin_amdgcn_readlane(f_val, 0);
        const int n = __builtin_amdgcn_readlane(f_val, 1) - beg;
        if (n <= 0) {
          const i32x4 d0 = s_desc[grp][0];
          zero_row(__builtin_amdgcn_readfirstlane(d0[0]), __builtin_amdgcn_readfirstlane(d0[1]));
          f_step = 1;
        } else {
          if (lane == 0) {
            s_desc[grp][0][2] = beg;
            s_desc[grp][0][3] = n;
          }
          // the first two key blocks (the first twice for a one-block row)
          // go by DMA into the descriptor's second vector, lanes 0 and 1
          if (lane < 2)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(reinterpret_cast<const void*>(ap(5) + (uintptr_t)beg * 4), 0xffffffffu),
                                                     (lds_void*)&s_desc[grp][1], 4, (lane < n ? lane : 0) * 4, 0,
                                                     0, 0);
          f_step = 0;
        }
      }
      if (r_known >= 0) {
        if (DENSE) {
          // (SPLITQ: part p runs over key blocks [p*n/S, (p+1)*n/S))
          const int sh = SPLITQ ? (int)argw(31) : 0;
          const int pt = SPLITQ ? r_known & ((1 << sh) - 1) : 0;
          const int kb_b = (pt * nkb_valid) >> sh, kb_e = ((pt + 1) * nkb_valid) >> sh;
          if (lane == 0) s_desc[grp][0] = i32x4{s_desc[grp][0][0], r_known, kb_b, kb_e - kb_b};
          if (lane == 0) s_desc[grp][1] = i32x4{kb_b, kb_e - kb_b > 1 ? kb_b + 1 : kb_b, 0, 0};
          f_step = 0;
        } else {
          if (lane == 0) s_desc[grp][0][1] = r_known;
          ld = rp_ + r_known;
          lcap = 2;
          f_step = 4;
        }
      }
      if (pop && lane == 0) {
        asm volatile("" : "+v"(fstv));
        f_pop = __hip_atomic_fetch_add(qu_ + __builtin_amdgcn_readlane(fstv, 0) * kQueueStride, 1,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (ld && lane < 2) f_val = ld[lane < lcap ? lane : 0];
      if (f_step == 0 || !finish) break;
      if (f_step != 1) wait_vm();
    }
  };

  // ---- the group's row state ----
  // (flags are ints: wave-uniform values the compiler keeps in scalar
  // registers, not per-lane masks)
  bool cur = false;    // a row is being computed (S side)
  int cb = 0, cr = 0, cbeg = 0, cnb = 0, cn = 0, j = 0;   // batch, row, list start, blocks, sub-tiles, sub-tile
  int kb0 = 0, kb1 = 0;         // key blocks of the current and the next block
  int cbase = 0, ck_cur = 0, ck_nxt = 0;   // readlane window over the row's list
  __amdgpu_buffer_rsrc_t rk = make_rsrc(K, 0), rv = make_rsrc(V, 0);
  bool pend = false;   // the previous row's O is due (after its last P*V); its row in s_prev
  float l_fin = 0.f;
  bool nxt = false;    // at a row's end: a next row is in the group's descriptor

  auto chunk_load = [&](int beg, int nblk, int cix) __attribute__((always_inline)) -> int {
    int i = 64 * cix + lane;
    i = i < nblk ? i : nblk - 1;
    return ((const g_i32*)ap(5))[beg + i];
  };
  // key block i of the current row (i grows by one per call, clamped to the row)
  auto blk_at = [&](int i) __attribute__((always_inline)) -> int {
    i = i < cnb ? i : cnb - 1;
    if (DENSE) return SPLITQ ? cbeg + i : i;
    const bool adv = (i >> 6) != cbase;
    if (adv) {
      ++cbase;
      ck_cur = ck_nxt;
    }
    const int v = __builtin_amdgcn_readlane(ck_cur, i & 63);
    if (adv) ck_nxt = chunk_load(cbeg, cnb, cbase + 1);
    return v;
  };
  auto set_row = [&](int b, int r, int beg, int nblk, int k0, int k1) __attribute__((always_inline)) {
    cb = b;
    cr = r;
    cbeg = beg;
    cnb = nblk;
    cn = 2 * nblk;
    j = 0;
    kb0 = k0;
    kb1 = k1;
    cbase = 0;
    const int h = head_of(row_of(r));
    const size_t base = ((size_t)b * nheads() + h) * (size_t)L * D;
    rk = make_rsrc((const bf16*)ap(1) + base, k_bytes);
    rv = make_rsrc((const bf16*)ap(2) + base, v_bytes);
  };
  // this lane's Q row of row (b, r): 8 consecutive d per k-step, raw bf16.
  // A padded query (q >= seq_len) is taken as zero, so that whatever the
  // padding holds its lane computes exactly what zero padding gives (its
  // output is zeroed anyway, but a non-finite value would also move the
  // wave's shared rescale decisions).
  auto q_load = [&](int b, int e, bf16x8* qr) __attribute__((always_inline)) {
    const int r = row_of(e);
    const int h = head_of(r), qb = r - h * nqb;
    const int q = qb * BLK + 32 * w + c;
    const int qsrc = SPLITQ ? (q < q_valid ? anchor_token(q, grid_rows, grid_cols, k_anchor) : 0) : q;
    const g_bf16* src = (const g_bf16*)ap(0) + ((size_t)b * nheads() + h) * (size_t)L * D + (size_t)qsrc * D + 8 * g;
    const bool live = SPLITQ || q < seq_len;
    // in this wave's k-step order (slot s holds k-step (s + KPW*w) mod DS)
#pragma unroll
    for (int s = 0; s < DS; ++s) qr[s] = live ? *(const g_bf16x8*)(src + 16 * ((s + KPW * w) % DS)) : bf16x8{};
  };

  // the row's Q: raw bf16 from the load until it is scaled in place
  bf16x8 qreg[DS];
  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  // Q is scaled by c2 (the softmax scale in log2 units) on loading and
  // rounded to bf16, so that the products give scores in log2 units and,
  // with the accumulators started at -ref, exp2 needs no vector arithmetic
  // before it
  auto q_scale = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < DS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qreg[s][e] = (bf16)((float)qreg[s][e] * __uint_as_float(argw(18)));
  };
  // the group's reference (log2 units) and row sum; fresh until the
  // reference has been set from the maximum of a sub-tile with valid keys
  float ref = 0.f, l_run = 0.f;
  bool fresh = true;
  f32x16 cneg = {};   // -ref in every accumulator register
  f32x16 sacc[2];
  bf16x8 pb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) pb[ks] = bf16x8{};
  bool rescale = false;   // O *= alpha is due before the next P*V
  float alpha = 1.f;

  // ---- prologue: each group's first row, its K(0) tile and Q ----
  // the group's descriptor, read as two vectors (one LDS round trip)
  auto row_desc = [&](int* v) __attribute__((always_inline)) {
    const i32x4 d0 = s_desc[grp][0], d1 = s_desc[grp][1];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __builtin_amdgcn_readfirstlane(d0[i]);
    v[4] = __builtin_amdgcn_readfirstlane(d1[0]);
    v[5] = __builtin_amdgcn_readfirstlane(d1[1]);
  };
  if (w == 0) {
    fetch(true);
    wait_vm();   // the descriptor's key blocks arrive by DMA
  }
  __syncthreads();
  {
    int dv[6];
    row_desc(dv);
    if (dv[1] >= 0) {
      set_row(dv[0], dv[1], dv[2], dv[3], dv[4], dv[5]);
      if (!DENSE) {
        ck_cur = chunk_load(cbeg, cnb, 0);
        ck_nxt = chunk_load(cbeg, cnb, 1);
      }
#pragma unroll
      for (int i = 0; i < NDMA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kst[0] + gbase + (w * NDMA + i) * 1024), 16, kpat,
                                                 (kb0 * BLK + i * RPI) * RB + w * CPW * 16, 0, 0);
      q_load(cb, cr, qreg);
      cur = true;
      f_step = 1;
    } else {
      f_step = 0;
      if (w == 0 && lane == 0) s_fin[grp] = -1;
    }
    wait_vm();
    if (cur) q_scale();
  }
  __syncthreads();
  if (s_fin[0] < 0 && s_fin[1] < 0) return;
  int done = !cur;   // the group has finished (read through readfirstlane: uniform)

  // operand ring of a matrix phase (each slot's pair read PF slots ahead);
  // its first NPRE slots read this wave's own quarter of the K stage and are
  // read before the phase, at the end of the vector phase before it (or
  // here), once the wave's own DMA has landed
  constexpr int PF = 2, NPRE = PF < KPW ? PF : KPW;
  u32x4 ra[PF + 1][2];
  auto pre_read = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int sl = 0; sl < NPRE; ++sl) {
      ra[sl][0] = kread(st, 0, sl);
      ra[sl][1] = kread(st, 1, sl);
    }
  };
  if (cur) pre_read(0);

  // matrix phase of stream cycle x (TM = x % 2 fixes the stages)
  auto mphase = [&](auto tmc) __attribute__((always_inline)) {
    constexpr int TM = decltype(tmc)::value;
    asm volatile("" : "+v"(argv));
    if (__builtin_expect(!cur && !pend, 0)) {
      lds_barrier();
      return;
    }
    // O moves to the reference P(x-1) was computed against
    if (__builtin_expect(rescale, 0)) {
#pragma unroll
      for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
      rescale = false;
    }
    // K(x+1): the second half of this block, the next block, or at the end
    // of a row the next row's first block; V(x): this sub-tile
    int kd = TM == 0 ? kb0 * BLK + 64 : kb1 * BLK;
    __amdgpu_buffer_rsrc_t rkd = rk;
    const bool last = TM == 1 && cur && j == cn - 1;
    int nb = 0, nr = 0;
    if (__builtin_expect(last, 0)) {
      int dv[6];
      row_desc(dv);
      nr = dv[1];
      nxt = nr >= 0;
      if (nxt) {
        nb = dv[0];
        rkd = make_rsrc((const bf16*)ap(1) + ((size_t)nb * nheads() + head_of(row_of(nr))) * (size_t)L * D, k_bytes);
        kd = dv[4] * BLK;
        // the current row's list is not read past this point
        if (!DENSE) {
          ck_cur = chunk_load(dv[2], dv[3], 0);
          ck_nxt = chunk_load(dv[2], dv[3], 1);
        }
      }
    }
    const int vd = kb0 * BLK + TM * 64;
    // this wave's first DMA destination in its group's half of a stage,
    // re-formed in every phase so that the destinations (one per stage and
    // instruction) are not all kept in scalar registers through the loop
    int wq, wdst;
    asm volatile("s_mov_b32 %0, %1" : "=s"(wq) : "s"(w));
    asm volatile("s_mov_b32 %0, %1" : "=s"(wdst) : "s"(gbase));
    const int kdst = wdst + wq * NDMA * 1024;
    wdst += wq * 1024;
    auto dma_share = [&](int s) __attribute__((always_inline)) {
#pragma unroll
      for (int i = s * 2 * NDMA / DS; i < (s + 1) * 2 * NDMA / DS; ++i) {
        const int m = wq + 4 * (i % NDMA);
        if (i < NDMA) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rkd, (lds_void*)(kst[TM ^ 1] + kdst + 1024 * i), 16,
                                                   kpat, (kd + i * RPI) * RB + wq * CPW * 16, 0, 0);
        } else {
          const int soff = VT ? vd * 2 + m * 16 * L : vd * RB + m * 1024;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vst[TM] + wdst + 4096 * (i - NDMA)), 16,
                                                   vpat, soff, 0, 0);
        }
      }
    };
    __builtin_amdgcn_s_setprio(2);
    // S(x) and P*V(x-1) run as one sequence of slots, each one pair of
    // products and the operand reads of the slot PF ahead
    constexpr int NSL = DS + DT * KS / 2;
    auto rd = [&](int sl, int h) __attribute__((always_inline)) -> u32x4 {
      if (sl < DS) return kread(TM, h, sl);
      const int i = 2 * (sl - DS) + h;
      return vop(TM ^ 1, i % DT, i / DT);
    };
#pragma unroll
    for (int sl = NPRE; sl < PF; ++sl) {
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
        // past the row's last scores its Q is dead: load the next row's
        if (TM == 1 && sl == DS - 1 && __builtin_expect(last && nxt, 0)) q_load(nb, nr, qreg);
      } else {
        const int i0 = 2 * (sl - DS), i1 = i0 + 1;
        oacc[i0 % DT] = mfma_bf16(a0, pb[i0 / DT], oacc[i0 % DT]);
        oacc[i1 % DT] = mfma_bf16(a1, pb[i1 / DT], oacc[i1 % DT]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    lds_barrier();
  };

  // vector phase of stream cycle x; gp is the global phase index
  auto vphase = [&](auto tmc, int gp) __attribute__((always_inline)) {
    constexpr int TM = decltype(tmc)::value;
    asm volatile("" : "+v"(argv));
    if (__builtin_expect(!cur && !pend, 0)) {
      // (nothing is in flight here; the wait tells the compiler so, which
      // keeps it from waiting for the DMA of a later phase before the LDS
      // accesses of the next)
      wait_vm();
      lds_barrier();
      return;
    }
    if (__builtin_expect(pend, 0)) {
      // the previous row's last P*V ran in the matrix phase just ended: O =
      // acc / l; padded query rows (and rows that saw no key) are zero.
      // In the accumulator layout a lane holds 8-byte pieces of one query's
      // row, so a direct store would touch 32 rows with 16 bytes each.  The
      // wave's 32 x D tile goes out through LDS instead, 64 columns at a
      // time, and each store writes whole 128-byte lines.  The staging
      // buffer is an LDS object of its own, which no DMA ever writes, so its
      // accesses need no wait for the tiles in flight.
      const i32x2 pv = s_prev[grp];
      const int pb = __builtin_amdgcn_readfirstlane(pv[0]);
      const int pr = __builtin_amdgcn_readfirstlane(pv[1]);
      const float l_tot = pair_sum(l_fin);
      const int prr = row_of(pr);
      const int q = (prr - head_of(prr) * nqb) * BLK + 32 * w + c;
      const bool valid = q < qlim && l_tot > 0.f;
      const float inv = valid ? 1.f / l_tot : 0.f;
      char* const stg = reinterpret_cast<char*>(s_ost) + w * (32 * 128);
      g_bf16* const Ob = (g_bf16*)ap(3) + o_row(pb, pr) + (size_t)(32 * w) * D;
#pragma unroll
      for (int hr = 0; hr < DT / 2; ++hr) {
        // lane (g, c) holds query c, d = 32t + 8rq + 4g + e: 8-byte pieces of
        // the staged row's 16-byte units 4(t - 2hr) + rq, the unit index
        // XORed with c % 8
#pragma unroll
        for (int t = 2 * hr; t < 2 * hr + 2; ++t) {
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = valid ? oacc[t][4 * rq + e] * inv : 0.f;
            *reinterpret_cast<bf16x4*>(stg + c * 128 + (((4 * (t - 2 * hr) + rq) ^ (c & 7)) * 16) + 8 * g) =
                __builtin_convertvector(x, bf16x4);
          }
          oacc[t] = f32x16{};
        }
        // read back: lane L takes unit L % 8 of row L / 8 (+ 8 rows per
        // instruction), 64 columns of each row
#pragma unroll 2
        for (int i = 0; i < 4; ++i) {
          const int row = 8 * i + lane / 8, u = lane % 8;
          const u32x4 v = *reinterpret_cast<const u32x4*>(stg + row * 128 + ((u ^ (row & 7)) * 16));
          *(g_u32x4*)(Ob + (size_t)row * D + 64 * hr + 8 * u) = v;
        }
      }
      pend = false;
      if (!cur) {
        done = 1;
        s_fin[grp] = gp;   // every lane of the group writes the same value
      }
    }
    if (__builtin_expect(cur, 1)) {
      const int k0 = kb0 * BLK + TM * 64;
      if (__builtin_expect(k0 + 64 > seq_len, 0)) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            if (k0 + 32 * mt + slice_key(rr, g) >= seq_len) sacc[mt][rr] = kNegInf;
      }
      // P rounded to bf16 for the products; its row sums in fp32 from the
      // unrounded values, in four chains (plain adds run beside the other
      // wave's matrix products far better than dot2 does)
      float ls[2] = {0.f, 0.f};
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
      // the reference moves to the row maximum on the first sub-tile with
      // valid keys, and later only when a lane's sum passes kSumCap
      bool redo = fresh && k0 < seq_len;
      if (__builtin_expect(!redo, 1)) {
        probs();
        redo = __any(!(ls[0] + ls[1] <= kSumCap));
      }
      if (__builtin_expect(redo, 0)) {
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
        probs();
      }
      l_run += ls[0] + ls[1];

      if (__builtin_expect(w == 0 && f_step != 0, 0)) fetch(j >= cn - 2);

      if (TM == 1 && __builtin_expect(j == cn - 1, 0)) {
        // the row's last sub-tile: its O is written after the next P*V.
        // Every wave of the group writes the same row to s_prev; it is read
        // in the next phase, after the barrier.
        l_fin = l_run;
        s_prev[grp] = i32x2{cb, cr};
        pend = true;
        if (SPLITQ && argw(31) != 0) {
          // a part's log-sum-exp (log2 units) for the merge of the parts:
          // floats after the 2^shift parts' rows of the head's output rows
          const float lt = pair_sum(l_run);
          const int r = row_of(cr), h = head_of(r);
          const int q = (r - h * nqb) * BLK + 32 * w + c;
          g_f32* const lse = reinterpret_cast<g_f32*>(
              (g_bf16*)ap(3) + (((size_t)cb * nheads() + h) * (size_t)argw(32) + ((size_t)Lq << argw(31))) * D);
          if (g == 0) lse[(size_t)part_of(cr) * Lq + q] = lt > 0.f ? ref + __log2f(lt) : kNegInf;
        }
        if (nxt) {
          int dv[6];
          row_desc(dv);
          set_row(dv[0], dv[1], dv[2], dv[3], dv[4], dv[5]);
          ref = 0.f;
          l_run = 0.f;
          fresh = true;
          cneg = f32x16{};
          wait_vm();
          q_scale();
          f_step = 1;
        } else {
          cur = false;
        }
      } else {
        ++j;
        if (TM == 1) {
          kb0 = kb1;
          kb1 = blk_at(j / 2 + 1);
        }
      }
    }
    wait_vm();
    if (__builtin_expect(cur, 1)) pre_read(TM ^ 1);
    lds_barrier();
  };

  // a finished group meets barriers until the other one has finished too;
  // both decide from values written before the same barrier
  int gp = 0;
  auto stop = [&](int p) __attribute__((always_inline)) -> bool {
    return __builtin_expect(__builtin_amdgcn_readfirstlane(done), 0) &&
           __builtin_amdgcn_readfirstlane(s_fin[grp ^ 1]) <= p;
  };
  if (grp == 1) {
    lds_barrier();
    if (stop(gp)) return;
    ++gp;
  }
  for (;;) {
    mphase(Cst<0>{});
    if (stop(gp)) break;
    ++gp;
    vphase(Cst<0>{}, gp);
    if (stop(gp)) break;
    ++gp;
    mphase(Cst<1>{});
    if (stop(gp)) break;
    ++gp;
    vphase(Cst<1>{}, gp);
    if (stop(gp)) break;
    ++gp;
  }
}

// float32 path: 32-key slices, fp32 matrix cores (32x32x2), P kept in float32.
// Lane (g, c) holds, for slice accumulator register r, key 2r + g (rows of
// the K slice are fed in that order), which is the B layout of P^T.
template <int D, int BLK, bool DENSE, bool VT>
__global__ __launch_bounds__(BLK * 2) void attn_fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
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

    float qreg[D / 2];   // a padded query is taken as zero
#pragma unroll
    for (int s = 0; s < D / 2; ++s) qreg[s] = q < seq_len ? Q[base + (size_t)q * D + 2 * s + g] : 0.f;

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
          if (VT) {
            const int vk = i % 32, vd = i / 32;   // V^T row vd, 32 consecutive keys
            ldsV[vk * KP + vd] = V[base + (size_t)vd * L + k0 + vk];
          } else {
            // padded keys meet zero probabilities: their V rows are taken as 0
            ldsV[kr * KP + dd] = k0 + kr < seq_len ? V[base + (size_t)(k0 + kr) * D + dd] : 0.f;
          }
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
    const bool valid = q < seq_len && l_tot > 0.f;
    const float inv = valid ? 1.f / l_tot : 0.f;
    float* Ob = O + base + (size_t)q * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr)
        Ob[32 * t + 8 * (rr >> 2) + 4 * g + (rr & 3)] = valid ? oacc[t][rr] * inv : 0.f;
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

template <int D, bool DENSE, bool SPLITQ, bool VT>
static hipError_t launch_pp(const AttnArgs& a, hipStream_t st) {
  const int Lq = SPLITQ ? a.Lq : a.L;
  const int items = (a.B * a.H * (Lq / 128)) << (SPLITQ ? a.split_shift : 0);
  const float c2 = a.scale * kLog2e;
  if (items == 0) return hipSuccess;
  // two rows in flight per workgroup (one per wave group)
  int grid = (items + 1) / 2;
  if (a.queue) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(kQueueInts), 0, st, a.queue, kQueueInts, 0);
    int per_cu = 1;
    hipError_t e = occupancy(attn_fwd_pp_kernel<D, DENSE, SPLITQ, VT>, 512, &per_cu);
    if (e != hipSuccess) return e;
    const long long cap = (long long)a.num_cu * (per_cu > 0 ? per_cu : 1);
    grid = (int)(cap < grid ? cap : grid);
  }
  hipLaunchKernelGGL((attn_fwd_pp_kernel<D, DENSE, SPLITQ, VT>), dim3(grid), dim3(512), 0, st, (const bf16*)a.Q,
                     (const bf16*)a.K, (const bf16*)a.V, (bf16*)a.O, a.row_ptr, a.col_idx, a.work_order, a.queue,
                     items, a.H, a.L, a.seq_len, a.nkb_valid, c2, Lq, SPLITQ ? a.q_valid : a.seq_len,
                     a.grid_rows, a.grid_cols, a.k_anchor, SPLITQ ? a.split_shift : 0,
                     SPLITQ && a.ostride > 0 ? a.ostride : Lq);
  return hipGetLastError();
}

hipError_t launch_anchor_attention(const AttnArgs& a, hipStream_t st) {
  if (a.dtype_f32 || a.block != 128 || !a.work_order || !a.queue) return hipErrorInvalidValue;
  if (a.d == 128)
    return a.v_transposed ? launch_pp<128, true, true, true>(a, st) : launch_pp<128, true, true, false>(a, st);
  return a.v_transposed ? launch_pp<64, true, true, true>(a, st) : launch_pp<64, true, true, false>(a, st);
}

template <int D, int BLK, bool DENSE, bool VT>
static hipError_t launch_typed(const AttnArgs& a, hipStream_t st) {
  if (BLK == 128 && !a.dtype_f32) return launch_pp<D, DENSE, false, VT>(a, st);
  const int threads = BLK * 2;
  const int items = a.B * a.H * (a.L / BLK);
  const float c2 = a.scale * kLog2e;
  if (items == 0) return hipSuccess;
  int grid = items;
  if (a.queue) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(kQueueInts), 0, st, a.queue, kQueueInts, 0);
    int per_cu = 1;
    hipError_t e = a.dtype_f32
        ? occupancy(attn_fwd_f32_kernel<D, BLK, DENSE, VT>, threads, &per_cu)
        : occupancy(attn_fwd_bf16_kernel<D, BLK, DENSE, VT>, threads, &per_cu);
    if (e != hipSuccess) return e;
    const long long cap = (long long)a.num_cu * (per_cu > 0 ? per_cu : 1);
    grid = (int)(cap < items ? cap : items);
  }
  if (a.dtype_f32) {
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D, BLK, DENSE, VT>), dim3(grid), dim3(threads), 0, st,
                       (const float*)a.Q, (const float*)a.K, (const float*)a.V, (float*)a.O,
                       a.row_ptr, a.col_idx, a.work_order, a.queue, items, a.H, a.L, a.seq_len,
                       a.nkb_valid, c2);
  } else {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, BLK, DENSE, VT>), dim3(grid), dim3(threads), 0, st,
                       (const bf16*)a.Q, (const bf16*)a.K, (const bf16*)a.V, (bf16*)a.O, a.row_ptr,
                       a.col_idx, a.work_order, a.queue, items, a.H, a.L, a.seq_len, a.nkb_valid, c2);
  }
  return hipGetLastError();
}

template <bool DENSE, bool VT>
static hipError_t dispatch(const AttnArgs& a, hipStream_t st) {
  if (a.d == 128 && a.block == 128) return launch_typed<128, 128, DENSE, VT>(a, st);
  if (a.d == 128 && a.block == 64) return launch_typed<128, 64, DENSE, VT>(a, st);
  if (a.d == 64 && a.block == 128) return launch_typed<64, 128, DENSE, VT>(a, st);
  return launch_typed<64, 64, DENSE, VT>(a, st);
}

hipError_t launch_attention(const AttnArgs& a, bool dense, hipStream_t st) {
  if (a.v_transposed) return dense ? dispatch<true, true>(a, st) : dispatch<false, true>(a, st);
  return dense ? dispatch<true, false>(a, st) : dispatch<false, false>(a, st);
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
