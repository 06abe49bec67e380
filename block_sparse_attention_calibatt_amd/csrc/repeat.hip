// Spatial-repetition heads on gfx950: the similarity score that selects
// them, and the anchor-row forward that runs them.
//
// Pages: Fig. 4 caption (in some heads a query frame's attention pattern
// repeats from one spatial row to the next), Fig. 5(b) caption (such heads
// compute attention for a few anchor rows per frame and hand the outputs to
// the neighbouring rows), Fig. 6 and Fig. S13 captions (one similarity score
// per map, heads above tau), Table S4 (anchors attend to all keys; 1 - k/30
// of the query rows are skipped).
//
// Token layout: token n < seq_len sits at frame f, spatial row y, column x of
// a (frames, rows, cols) grid with n = (f*rows + y)*cols + x.  The rows of a
// frame form k contiguous groups [floor(g*rows/k), floor((g+1)*rows/k)),
// anchored at their lower middle row.
//
// Similarity (spatial_sim_kernel): for each token with a row below it in the
// same frame, the cosine of the two tokens' softmax rows,
//     sum_j p_ij p_i'j / sqrt(sum_j p_ij^2 * sum_j p_i'j^2),  i' = i + cols,
// with p = exp(s - lse) from the row log-sum-exp pass of the pooling code.
// Both score tiles come from the matrix cores with the same lane layout, so
// the products are lane-local.  Each workgroup adds its 128 cosines in a
// fixed order in float64; a second kernel adds the workgroup partials in
// order, so the score is bitwise reproducible.
//
// Anchor forward: the persistent dense kernel runs over the anchor queries
// of the listed heads in its split-query mode (each query read in place
// through the anchor map; keys: the full K and V) into a [B, H, Lq, d]
// buffer (Lq = anchor count rounded up to 128), and every token's output
// row is then copied from its anchor's.  When the anchor rows are too few
// for the device's wave groups, each row is cut into parts over its key
// blocks, and a merge of the parts by their log-sum-exps comes first.
#include "tiles.h"
#include "launch.h"

namespace calibatt {

namespace {

// Index of the anchor query whose output token n takes (n < seq_len).
__device__ __forceinline__ int source_anchor(int n, int R, int C, int k) {
  const int RC = R * C;
  const int f = n / RC, rem = n - f * RC;
  const int y = rem / C, x = rem - y * C;
  const int g = ((y + 1) * k - 1) / R;   // the group g with lo_g <= y < lo_{g+1}
  return (f * k + g) * C + x;
}

// U = D*sizeof(T)/16 lanes copy one output row, 16 bytes each, so a wave's
// load or store covers 64/U consecutive rows (tokens next to each other in
// a grid row take anchors next to each other too: both sides stay
// contiguous).  A workgroup copies BC_PASSES groups of 256/U rows, its
// loads all issued before its stores.  grid.y enumerates the (batch entry,
// listed head) pairs, so the index arithmetic stays in 32 bits.
constexpr int BC_PASSES = 4;
template <typename T, int D>
__global__ __launch_bounds__(256) void anchor_broadcast_kernel(const T* __restrict__ Oa, T* __restrict__ O,
                                                               HeadList hl, int H, int L, int Lq, int seq_len,
                                                               int R, int C, int k) {
  constexpr int U = D * (int)sizeof(T) / 16;   // 16-byte units per row
  constexpr int RPP = 256 / U;                 // rows per pass
  const int u = threadIdx.x % U, rr = threadIdx.x / U;
  const int row0 = blockIdx.x * (RPP * BC_PASSES) + rr;
  const int slot = blockIdx.y % hl.n, b = blockIdx.y / hl.n;
  const size_t bh = (size_t)b * H + hl.h[slot];
  u32x4 v[BC_PASSES];
#pragma unroll
  for (int p = 0; p < BC_PASSES; ++p) {
    const int n = row0 + p * RPP;
    v[p] = u32x4{0u, 0u, 0u, 0u};
    if (n < seq_len) v[p] = reinterpret_cast<const u32x4*>(Oa + (bh * Lq + source_anchor(n, R, C, k)) * D)[u];
  }
#pragma unroll
  for (int p = 0; p < BC_PASSES; ++p) {
    const int n = row0 + p * RPP;
    if (n < L) reinterpret_cast<u32x4*>(O + (bh * L + n) * D)[u] = v[p];
  }
}

// Work order for the anchor rows: listed head i goes to partition i % 8,
// its entries (row*S + part) part by part, rows in order within a part, so
// that the rows in flight read the same key range; the partition offsets
// follow the H*nqb*S entry slots.
__global__ __launch_bounds__(256) void anchor_order_kernel(HeadList hl, int H, int nqb, int sh,
                                                           int32_t* __restrict__ order) {
  const int S = 1 << sh;
  const int per_head = nqb * S;
  const int slots = (H * nqb) << sh;
  auto part_heads = [&](int p) { return p < hl.n ? (hl.n - p + kParts - 1) / kParts : 0; };
  for (int i = threadIdx.x; i < hl.n * per_head; i += 256) {
    const int slot = i / per_head, rem = i - slot * per_head;
    const int pt = rem / nqb, qb = rem - pt * nqb;
    const int p = slot % kParts, j = slot / kParts;
    int off = 0;
    for (int q = 0; q < p; ++q) off += part_heads(q) * per_head;
    order[off + j * per_head + rem] = ((hl.h[slot] * nqb + qb) << sh) + pt;
  }
  if (threadIdx.x == 0) {
    int off = 0;
    for (int p = 0; p <= kParts; ++p) {
      order[slots + p] = off;
      if (p < kParts) off += part_heads(p) * per_head;
    }
  }
}

// Merge of the S = 2^sh parts of the anchor rows: for anchor query m < La of
// listed head h, with part p's normalised output o_p and log-sum-exp l_p
// (log2 units), O = sum_p 2^(l_p - l_max) o_p / sum_p 2^(l_p - l_max), the
// softmax over all keys recombined from its key ranges.  The parts sit in
// the head's rows of the final output (rows p*Lq .., then S*Lq floats of
// l_p); the merged rows go to Oa [B, H, Lq, D].  U lanes per row, 16 bytes
// (8 elements) each.
template <int D>
__global__ __launch_bounds__(256) void anchor_merge_kernel(const bf16* __restrict__ Op, bf16* __restrict__ Oa,
                                                           HeadList hl, int H, int L, int Lq, int La, int sh) {
  constexpr int U = D * 2 / 16;
  const int u = threadIdx.x % U;
  const int m = blockIdx.x * (256 / U) + threadIdx.x / U;
  const int slot = blockIdx.y % hl.n, b = blockIdx.y / hl.n;
  if (m >= La) return;
  const size_t bh = (size_t)b * H + hl.h[slot];
  const bf16* const base = Op + bh * L * D;
  const float* const lse = reinterpret_cast<const float*>(base + ((size_t)Lq << sh) * D);
  const int S = 1 << sh;
  float mx = kNegInf;
  for (int p = 0; p < S; ++p) mx = fmaxf(mx, lse[(size_t)p * Lq + m]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mx > kNegInf) {
    for (int p = 0; p < S; ++p) {
      const float wp = fast_exp2(lse[(size_t)p * Lq + m] - mx);
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(base + ((size_t)p * Lq + m) * D + 8 * u);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wp * (float)x[e];
      wsum += wp;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  bf16x8 y;
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = (bf16)(acc[e] * inv);
  *reinterpret_cast<bf16x8*>(Oa + (bh * Lq + m) * D + 8 * u) = y;
}

template <int D>
__global__ __launch_bounds__(256) void spatial_sim_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                                          const float* __restrict__ lse,
                                                          double* __restrict__ part, int L, int seq_len,
                                                          int nkb_valid, int C, int RC, float c2) {
  constexpr int BLK = 128, DS = D / 16, CH = D / 8;
  __shared__ u32x4 ldsK[BLK * D / 8];
  __shared__ double wsum[4];
  const int nqb = L / BLK;
  const int item = blockIdx.x;
  const int bh = item / nqb, qt = item - bh * nqb;
  const size_t base = (size_t)bh * L * D;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 5, c = lane & 31;
  const int q = qt * BLK + 32 * w + c;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + base, (uint32_t)L * D * 2);
  // a token counts when the row below it lies in the same frame
  const bool prim = q < seq_len && (q % RC) < RC - C;
  const int q2 = prim ? q + C : q;
  const float l1 = prim ? lse[(size_t)bh * L + q] * kLog2e : 0.f;
  const float l2 = prim ? lse[(size_t)bh * L + q2] * kLog2e : 0.f;

  bf16x8 qa[DS], qb2[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    qa[s] = *reinterpret_cast<const bf16x8*>(Q + base + (size_t)q * D + 16 * s + 8 * g);
    qb2[s] = *reinterpret_cast<const bf16x8*>(Q + base + (size_t)q2 * D + 16 * s + 8 * g);
  }
  const int prow = qk_row_perm(c);
  float dot = 0.f, n1 = 0.f, n2 = 0.f;
  for (int kb = 0; kb < nkb_valid; ++kb) {
    __syncthreads();
    dma_k_tile<D, BLK>(rk, kb * BLK, ldsK, wu, lane);
    wait_vm_all();
    __syncthreads();
    const int k0 = kb * BLK;
#pragma unroll
    for (int mt = 0; mt < BLK / 32; ++mt) {
      f32x16 s1 = {}, s2 = {};
      const int row = 32 * mt + prow;
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, ldsK[chunk_index<CH>(row, 2 * s + g)]);
        s1 = mfma_bf16(a, qa[s], s1);
        s2 = mfma_bf16(a, qb2[s], s2);
      }
      if (k0 + BLK > seq_len) {   // the tile holding the padded keys
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const bool kv = k0 + 32 * mt + slice_key(rr, g) < seq_len;
          const float p1 = kv ? fast_exp2(fmaf(s1[rr], c2, -l1)) : 0.f;
          const float p2 = kv ? fast_exp2(fmaf(s2[rr], c2, -l2)) : 0.f;
          dot = fmaf(p1, p2, dot);
          n1 = fmaf(p1, p1, n1);
          n2 = fmaf(p2, p2, n2);
        }
      } else {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const float p1 = fast_exp2(fmaf(s1[rr], c2, -l1));
          const float p2 = fast_exp2(fmaf(s2[rr], c2, -l2));
          dot = fmaf(p1, p2, dot);
          n1 = fmaf(p1, p1, n1);
          n2 = fmaf(p2, p2, n2);
        }
      }
    }
  }
  dot = pair_sum(dot);
  n1 = pair_sum(n1);
  n2 = pair_sum(n2);
  double cs = (prim && g == 0) ? (double)(dot / sqrtf(n1 * n2)) : 0.0;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cs += __shfl_xor(cs, off);
  if (lane == 0) wsum[w] = cs;
  __syncthreads();
  if (threadIdx.x == 0) part[item] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
}

__global__ __launch_bounds__(64) void spatial_sim_reduce_kernel(const double* __restrict__ part, int BH, int nqb,
                                                                double inv_pairs, double* __restrict__ sim) {
  const int bh = blockIdx.x * 64 + threadIdx.x;
  if (bh >= BH) return;
  double s = 0.0;
  for (int i = 0; i < nqb; ++i) s += part[(size_t)bh * nqb + i];
  sim[bh] = s * inv_pairs;
}

}  // namespace

hipError_t launch_spatial_similarity(const SimArgs& a, hipStream_t st) {
  MassArgs m;
  m.Q = a.Q;
  m.K = a.K;
  m.lse = a.lse;
  m.mass = nullptr;
  m.B = a.B;
  m.H = a.H;
  m.L = a.L;
  m.seq_len = a.seq_len;
  m.d = a.d;
  m.block = 128;
  m.nkb_valid = (a.seq_len + 127) / 128;
  m.scale = a.scale;
  const float* lse = a.lse_in;
  if (!lse) {
    hipError_t e0 = launch_row_lse(m, st);
    if (e0 != hipSuccess) return e0;
    lse = a.lse;
  }
  hipError_t e;
  const int nqb = a.L / 128;
  const int items = a.B * a.H * nqb;
  const float c2 = a.scale * kLog2e;
  if (a.d == 128)
    hipLaunchKernelGGL((spatial_sim_kernel<128>), dim3(items), dim3(256), 0, st, (const bf16*)a.Q,
                       (const bf16*)a.K, lse, a.part, a.L, a.seq_len, m.nkb_valid, a.cols, a.rows * a.cols, c2);
  else
    hipLaunchKernelGGL((spatial_sim_kernel<64>), dim3(items), dim3(256), 0, st, (const bf16*)a.Q,
                       (const bf16*)a.K, lse, a.part, a.L, a.seq_len, m.nkb_valid, a.cols, a.rows * a.cols, c2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const double pairs = (double)a.frames * (a.rows - 1) * a.cols;
  hipLaunchKernelGGL(spatial_sim_reduce_kernel, dim3((a.B * a.H + 63) / 64), dim3(64), 0, st,
                     (const double*)a.part, a.B * a.H, nqb, 1.0 / pairs, a.sim);
  return hipGetLastError();
}

template <int D>
static hipError_t anchor_broadcast(const AnchorArgs& a, hipStream_t st) {
  constexpr int rows_per_block = 256 / (D * 2 / 16) * BC_PASSES;
  const dim3 grid((unsigned)((a.L + rows_per_block - 1) / rows_per_block), (unsigned)(a.B * a.heads.n));
  hipLaunchKernelGGL((anchor_broadcast_kernel<bf16, D>), grid, dim3(256), 0, st, (const bf16*)a.Oa, (bf16*)a.O,
                     a.heads, a.H, a.L, a.Lq, a.seq_len, a.rows, a.cols, a.k);
  return hipGetLastError();
}

// Parts per anchor row: every group of the persistent grid (two per CU)
// takes whole rows, so few long rows leave groups idle at the end (k = 3 at
// 40 heads x 26 rows: 1,040 rows on 512 groups, 3 rows on the busiest).
// Cutting each row into S parts over its key blocks evens that out at the
// price of one row switch per part (~4 key blocks of work) and a merge pass.
// S = 2^sh <= kMaxSplit minimises ceil(rows*S/groups) * (ceil(n/S) + 4) over
// n key blocks, a larger S only when it saves 2%; the parts must fit in the
// output's head rows (S*Lq*(2d+4) bytes <= L*2d) and keep a block each.
int anchor_split_shift(long long rows, int groups, int nkb, long long Lq, long long L, int d) {
  int best = 0;
  double best_cost = 0.0;
  for (int sh = 0; (1 << sh) <= kMaxSplit; ++sh) {
    const int S = 1 << sh;
    if (S > nkb) break;
    if (S > 1 && (long long)S * Lq * (2 * d + 4) > L * 2 * d) break;
    const double waves = (double)((rows * S + groups - 1) / groups);
    const double cost = waves * ((double)((nkb + S - 1) / S) + 4.0);
    if (sh == 0 || cost < 0.98 * best_cost) {
      best = sh;
      best_cost = cost;
    }
  }
  return best;
}

hipError_t launch_anchor_fwd(const AnchorArgs& a, hipStream_t st) {
  if (a.heads.n == 0) return hipSuccess;
  const int nqb = a.Lq / 128;
  const int nkb = (a.seq_len + 127) / 128;
  const int sh = anchor_split_shift((long long)a.B * a.heads.n * nqb, 2 * a.num_cu, nkb, a.Lq, a.L, a.d);
  hipLaunchKernelGGL(anchor_order_kernel, dim3(1), dim3(256), 0, st, a.heads, a.H, nqb, sh, a.order);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  AttnArgs t;
  t.Q = a.Q;
  t.K = a.K;
  t.V = a.V;
  t.v_transposed = a.v_transposed;
  t.O = a.Oa;
  t.row_ptr = nullptr;
  t.col_idx = nullptr;
  t.work_order = a.order;
  t.queue = a.queue;
  t.B = a.B;
  t.H = a.H;
  t.L = a.L;
  t.seq_len = a.seq_len;
  t.d = a.d;
  t.block = 128;
  t.nkb_valid = (a.seq_len + 127) / 128;
  t.scale = a.scale;
  t.dtype_f32 = false;
  t.num_cu = a.num_cu;
  t.Lq = a.Lq;
  t.q_valid = a.La;
  t.grid_rows = a.rows;
  t.grid_cols = a.cols;
  t.k_anchor = a.k;
  t.split_shift = sh;
  if (sh > 0) {
    // the parts go to the listed heads' rows of O, which the copy below
    // overwrites after the merge has read them
    t.O = a.O;
    t.ostride = a.L;
  }
  e = launch_anchor_attention(t, st);
  if (e != hipSuccess) return e;
  if (sh > 0) {
    const int rpb = 256 / (a.d * 2 / 16);
    const dim3 grid((unsigned)((a.La + rpb - 1) / rpb), (unsigned)(a.B * a.heads.n));
    if (a.d == 128)
      hipLaunchKernelGGL(anchor_merge_kernel<128>, grid, dim3(256), 0, st, (const bf16*)a.O, (bf16*)a.Oa, a.heads,
                         a.H, a.L, a.Lq, a.La, sh);
    else
      hipLaunchKernelGGL(anchor_merge_kernel<64>, grid, dim3(256), 0, st, (const bf16*)a.O, (bf16*)a.Oa, a.heads,
                         a.H, a.L, a.Lq, a.La, sh);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return a.d == 128 ? anchor_broadcast<128>(a, st) : anchor_broadcast<64>(a, st);
}

}  // namespace calibatt
