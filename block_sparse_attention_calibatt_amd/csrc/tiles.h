// Shared device helpers for the gfx950 (CDNA4) attention and calibration kernels.
//
// Matrix-core layouts (v_mfma_f32_32x32x16_bf16, wave of 64 lanes; lane l,
// half g = l / 32, column c = l % 32):
//   A operand (32 x 16): lane holds A[c][8g .. 8g+7]
//   B operand (16 x 32): lane holds B[8g .. 8g+7][c]
//   C/D       (32 x 32): lane holds D[8*(r/4) + 4g + r%4][c], r = 0..15
//
// Scores are computed transposed, S^T = K * Q^T, so that every lane owns one
// query (column c) and the softmax over keys needs only lane-local work plus
// one exchange with lane l^32.  The K rows fed to the A operand are permuted
// (bits 2 and 3 of the row index swapped) so that lane half g ends up holding
// keys 16*(r/8) + 8g + (r%8) of each 32-key slice: exactly the B-operand
// layout the P*V product needs, with no data movement between the products.
//
// LDS tiles are rows of 16-byte chunks with an XOR swizzle on the chunk
// index, so that the matrix-core operand reads (16 consecutive rows, one
// chunk) spread over all bank groups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace calibatt {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Chunk swizzle for a row of CH 16-byte chunks (CH = 16 or 8).  Reads of 16
// consecutive rows at one chunk hit 16 distinct 16-byte bank groups; the
// swizzle uses only row bits 0..4, so rows 32 apart share it and an operand
// address advances by a constant between 32-row tiles.  For 8-chunk rows the
// extra bit-4 term also spreads the transposed V writes (rows 4 apart) over 8
// groups.
template <int CH>
__device__ __forceinline__ int swz(int row) {
  if constexpr (CH == 16) {
    return row & 15;
  } else {
    return ((row >> 1) & 7) ^ ((row >> 4) & 1);
  }
}

// Unit swizzle of a V stage in natural layout (64 key rows of D/8 units).
// The transposed operand reads of 16 lanes cover 4 consecutive rows at 2
// units, those of 32 lanes 4 rows at 4 units; XOR-ing bits 2..3 of the unit
// with row bits 0..1 (D = 128, rows of 256 bytes) or row bit 1 (D = 64, rows
// of 128 bytes) puts them in distinct bank groups.  Rows that share row bits
// 0..1 share it, so a read advances by a constant between such rows.
template <int D>
__device__ __forceinline__ int vswz(int row) {
  if constexpr (D == 128) {
    return 4 * (row & 3);
  } else {
    return 4 * ((row >> 1) & 1);
  }
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Transposed LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// 4j + m reads 4 consecutive 16-bit elements at its own address, and lane i
// receives element i % 4 of the reads of lanes i / 4, 4 + i / 4, 8 + i / 4,
// 12 + i / 4: the group reads a 4 x 16 block (lanes 4j .. 4j+3 one row of 16)
// and lane i gets column i of it.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
}

template <int CH>
__device__ __forceinline__ int chunk_index(int row, int chunk) {
  return row * CH + (chunk ^ swz<CH>(row));
}

// Row of the K tile read by lane column c for the A operand: bits 2 and 3 swapped.
__device__ __forceinline__ int qk_row_perm(int c) {
  return (c & 0x13) | ((c & 4) << 1) | ((c & 8) >> 1);
}

// Key (within a 32-key slice) held in accumulator register r by lane half g.
__device__ __forceinline__ int slice_key(int r, int g) { return 16 * (r >> 3) + 8 * g + (r & 7); }

typedef __attribute__((address_space(3))) void lds_void;

// Global-memory (address space 1) views, for pointers rebuilt from integers:
// accesses through them are global, not flat, instructions, so that they are
// not counted with the LDS accesses (a flat access counts toward both
// counters, and would make every later LDS wait also wait for it).
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) int32_t g_i32;
typedef __attribute__((address_space(1))) float g_f32;
typedef __attribute__((address_space(1))) __bf16 g_bf16;
typedef __attribute__((address_space(1))) bf16x8 g_bf16x8;
typedef __attribute__((address_space(1))) bf16x4 g_bf16x4;
typedef __attribute__((address_space(1))) u32x4 g_u32x4;

// Buffer resource over `bytes` bytes at base: loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// K tile [BLK keys][D] bf16 (row-major in the slab behind rk, keys k0 ..
// k0+BLK-1) -> swizzled LDS (the chunk_index layout), by LDS DMA with no
// register staging.  Instruction m writes LDS units 64m .. 64m+63, i.e. key
// rows m*(64/CH) ..; wave w of the BLK/32 waves issues m = w, w + BLK/32, ...
// The caller waits (s_waitcnt vmcnt) and then synchronises the workgroup
// before reading the tile.
template <int D, int BLK>
__device__ __forceinline__ void dma_k_tile(__amdgpu_buffer_rsrc_t rk, int k0, u32x4* lds, int w, int lane) {
  constexpr int CH = D / 8;
  constexpr int NW = BLK / 32;
  constexpr int NI = BLK * CH / 64;
  static_assert(NI % NW == 0, "tile must split evenly over the waves");
#pragma unroll
  for (int i = 0; i < NI / NW; ++i) {
    const int m = w + NW * i;
    const int row = m * (64 / CH) + lane / CH;
    const int voff = (lane / CH) * D * 2 + (((lane % CH) ^ swz<CH>(row)) * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(lds + 64 * m), 16, voff, k0 * D * 2 + m * 1024, 0, 0);
  }
}

// s_waitcnt vmcnt(0) with expcnt and lgkmcnt left unconstrained (gfx9
// encoding), written with the builtin so that the compiler's own wait
// insertion knows the DMA has landed.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8)); }

// S^T for one wave: BLK keys x 32 queries, as BLK/32 accumulators of 32x32.
template <int D, int BLK>
__device__ __forceinline__ void qk_tile(const u32x4* __restrict__ ldsK, const bf16x8* qreg,
                                        f32x16* sacc, int g, int c) {
  constexpr int CH = D / 8;
  const int prow = qk_row_perm(c);
#pragma unroll
  for (int mt = 0; mt < BLK / 32; ++mt) {
    f32x16 acc = {};
    const int row = 32 * mt + prow;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const u32x4 a = ldsK[chunk_index<CH>(row, 2 * s + g)];
      acc = mfma_bf16(__builtin_bit_cast(bf16x8, a), qreg[s], acc);
    }
    sacc[mt] = acc;
  }
}

// Max with the partner lane l^32 (same query, other half of the keys).
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Spatial-repetition anchor rows: anchor query m (frame-major, then group,
// then column) of a (frames, R rows, C columns) token grid with k groups of
// rows [floor(g R / k), floor((g+1) R / k)), each anchored at its lower
// middle row, is token (f R + a) C + x.
__device__ __forceinline__ int anchor_token(int m, int R, int C, int k) {
  const int per_frame = k * C;
  const int f = m / per_frame, rem = m - f * per_frame;
  const int g = rem / C, x = rem - g * C;
  const int lo = (g * R) / k, hi = ((g + 1) * R) / k;
  return (f * R + (lo + hi - 1) / 2) * C + x;
}

}  // namespace calibatt
