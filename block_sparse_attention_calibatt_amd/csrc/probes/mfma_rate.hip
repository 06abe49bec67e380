// Sustained rate of v_mfma_f32_32x32x16_bf16 on this GPU, for the roofline
// of the attention kernels.  One workgroup of 8 waves per CU (2 per SIMD,
// the attention kernel's occupancy), each wave issuing products on four
// independent accumulators from operands held in registers; the shader clock
// over the run is read from s_memtime against the 100 MHz s_memrealtime.
//
// Two runs: operands all zero (the matrix cores' issue-rate limit) and
// random N(0,1) bf16 operands (the data the attention kernel multiplies).
// Under sustained random-operand products the GPU lowers its clock to stay
// within its power limit, so the second rate, not the vendor figure, is what
// a matrix-core-bound kernel can reach.
//
// Also the vector pipe's issue interval for the three instructions the
// calibration pooling spends per score (exp2, fma, add): two waves per SIMD,
// 32 independent values per lane, cycles per wave-wide instruction per SIMD
// from s_memtime.
//
// And the pooling's mix as one SIMD runs it: four waves per SIMD (four
// 256-thread workgroups per CU, held there by their LDS), each iteration one
// wave's share of a 128-key tile at d = 128: 32 products in four chains of
// eight on random operands, then fma, exp2 and add on each of its 64 scores.
// Run as the products alone, the vector work alone and both; cycles per
// wave and tile from the elapsed time and the clock read as above.  Prints
// one JSON line.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define CHECK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "mfma_rate: %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(1);                                                                \
    }                                                                         \
  } while (0)

constexpr int kThreads = 512;
constexpr int kOperands = 16;   // bf16x8 operand registers per lane

template <bool RANDOM>
__global__ __launch_bounds__(kThreads) void mfma_rate_kernel(const bf16x8* __restrict__ in, float* __restrict__ out,
                                                             unsigned long long* __restrict__ clk, int iters) {
  bf16x8 a[8], b[8];
  const size_t base = ((size_t)blockIdx.x * kThreads + threadIdx.x) * kOperands;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = RANDOM ? in[base + i] : bf16x8{};
    b[i] = RANDOM ? in[base + 8 + i] : bf16x8{};
  }
  f32x16 acc[4] = {};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(j + t) & 7], acc[t], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(a[j]));
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float r = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) r += acc[t][0] + acc[t][7];
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = r;
  if (threadIdx.x == 0 && blockIdx.x < 8) {
    clk[blockIdx.x * 2] = t1 - t0;
    clk[blockIdx.x * 2 + 1] = r1 - r0;
  }
}

// OP 0: v_exp_f32, 1: v_fma_f32, 2: v_add_f32; 32 per lane per iteration.
template <int OP>
__global__ __launch_bounds__(kThreads) void valu_rate_kernel(float* __restrict__ out,
                                                             unsigned long long* __restrict__ clk, int iters) {
  const int lane = threadIdx.x & 63;
  float x[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) x[e] = -(lane * 0.001f + e * 0.01f);
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    // the inputs are opaque to the compiler, so nothing leaves the loop
#pragma unroll
    for (int e = 0; e < 32; e += 8)
      asm volatile("" : "+v"(x[e]), "+v"(x[e + 1]), "+v"(x[e + 2]), "+v"(x[e + 3]), "+v"(x[e + 4]),
                   "+v"(x[e + 5]), "+v"(x[e + 6]), "+v"(x[e + 7]));
    float y[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      if (OP == 0) y[e] = __builtin_amdgcn_exp2f(x[e]);
      else if (OP == 1) y[e] = fmaf(x[e], 1.0001f, -0.5f);
      else y[e] = x[e] + x[(e + 1) & 31];
    }
#pragma unroll
    for (int e = 0; e < 32; e += 8)
      asm volatile("" ::"v"(y[e]), "v"(y[e + 1]), "v"(y[e + 2]), "v"(y[e + 3]), "v"(y[e + 4]), "v"(y[e + 5]),
                   "v"(y[e + 6]), "v"(y[e + 7]));
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = x[0] + x[31];
  if (threadIdx.x == 0 && blockIdx.x < 8) clk[blockIdx.x * 2] = t1 - t0;
}

// MODE 1: products only, 2: vector work only, 3: both (products, then the
// scores they gave), as the pooling does per tile.
constexpr int kMixThreads = 256;
template <int MODE>
__global__ __launch_bounds__(kMixThreads, 4) void mix_rate_kernel(const bf16x8* __restrict__ in, float* __restrict__ out,
                                                                 unsigned long long* __restrict__ clk, int iters) {
  __shared__ float hold[9 * 1024];   // 36 KiB: four workgroups per CU, not five
  const size_t base = ((size_t)blockIdx.x * kMixThreads + threadIdx.x) * kOperands;
  hold[threadIdx.x * 4] = 0.f;
  __syncthreads();
  bf16x8 a[2], b[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) a[i] = in[base + i];
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = in[base + 8 + i];
  f32x16 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][r] = 0.01f * (float)((threadIdx.x + 3 * r + 7 * m) & 15);
  float ch[4] = {0.f, 0.f, 0.f, 0.f};
  const float c2 = 0.12752f, mc = 2.f;   // scale * log2(e) at d = 128, a reference
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    if (MODE != 2) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f32x16 x = acc[m];
#pragma unroll
        for (int s = 0; s < 8; ++s) x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s & 1], b[s & 3], x, 0, 0, 0);
        acc[m] = x;
      }
    } else {
      // the scores are opaque to the compiler, so nothing leaves the loop
#pragma unroll
      for (int m = 0; m < 4; ++m) asm volatile("" : "+v"(acc[m]));
    }
    if (MODE != 1) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) ch[r & 3] += __builtin_amdgcn_exp2f(fmaf(acc[m][r], c2, -mc));
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float r = ch[0] + ch[1] + ch[2] + ch[3] + hold[(threadIdx.x * 28) & 1020];
#pragma unroll
  for (int m = 0; m < 4; ++m) r += acc[m][0] + acc[m][9];
  out[(size_t)blockIdx.x * kMixThreads + threadIdx.x] = r;
  if (threadIdx.x == 0 && blockIdx.x < 8) {
    clk[blockIdx.x * 2] = t1 - t0;
    clk[blockIdx.x * 2 + 1] = r1 - r0;
  }
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 40000;
  int ncu = 0;
  CHECK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, 0));
  const size_t lanes = (size_t)ncu * kThreads;
  // N(0, 1) operands (Box-Muller on a 64-bit LCG), rounded to bf16: the
  // distribution of the attention inputs
  std::vector<unsigned short> h(lanes * kOperands * 8);
  unsigned long long st = 0x9e3779b97f4a7c15ull;
  auto uni = [&]() {
    st = st * 6364136223846793005ull + 1442695040888963407ull;
    return ((st >> 11) + 0.5) * (1.0 / 9007199254740992.0);
  };
  for (size_t i = 0; i < h.size(); i += 2) {
    const double r = sqrt(-2.0 * log(uni())), th = 6.283185307179586 * uni();
    const float v[2] = {(float)(r * cos(th)), (float)(r * sin(th))};
    for (int k = 0; k < 2 && i + k < h.size(); ++k) {
      unsigned u;
      memcpy(&u, &v[k], 4);
      u += 0x7fffu + ((u >> 16) & 1u);   // round to nearest even
      h[i + k] = (unsigned short)(u >> 16);
    }
  }
  bf16x8* in = nullptr;
  float* out = nullptr;
  unsigned long long* clk = nullptr;
  CHECK(hipMalloc(&in, h.size() * 2));
  CHECK(hipMalloc(&out, lanes * 4));
  CHECK(hipMalloc(&clk, 16 * sizeof(unsigned long long)));
  CHECK(hipMemcpy(in, h.data(), h.size() * 2, hipMemcpyHostToDevice));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  double tf[2], ghz[2];
  for (int mode = 0; mode < 2; ++mode) {
    auto kern = mode ? mfma_rate_kernel<true> : mfma_rate_kernel<false>;
    hipLaunchKernelGGL(kern, dim3(ncu), dim3(kThreads), 0, 0, in, out, clk, iters / 4);   // warm up
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(kern, dim3(ncu), dim3(kThreads), 0, 0, in, out, clk, iters);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    unsigned long long c[16];
    CHECK(hipMemcpy(c, clk, sizeof(c), hipMemcpyDeviceToHost));
    double g = 0.0;
    for (int i = 0; i < 8; ++i) g += (double)c[2 * i] / ((double)c[2 * i + 1] / 1e8) / 1e9 / 8.0;
    const double flops = (double)ncu * 8 * iters * 32 * (32.0 * 32 * 16 * 2);
    tf[mode] = flops / (ms * 1e-3) / 1e12;
    ghz[mode] = g;
  }
  // vector pipe: cycles per wave-wide instruction per SIMD (two waves issue 32 each per iteration)
  double vcyc[3];
  const int viters = 4000;
  for (int op = 0; op < 3; ++op) {
    auto kern = op == 0 ? valu_rate_kernel<0> : (op == 1 ? valu_rate_kernel<1> : valu_rate_kernel<2>);
    for (int rep = 0; rep < 2; ++rep) {
      hipLaunchKernelGGL(kern, dim3(ncu), dim3(kThreads), 0, 0, out, clk, viters);
      CHECK(hipGetLastError());
      CHECK(hipDeviceSynchronize());
    }
    unsigned long long c[16];
    CHECK(hipMemcpy(c, clk, sizeof(c), hipMemcpyDeviceToHost));
    double s = 0.0;
    for (int i = 0; i < 8; ++i) s += (double)c[2 * i] / 8.0;
    vcyc[op] = s / viters / 64.0;
  }
  // the pooling's mix: cycles per wave and tile at four waves per SIMD
  double mix[3], mixghz[3];
  const int miters = 1000;
  bf16x8* min_ = nullptr;
  const size_t mlanes = (size_t)ncu * 4 * kMixThreads;
  CHECK(hipMalloc(&min_, mlanes * kOperands * 16));
  float* mout = nullptr;
  CHECK(hipMalloc(&mout, mlanes * 4));
  for (size_t off = 0; off < mlanes * kOperands * 8; off += h.size())   // the same random operands, repeated
    CHECK(hipMemcpy((unsigned short*)min_ + off, h.data(), std::min(h.size(), mlanes * kOperands * 8 - off) * 2,
                    hipMemcpyHostToDevice));
  for (int mode = 0; mode < 3; ++mode) {
    auto kern = mode == 0 ? mix_rate_kernel<1> : (mode == 1 ? mix_rate_kernel<2> : mix_rate_kernel<3>);
    hipLaunchKernelGGL(kern, dim3(ncu * 4), dim3(kMixThreads), 0, 0, min_, mout, clk, miters / 4);   // warm up
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(kern, dim3(ncu * 4), dim3(kMixThreads), 0, 0, min_, mout, clk, miters);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    unsigned long long c[16];
    CHECK(hipMemcpy(c, clk, sizeof(c), hipMemcpyDeviceToHost));
    double g = 0.0;
    for (int i = 0; i < 8; ++i) g += (double)c[2 * i] / ((double)c[2 * i + 1] / 1e8) / 1e9 / 8.0;
    mixghz[mode] = g;
    mix[mode] = ms * 1e-3 * g * 1e9 / miters / 4.0;   // four waves share a SIMD
  }
  CHECK(hipFree(min_));
  CHECK(hipFree(mout));
  printf("{\"zero_operands_tflops\": %.1f, \"zero_operands_clock_ghz\": %.3f, "
         "\"random_operands_tflops\": %.1f, \"random_operands_clock_ghz\": %.3f, \"cus\": %d, "
         "\"valu_cycles_per_wave_instruction\": {\"exp2\": %.2f, \"fma\": %.2f, \"add\": %.2f}, "
         "\"pooling_mix_cycles_per_wave_tile\": {\"products\": %.0f, \"vector\": %.0f, \"both\": %.0f, "
         "\"clock_ghz\": [%.3f, %.3f, %.3f]}}\n",
         tf[0], ghz[0], tf[1], ghz[1], ncu, vcyc[0], vcyc[1], vcyc[2], mix[0], mix[1], mix[2], mixghz[0],
         mixghz[1], mixghz[2]);
  CHECK(hipFree(in));
  CHECK(hipFree(out));
  CHECK(hipFree(clk));
  return 0;
}
