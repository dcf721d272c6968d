// Measured ceilings of the part the layer runs on: an MFMA-only loop of each
// matrix instruction the GEMMs use, and a plain device copy. They are not part
// of the layer; the benchmark reports each GEMM's rate against these beside
// the published peaks (the pages give no kernel-level figures to compare with).
#include "svdq_device.h"
#include "svdq_internal.h"

namespace svdq {

namespace {
constexpr int kPeakWaves = 8;    // waves per workgroup (two per SIMD)
constexpr int kPeakChains = 4;   // independent accumulators per wave

// splitmix64 finalizer (Steele, Lea and Flood, "Fast splittable pseudorandom
// number generators"), for operand bits that change from lane to lane
__device__ __forceinline__ uint32_t mix32(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return (uint32_t)((z ^ (z >> 31)) >> 32);
}

// kind 0: v_mfma_scale_f32_32x32x64_f8f6f4 on E2M1 operands (unit E8M0
// scales); 1: v_mfma_i32_32x32x32_i8; 2: v_mfma_f32_32x32x16_bf16. Operand
// bits are random per lane, or (constant != 0) one fixed pattern.
template <int KIND>
__global__ __launch_bounds__(64 * kPeakWaves) void mfma_peak_kernel(int iters, int constant, float* sink,
                                                                     int store) {
  const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  auto bits = [&](int j) { return constant ? 0x3a3a3a3au : mix32(t * 8 + j); };
  const i32x8 a8 = {(int)bits(0), (int)bits(1), (int)bits(2), (int)bits(3), 0, 0, 0, 0};
  const i32x8 b8 = {(int)bits(4), (int)bits(5), (int)bits(6), (int)bits(7), 0, 0, 0, 0};
  // bf16: the top exponent bit cleared, so no operand is Inf or NaN
  const uint32_t m = KIND == 2 ? 0xBFFFBFFFu : 0xFFFFFFFFu;
  const i32x4 a4 = {(int)(bits(0) & m), (int)(bits(1) & m), (int)(bits(2) & m), (int)(bits(3) & m)};
  const i32x4 b4 = {(int)(bits(4) & m), (int)(bits(5) & m), (int)(bits(6) & m), (int)(bits(7) & m)};
  float out = 0.f;
  if constexpr (KIND == 1) {
    i32x16 acc[kPeakChains];
#pragma unroll
    for (int c = 0; c < kPeakChains; ++c) acc[c] = i32x16{};
#pragma unroll 4
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int c = 0; c < kPeakChains; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, b4, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < kPeakChains; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) out += (float)acc[c][e];
  } else {
    f32x16 acc[kPeakChains];
#pragma unroll
    for (int c = 0; c < kPeakChains; ++c) acc[c] = f32x16{};
#pragma unroll 4
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int c = 0; c < kPeakChains; ++c) {
        if constexpr (KIND == 0)
          acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[c], 4, 4, 0, 127, 0, 127);
        else
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4), __builtin_bit_cast(bf16x8, b4),
                                                           acc[c], 0, 0, 0);
      }
#pragma unroll
    for (int c = 0; c < kPeakChains; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) out += acc[c][e];
  }
  if (store) sink[t] = out;   // the host passes store = 0; the loop cannot be dropped
}

// dst = src, 16 bytes per lane per step, grid-stride
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}
}  // namespace

hipError_t launch_mfma_peak(int kind, int constant, int iters, int grid, float* sink, hipStream_t st,
                            double* flops) {
  const double per = kind == 0 ? 2.0 * 32 * 32 * 64 : (kind == 1 ? 2.0 * 32 * 32 * 32 : 2.0 * 32 * 32 * 16);
  *flops = per * kPeakChains * (double)iters * kPeakWaves * grid;
  const dim3 g(grid), b(64 * kPeakWaves);
  if (kind == 0)
    hipLaunchKernelGGL(mfma_peak_kernel<0>, g, b, 0, st, iters, constant, sink, 0);
  else if (kind == 1)
    hipLaunchKernelGGL(mfma_peak_kernel<1>, g, b, 0, st, iters, constant, sink, 0);
  else
    hipLaunchKernelGGL(mfma_peak_kernel<2>, g, b, 0, st, iters, constant, sink, 0);
  return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, size_t bytes, int num_cus, hipStream_t st) {
  const size_t n = bytes / 16;
  const int grid = (num_cus > 0 ? num_cus : 256) * 8;
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, st, (const u32x4*)src, (u32x4*)dst, n);
  return hipGetLastError();
}

}  // namespace svdq
