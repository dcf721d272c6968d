// Kernel (1) of the forward: one read of X feeds three steps.
//   - smoothing: x_hat = fl32(x * mu_k) (aiflownews.com, "What SVDQuant actually
//     does": activation outliers are moved into the weights, so the runtime
//     divides X by lambda; mu = 1/lambda is stored);
//   - per-token 4-bit quantization of x_hat (INT4 per 64 channels, or MXFP4
//     per 32 channels);
//   - the low-rank down-projection Z = x_hat L1 on bf16 MFMA, with x_hat
//     rounded to bf16 ("the low rank branch held at higher precision such as
//     16 bit"; the branches "share inputs", same page).
//
// Work split: a workgroup owns 32 tokens; its WAVES waves split K in steps of
// 128 channels (wave w takes steps w, w+WAVES, ...). Per step a wave
//   1. loads the 32x128 bf16 slab with coalesced 16-byte loads (4 rows per
//      instruction) and writes it to its own LDS slab (row pitch 272 bytes);
//   2. reads it back so that lane (r = l%32, h = l/32) holds row r, channels
//      [64h, 64h+64) of the step: exactly one INT4 group (two MXFP4 blocks),
//      and exactly the A-operand run of eight 32x32x16 bf16 MFMAs;
//   3. quantizes its group alone (no cross-lane reduction) and stores 32
//      bytes of codes plus the scale;
//   4. accumulates Z on MFMA against L1, which the pack stores in the same
//      lane order (one contiguous 1 KiB per wave per MFMA).
// The WAVES partial Z tiles are summed in LDS in wave order (deterministic)
// and stored as bf16 [M][rank32].
#include "svdq_device.h"
#include "svdq_internal.h"

namespace svdq {

constexpr int S1_ROWS = 32;
constexpr int S1_PITCH = 272;  // bytes per LDS row: 256 data + 16 pad

template <int FMT, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void stage1_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ mu, const uint16_t* __restrict__ l1s,
    uint8_t* __restrict__ qx, void* __restrict__ sx, uint16_t* __restrict__ z, int M, int K,
    int r32) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m0 = blockIdx.x * S1_ROWS;
  const int nsteps = K / 128;
  const int Mp = (M + 15) / 16 * 16;   // row stride of the INT4 scales
  const int MB = (M + 31) / 32;        // 32-row blocks (MXFP4 fragment order)
  const int ncb = r32 / 32;
  uint8_t* slab = smem + wave * (S1_ROWS * S1_PITCH);

  // MFMA-layout coordinates of this lane
  const int r = lane & 31, h = lane >> 5;
  const int m = m0 + r;
  const bool row_ok = m < M;
  // coalesced-load coordinates
  const int lr = lane >> 4, lc = lane & 15;

  f32x16 zacc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) zacc[c] = f32x16{};

  for (int s = wave; s < nsteps; s += WAVES) {
    // 1. coalesced load of the 32 x 128 slab, 4 rows per instruction
    u32x4 raw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int row = min(m0 + 4 * j + lr, M - 1);
      raw[j] = *reinterpret_cast<const u32x4*>(x + (size_t)row * K + s * 128 + lc * 8);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<u32x4*>(slab + (4 * j + lr) * S1_PITCH + lc * 16) = raw[j];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // 2. group layout: lane (r, h) takes row r, channels 64h .. 64h+63 of the step
    u32x4 xv[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
      xv[t] = *reinterpret_cast<const u32x4*>(slab + r * S1_PITCH + h * 128 + t * 16);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const int k0 = s * 128 + h * 64;
    float xh[64];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const f32x4 mv = *reinterpret_cast<const f32x4*>(mu + k0 + 4 * t);
      const uint32_t w0 = xv[t / 2][(t & 1) * 2 + 0];
      const uint32_t w1 = xv[t / 2][(t & 1) * 2 + 1];
      xh[4 * t + 0] = bf16lo(w0) * mv.x;
      xh[4 * t + 1] = bf16hi(w0) * mv.y;
      xh[4 * t + 2] = bf16lo(w1) * mv.z;
      xh[4 * t + 3] = bf16hi(w1) * mv.w;
    }

    // 3. quantize the lane's 64 values
    uint32_t packed[8];
    if constexpr (FMT == SVDQ_FMT_INT4_G64) {
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 64; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(xh[i]));
      const float sc = amax / 7.0f;            // IEEE-rounded division
      const bool zero = !(sc > 0.f);
      const float inv = zero ? 0.f : 1.0f / sc;
      const bool exact_all = sc < 0x1p-100f;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          int q = zero ? 0 : q_int4(xh[8 * w + j], sc, inv, exact_all);
          word |= ((uint32_t)q & 15u) << (4 * j);
        }
        packed[w] = word;
      }
      if (row_ok) reinterpret_cast<float*>(sx)[(size_t)(2 * s + h) * Mp + m] = sc;
    } else {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(xh[32 * b + i]));
        const int e = mx_exponent(amax);
        const float sinv = exp2_neg(e);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t word = 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) word |= e2m1_code(xh[32 * b + 8 * w + j] * sinv) << (4 * j);
          packed[4 * b + w] = word;
        }
        if (row_ok) {
          // fragment-order scale byte: block kb = 4s + 2h + b -> stage s, step h, half b
          reinterpret_cast<uint8_t*>(sx)[(((size_t)s * MB + m / 32) * 64 + 32 * b + r) * 2 + h] =
              (uint8_t)(e + 127);
        }
      }
    }
    if (row_ok) {
      if constexpr (FMT == SVDQ_FMT_INT4_G64) {
        u32x4* dst = reinterpret_cast<u32x4*>(qx + (size_t)m * (K / 2) + k0 / 2);
        dst[0] = u32x4{packed[0], packed[1], packed[2], packed[3]};
        dst[1] = u32x4{packed[4], packed[5], packed[6], packed[7]};
      } else {
        // fragment order: step S = 2s + h of row block m/32, lanes r and 32 + r
        uint8_t* blk = qx + ((size_t)(m / 32) * (K / 64) + 2 * s + h) * 1024;
        *reinterpret_cast<u32x4*>(blk + r * 16) = u32x4{packed[0], packed[1], packed[2], packed[3]};
        *reinterpret_cast<u32x4*>(blk + (32 + r) * 16) = u32x4{packed[4], packed[5], packed[6], packed[7]};
      }
    }

    // 4. Z += bf16(x_hat) L1 on 32x32x16 bf16 MFMA (8 per 32 columns)
    if (ncb > 0) {
      uint32_t ab[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) ab[i] = pack_bf16x2(xh[2 * i], xh[2 * i + 1]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c < ncb) {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            u32x4 bv = *reinterpret_cast<const u32x4*>(
                l1s + ((((size_t)s * ncb + c) * 8 + t) * 64 + lane) * 8);
            u32x4 av = u32x4{ab[4 * t], ab[4 * t + 1], ab[4 * t + 2], ab[4 * t + 3]};
            zacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                *reinterpret_cast<bf16x8*>(&av), *reinterpret_cast<bf16x8*>(&bv), zacc[c], 0, 0, 0);
          }
        }
      }
    }
  }

  if (ncb == 0) return;
  // reduce the WAVES partial Z tiles in wave order and store bf16
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (c < ncb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) red[((wave * ncb + c) * 16 + i) * 64 + lane] = zacc[c][i];
    }
  __syncthreads();
  const int total = ncb * 16 * 64;
  for (int idx = threadIdx.x; idx < total; idx += 64 * WAVES) {
    float acc = 0.f;
    for (int w = 0; w < WAVES; ++w) acc += red[w * total + idx];
    const int l = idx & 63, i = (idx >> 6) & 15, c = idx >> 10;
    const int row = m0 + 8 * (i / 4) + 4 * (l / 32) + (i % 4);
    const int col = 32 * c + (l & 31);
    if (row < M) {
      if constexpr (FMT == SVDQ_FMT_INT4_G64) {
        z[(size_t)row * r32 + col] = (uint16_t)f2bf(acc);
      } else {   // fragment order: (row block, 16-column step, lane 32h + row%32, element)
        z[((((size_t)(row / 32) * (r32 / 16) + col / 16) * 64 + 32 * ((col % 16) / 8) + row % 32) * 8) +
          col % 8] = (uint16_t)f2bf(acc);
      }
    }
  }
}

template <int FMT, int WAVES>
static hipError_t launch_t(const Stage1Args& a, hipStream_t st) {
  const int r32 = a.r32;
  size_t slab = (size_t)WAVES * S1_ROWS * S1_PITCH;
  size_t red = (size_t)WAVES * (r32 / 32) * 16 * 64 * 4;
  size_t lds = slab > red ? slab : red;
  dim3 grid((a.M + S1_ROWS - 1) / S1_ROWS);
  hipLaunchKernelGGL((stage1_kernel<FMT, WAVES>), grid, dim3(64 * WAVES), lds, st, a.x, a.mu,
                     a.l1s, a.qx, a.sx, a.z, a.M, a.K, r32);
  return hipGetLastError();
}

hipError_t launch_stage1(const Stage1Args& a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  if (a.fmt == SVDQ_FMT_INT4_G64) return launch_t<SVDQ_FMT_INT4_G64, 4>(a, st);
  return launch_t<SVDQ_FMT_MXFP4_G32, 4>(a, st);
}

}  // namespace svdq
