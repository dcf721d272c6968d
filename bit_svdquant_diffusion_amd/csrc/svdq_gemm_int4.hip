// Kernel (2) of the forward for INT4 layers: Q4(X_hat) Q4(R)^T with per-group
// dequantization, plus the epilogue that adds (X_hat L1) L2 and the bias
// before the single bf16 write of Y (aiflownews.com, "What SVDQuant actually
// does": the two-branch computation; "Nunchaku: the inference engine...": the
// branches share the output write).
//
// Nibbles are widened in registers to int8 holding 16*q ((w<<4)&0xF0F0F0F0 for
// even channels, w&0xF0F0F0F0 for odd ones); one v_mfma_i32_16x16x64_i8 per
// 64-channel group gives 256*P exactly in int32; the group is dequantized as
// acc += float(256 P) * (s_x s_w / 256). Operands are staged through LDS in
// K-stages of 128 channels (two groups), double buffered.
#include "svdq_gemm_common.h"
#include "svdq_internal.h"

namespace svdq {

// ------------------------------------------------------------------------------------
// INT4: 128 x 128 tile, 4 waves of 64 x 64, one 16x16x64 i8 MFMA per block and group.
// ------------------------------------------------------------------------------------
template <bool DEBUG_P>
__global__ __launch_bounds__(256) void gemm_int4_kernel(GemmArgs a, int tiles_m, int tiles_n,
                                                        int tm_off, int tn_off) {
  constexpr int BM = 128, BN = 128, WM = 64, WN = 64, TM = 4, TN = 4, LA = 2, LB = 2;
  constexpr int STAGE = (BM + BN) * G_PITCH;
  __shared__ __align__(16) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  TileMap tmap;
  if (DEBUG_P) {
    tmap.tm = tm_off + blockIdx.x % tiles_m;
    tmap.tn = tn_off + blockIdx.x / tiles_m;
  } else {
    tmap = map_tile(blockIdx.x, tiles_m, tiles_n, 8);
  }
  const int m0 = tmap.tm * BM, n0 = tmap.tn * BN;
  const int M = a.M, N = a.N, K = a.K;
  const int KB = K / 2, nst = K / 128, G = K / 64;
  const int Mp = (M + 15) / 16 * 16;

  const int lrow = tid >> 2, lchk = tid & 3;
  const uint8_t* ga[LA];
  const uint8_t* gb[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) ga[i] = a.qx + (size_t)min(m0 + lrow + 64 * i, M - 1) * KB + lchk * 16;
#pragma unroll
  for (int i = 0; i < LB; ++i) gb[i] = a.qw + (size_t)min(n0 + lrow + 64 * i, N - 1) * KB + lchk * 16;

  const int q = lane >> 4, c16 = lane & 15;   // 16x16 layout: rows 4q+i, col c16
  const float* sxp[TM];
  const float* swp[TN];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    int row4 = min(m0 + wm * WM + t * 16 + 4 * q, Mp - 4);
    sxp[t] = reinterpret_cast<const float*>(a.sx) + row4;
  }
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    int col = min(n0 + wn * WN + t * 16 + c16, N - 1);
    swp[t] = reinterpret_cast<const float*>(a.sw) + col;
  }

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{};

  u32x4 ra[LA], rb[LB];
  auto gload = [&](int st) {
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const u32x4*>(ga[i] + st * 64);
#pragma unroll
    for (int i = 0; i < LB; ++i) rb[i] = *reinterpret_cast<const u32x4*>(gb[i] + st * 64);
  };
  auto lstore = [&](int buf) {
    uint8_t* base = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < LA; ++i)
      *reinterpret_cast<u32x4*>(base + (lrow + 64 * i) * G_PITCH + lchk * 16) = ra[i];
#pragma unroll
    for (int i = 0; i < LB; ++i)
      *reinterpret_cast<u32x4*>(base + (BM + lrow + 64 * i) * G_PITCH + lchk * 16) = rb[i];
  };
  auto widen = [](u32x2 w) {
    return i32x4{(int)((w.x << 4) & 0xF0F0F0F0u), (int)(w.x & 0xF0F0F0F0u),
                 (int)((w.y << 4) & 0xF0F0F0F0u), (int)(w.y & 0xF0F0F0F0u)};
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) gload(st + 1);
    const uint8_t* base = smem + buf * STAGE;
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const int g = 2 * st + gg;
      i32x4 fa[TM], fb[TN];
#pragma unroll
      for (int t = 0; t < TM; ++t)
        fa[t] = widen(*reinterpret_cast<const u32x2*>(base + (wm * WM + t * 16 + c16) * G_PITCH + gg * 32 + q * 8));
#pragma unroll
      for (int t = 0; t < TN; ++t)
        fb[t] = widen(*reinterpret_cast<const u32x2*>(base + (BM + wn * WN + t * 16 + c16) * G_PITCH + gg * 32 + q * 8));
      f32x4 sxv[TM];
      float swv[TN];
      if (!DEBUG_P) {
#pragma unroll
        for (int t = 0; t < TM; ++t) sxv[t] = *reinterpret_cast<const f32x4*>(sxp[t] + (size_t)g * Mp);
#pragma unroll
        for (int t = 0; t < TN; ++t) swv[t] = swp[t][(size_t)g * N] * (1.0f / 256.0f);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          i32x4 p = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], i32x4{}, 0, 0, 0);
          if (DEBUG_P) {
            const int col = n0 + wn * WN + j * 16 + c16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int row = m0 + wm * WM + i * 16 + 4 * q + e;
              if (row >= a.m0 && row < a.m0 + a.mc && col >= a.n0 && col < a.n0 + a.nc && row < M)
                a.p[((size_t)(row - a.m0) * a.nc + (col - a.n0)) * G + g] = p[e] / 256;
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] += (float)p[e] * (sxv[i][e] * swv[j]);
          }
        }
    }
    if (st + 1 < nst) lstore(buf ^ 1);
    __syncthreads();
  }
  if (DEBUG_P) return;

  if (a.r32 > 0) {
    for (int c = 0; c < a.r32 / 32; ++c) {
      bf16x8 za[TM], lb[TN];
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        int row = min(m0 + wm * WM + t * 16 + c16, M - 1);
        uint4 v = *reinterpret_cast<const uint4*>(a.z + (size_t)row * a.r32 + 32 * c + 8 * q);
        za[t] = *reinterpret_cast<bf16x8*>(&v);
      }
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        int col = min(n0 + wn * WN + t * 16 + c16, N - 1);
        uint4 v = *reinterpret_cast<const uint4*>(a.l2t + (size_t)col * a.r32 + 32 * c + 8 * q);
        lb[t] = *reinterpret_cast<bf16x8*>(&v);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(za[i], lb[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n0 + wn * WN + j * 16 + c16;
    if (col >= N) continue;
    const float bv = __uint_as_float((uint32_t)a.bias[col] << 16);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm * WM + i * 16 + 4 * q + e;
        if (row < M) a.y[(size_t)row * N + col] = (uint16_t)f2bf(acc[i][j][e] + bv);
      }
  }
}

hipError_t launch_gemm_int4(const GemmArgs& a, hipStream_t st) {
  constexpr int BM = 128, BN = 128;
  if (a.p) {
    const int tm0 = a.m0 / BM, tm1 = (a.m0 + a.mc + BM - 1) / BM;
    const int tn0 = a.n0 / BN, tn1 = (a.n0 + a.nc + BN - 1) / BN;
    const int tm = tm1 - tm0, tn = tn1 - tn0;
    hipLaunchKernelGGL((gemm_int4_kernel<true>), dim3(tm * tn), dim3(256), 0, st, a, tm, tn, tm0, tn0);
    return hipGetLastError();
  }
  const int tm = (a.M + BM - 1) / BM, tn = (a.N + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_int4_kernel<false>), dim3(tm * tn), dim3(256), 0, st, a, tm, tn, 0, 0);
  return hipGetLastError();
}

}  // namespace svdq
