// Kernel (2) of the forward: the 4-bit GEMM Q4(X_hat) Q4(R)^T with its
// dequantization, plus an epilogue that adds the low-rank up-projection
// (X_hat L1) L2 and the bias before the single bf16 write of Y
// (aiflownews.com, "What SVDQuant actually does": the two-branch computation;
// "Nunchaku: the inference engine...": the branches share the output write).
//
// MXFP4: E2M1 operands with E8M0 block scales go straight into
//   v_mfma_scale_f32_32x32x64_f8f6f4; the hardware applies 2^(ex+ew) per
//   32-channel block and accumulates in fp32.
// INT4: nibbles are widened in registers to int8 holding 16*q ((w<<4)&0xF0F0F0F0
//   for even channels, w&0xF0F0F0F0 for odd ones), one v_mfma_i32_16x16x64_i8
//   per 64-channel group gives 256*P exactly in int32, and the group is
//   dequantized as acc += float(256 P) * (s_x s_w / 256).
//
// Tiles: a workgroup of 4 waves (2x2) owns a BM x BN output tile; operands are
// staged through LDS in K-stages of 128 channels (64 bytes per row), double
// buffered, row pitch 80 bytes. Workgroups are mapped to tiles so that each
// of the 8 XCDs (workgroup i runs on XCD i%8) walks a contiguous, row-grouped
// range of tiles and keeps its operand panels in its own L2.
#include <type_traits>

#include "svdq_device.h"
#include "svdq_internal.h"

namespace svdq {

constexpr int G_PITCH = 80;

struct TileMap {
  int tm, tn;
};
__device__ __forceinline__ TileMap map_tile(int bid, int tiles_m, int tiles_n, int group_m) {
  const int T = tiles_m * tiles_n;
  const int xcd = bid & 7, j = bid >> 3;
  const int per = T >> 3, rem = T & 7;
  const int t = xcd * per + (xcd < rem ? xcd : rem) + j;
  const int gsz = group_m * tiles_n;
  const int g = t / gsz;
  const int first = g * group_m;
  const int gm = min(tiles_m - first, group_m);
  const int in = t - g * gsz;
  return TileMap{first + in % gm, in / gm};
}

// ------------------------------------------------------------------------------------
// MXFP4: BM x BN tile, 4 waves of (BM/2) x (BN/2), 32x32x64 scaled FP4 MFMA.
// ------------------------------------------------------------------------------------
template <int BM, int BN>
__global__ __launch_bounds__(256, 1) void gemm_mxfp4_kernel(GemmArgs a, int tiles_m, int tiles_n) {
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  constexpr int LA = BM / 64, LB = BN / 64;       // 16-byte loads per thread per stage
  constexpr int STAGE = (BM + BN) * G_PITCH;
  extern __shared__ __align__(16) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const TileMap tmap = map_tile(blockIdx.x, tiles_m, tiles_n, 8);
  const int m0 = tmap.tm * BM, n0 = tmap.tn * BN;
  const int M = a.M, N = a.N, K = a.K;
  const int KB = K / 2;          // bytes per row
  const int nst = K / 128;       // stages
  const int nch = K / 256;       // scale words per row and half

  // global -> LDS load mapping: row tid/4 (+64 i), 16-byte chunk tid%4
  const int lrow = tid >> 2, lchk = tid & 3;
  const uint8_t* ga[LA];
  const uint8_t* gb[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) ga[i] = a.qx + (size_t)min(m0 + lrow + 64 * i, M - 1) * KB + lchk * 16;
#pragma unroll
  for (int i = 0; i < LB; ++i) gb[i] = a.qw + (size_t)min(n0 + lrow + 64 * i, N - 1) * KB + lchk * 16;

  // scale words: lane (row l%32, half l/32) of each 32-row block
  const int h = lane >> 5, lr = lane & 31;
  const uint32_t* sa_p[TM];
  const uint32_t* sb_p[TN];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    int row = min(m0 + wm * WM + t * 32 + lr, M - 1);
    sa_p[t] = reinterpret_cast<const uint32_t*>(a.sx) + (size_t)row * nch * 2 + h;
  }
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    int col = min(n0 + wn * WN + t * 32 + lr, N - 1);
    sb_p[t] = reinterpret_cast<const uint32_t*>(a.sw) + (size_t)col * nch * 2 + h;
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  uint4 ra[LA], rb[LB];
  auto gload = [&](int st) {
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const uint4*>(ga[i] + st * 64);
#pragma unroll
    for (int i = 0; i < LB; ++i) rb[i] = *reinterpret_cast<const uint4*>(gb[i] + st * 64);
  };
  auto lstore = [&](int buf) {
    uint8_t* base = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < LA; ++i)
      *reinterpret_cast<uint4*>(base + (lrow + 64 * i) * G_PITCH + lchk * 16) = ra[i];
#pragma unroll
    for (int i = 0; i < LB; ++i)
      *reinterpret_cast<uint4*>(base + (BM + lrow + 64 * i) * G_PITCH + lchk * 16) = rb[i];
  };

  uint32_t swa[TM], swb[TN];
  auto sload = [&](int c) {
#pragma unroll
    for (int t = 0; t < TM; ++t) swa[t] = sa_p[t][2 * c];
#pragma unroll
    for (int t = 0; t < TN; ++t) swb[t] = sb_p[t][2 * c];
  };

  // one K-stage (two 64-channel steps) from LDS buffer `buf`; OPS0 = opsel of step 0
  auto compute = [&](int buf, auto ops0) {
    constexpr int O0 = decltype(ops0)::value;
    const uint8_t* base = smem + buf * STAGE;
#pragma unroll
    for (int step = 0; step < 2; ++step) {
      i32x8 fa[TM], fb[TN];
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        uint4 v = *reinterpret_cast<const uint4*>(base + (wm * WM + t * 32 + lr) * G_PITCH + step * 32 + h * 16);
        fa[t] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        uint4 v = *reinterpret_cast<const uint4*>(base + (BM + wn * WN + t * 32 + lr) * G_PITCH + step * 32 + h * 16);
        fb[t] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if (step == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fa[i], fb[j], acc[i][j], 4, 4, O0, (int)swa[i], O0, (int)swb[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fa[i], fb[j], acc[i][j], 4, 4, O0 + 1, (int)swa[i], O0 + 1, (int)swb[j]);
        }
    }
  };

  gload(0);
  lstore(0);
  sload(0);
  __syncthreads();
  for (int st = 0; st < nst; st += 2) {
    // stage st (even): scale bytes 0,1 of chunk st/2
    gload(st + 1);
    compute(0, std::integral_constant<int, 0>{});
    lstore(1);
    __syncthreads();
    // stage st+1 (odd): scale bytes 2,3
    if (st + 2 < nst) gload(st + 2);
    compute(1, std::integral_constant<int, 2>{});
    if (st + 2 < nst) {
      lstore(0);
      sload((st + 2) / 2);
    }
    __syncthreads();
  }

  // epilogue: + Z L2 on bf16 MFMA, + bias, bf16 store
  if (a.r32 > 0) {
    for (int c = 0; c < a.r32 / 16; ++c) {
      bf16x8 za[TM], lb[TN];
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        int row = min(m0 + wm * WM + t * 32 + lr, M - 1);
        uint4 v = *reinterpret_cast<const uint4*>(a.z + (size_t)row * a.r32 + 16 * c + 8 * h);
        za[t] = *reinterpret_cast<bf16x8*>(&v);
      }
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        int col = min(n0 + wn * WN + t * 32 + lr, N - 1);
        uint4 v = *reinterpret_cast<const uint4*>(a.l2t + (size_t)col * a.r32 + 16 * c + 8 * h);
        lb[t] = *reinterpret_cast<bf16x8*>(&v);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(za[i], lb[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n0 + wn * WN + j * 32 + lr;
    if (col >= N) continue;
    const float bv = __uint_as_float((uint32_t)a.bias[col] << 16);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * WM + i * 32 + 8 * (e / 4) + 4 * h + (e % 4);
        if (row < M) a.y[(size_t)row * N + col] = (uint16_t)f2bf(acc[i][j][e] + bv);
      }
  }
}

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

  uint4 ra[LA], rb[LB];
  auto gload = [&](int st) {
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const uint4*>(ga[i] + st * 64);
#pragma unroll
    for (int i = 0; i < LB; ++i) rb[i] = *reinterpret_cast<const uint4*>(gb[i] + st * 64);
  };
  auto lstore = [&](int buf) {
    uint8_t* base = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < LA; ++i)
      *reinterpret_cast<uint4*>(base + (lrow + 64 * i) * G_PITCH + lchk * 16) = ra[i];
#pragma unroll
    for (int i = 0; i < LB; ++i)
      *reinterpret_cast<uint4*>(base + (BM + lrow + 64 * i) * G_PITCH + lchk * 16) = rb[i];
  };
  auto widen = [](uint2 w) {
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
        fa[t] = widen(*reinterpret_cast<const uint2*>(base + (wm * WM + t * 16 + c16) * G_PITCH + gg * 32 + q * 8));
#pragma unroll
      for (int t = 0; t < TN; ++t)
        fb[t] = widen(*reinterpret_cast<const uint2*>(base + (BM + wn * WN + t * 16 + c16) * G_PITCH + gg * 32 + q * 8));
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

// One-time per-device set-up: allow the MXFP4 kernel its 80 KiB of LDS.
hipError_t prepare_kernels() {
  return hipFuncSetAttribute((const void*)gemm_mxfp4_kernel<256, 256>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, 2 * 512 * G_PITCH);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  if (a.fmt == SVDQ_FMT_MXFP4_G32) {
    constexpr int BM = 256, BN = 256;
    const int tm = (a.M + BM - 1) / BM, tn = (a.N + BN - 1) / BN;
    const size_t lds = 2 * (size_t)(BM + BN) * G_PITCH;
    hipLaunchKernelGGL((gemm_mxfp4_kernel<BM, BN>), dim3(tm * tn), dim3(256), lds, st, a, tm, tn);
    return hipGetLastError();
  }
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
