// Kernel (2) of the forward for MXFP4 layers: Q4(X_hat) Q4(R)^T on the
// block-scaled FP4 MFMA, plus the epilogue that adds (X_hat L1) L2 and the
// bias before the single bf16 write of Y (aiflownews.com, "What SVDQuant
// actually does": two-branch computation, FP4 data type; "Nunchaku: the
// inference engine...": the branches share the output write).
//
// E2M1 operands and their E8M0 block scales go straight into
// v_mfma_scale_f32_32x32x64_f8f6f4: the hardware applies 2^(e_w + e_x) per
// 32-channel block and accumulates in fp32, so no dequantization runs on the
// vector ALUs. The MFMA is issued with the weight fragment as operand A and
// the activation fragment as operand B, so a lane's 16 results are 4 runs of
// 4 consecutive output channels of one token: Y is written 8 bytes at a time.
//
// Tiling: a BM x BN output tile per workgroup of WGM x WGN waves (two waves
// per SIMD for the default 256 x 256 / 8-wave shape, so one wave's barrier
// and LDS traffic hide behind the other's MFMAs). K advances in stages of 128
// channels (64 bytes per row), double buffered in LDS; global loads for stage
// s+2 are in flight while stage s computes.
#include "svdq_gemm_common.h"
#include "svdq_internal.h"

namespace svdq {

template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_mxfp4_kernel(GemmArgs a, int tiles_m,
                                                                  int tiles_n) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int LA = BM * 4 / NT, LB = BN * 4 / NT;   // 16-byte chunks per thread per stage
  static_assert(LA * NT == BM * 4 && LB * NT == BN * 4, "tile / thread mismatch");
  constexpr int STAGE = (BM + BN) * G_PITCH;
  extern __shared__ __align__(16) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const TileMap tmap = map_tile(blockIdx.x, tiles_m, tiles_n, 8);
  const int m0 = tmap.tm * BM, n0 = tmap.tn * BN;
  const int M = a.M, N = a.N, K = a.K;
  const int KB = K / 2;        // bytes per row
  const int nst = K / 128;     // K-stages (even: K % 256 == 0)
  const int nch = K / 256;     // scale words per row and half

  // global -> LDS staging: chunk c = tid + NT i covers row c/4, bytes 16 (c%4)
  const uint8_t* ga[LA];
  const uint8_t* gb[LB];
  int la[LA], lb[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int c = tid + NT * i, row = c >> 2, chk = c & 3;
    ga[i] = a.qx + (size_t)min(m0 + row, M - 1) * KB + chk * 16;
    la[i] = row * G_PITCH + chk * 16;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int c = tid + NT * i, row = c >> 2, chk = c & 3;
    gb[i] = a.qw + (size_t)min(n0 + row, N - 1) * KB + chk * 16;
    lb[i] = (BM + row) * G_PITCH + chk * 16;
  }

  // MFMA lane roles: lane (lr = l%32, h = l/32) holds row lr of a 32-row block
  // and channels [32h, 32h+32) of each 64-channel step.
  const int h = lane >> 5, lr = lane & 31;
  const int fa_off = (wm * WM + lr) * G_PITCH + h * 16;        // + t*32*G_PITCH + step*32
  const int fb_off = (BM + wn * WN + lr) * G_PITCH + h * 16;
  // scale words (4 E8M0 bytes = 4 consecutive 64-channel steps) per row and half
  const uint32_t* sxp[TM];
  const uint32_t* swp[TN];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    const int row = min(m0 + wm * WM + t * 32 + lr, M - 1);
    sxp[t] = reinterpret_cast<const uint32_t*>(a.sx) + (size_t)row * nch * 2 + h;
  }
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int col = min(n0 + wn * WN + t * 32 + lr, N - 1);
    swp[t] = reinterpret_cast<const uint32_t*>(a.sw) + (size_t)col * nch * 2 + h;
  }

  f32x16 acc[TN][TM];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i) acc[j][i] = f32x16{};

  u32x4 ra[LA], rb[LB];
  uint32_t sx[TM], sw[TN], sxn[TM], swn[TN];

  // prologue: stage 0 into LDS buffer 0, stage 1 in registers, scale words of chunks 0, 1
#pragma unroll
  for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const u32x4*>(ga[i]);
#pragma unroll
  for (int i = 0; i < LB; ++i) rb[i] = *reinterpret_cast<const u32x4*>(gb[i]);
#pragma unroll
  for (int i = 0; i < LA; ++i) *reinterpret_cast<u32x4*>(smem + la[i]) = ra[i];
#pragma unroll
  for (int i = 0; i < LB; ++i) *reinterpret_cast<u32x4*>(smem + lb[i]) = rb[i];
#pragma unroll
  for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const u32x4*>(ga[i] + 64);
#pragma unroll
  for (int i = 0; i < LB; ++i) rb[i] = *reinterpret_cast<const u32x4*>(gb[i] + 64);
#pragma unroll
  for (int t = 0; t < TM; ++t) sx[t] = sxp[t][0];
#pragma unroll
  for (int t = 0; t < TN; ++t) sw[t] = swp[t][0];
  const int c1 = nch > 1 ? 1 : 0;
#pragma unroll
  for (int t = 0; t < TM; ++t) sxn[t] = sxp[t][2 * c1];
#pragma unroll
  for (int t = 0; t < TN; ++t) swn[t] = swp[t][2 * c1];
  __syncthreads();

#define SVDQ_MX_COMPUTE(BUF, O0)                                                                 \
  {                                                                                              \
    const uint8_t* base = smem + (BUF) * STAGE;                                                  \
    _Pragma("unroll") for (int step = 0; step < 2; ++step) {                                     \
      i32x8 fa[TM], fb[TN];                                                                      \
      _Pragma("unroll") for (int t = 0; t < TM; ++t) {                                           \
        const u32x4 v = *reinterpret_cast<const u32x4*>(base + fa_off + t * 32 * G_PITCH + step * 32); \
        fa[t] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};                       \
      }                                                                                          \
      _Pragma("unroll") for (int t = 0; t < TN; ++t) {                                           \
        const u32x4 v = *reinterpret_cast<const u32x4*>(base + fb_off + t * 32 * G_PITCH + step * 32); \
        fb[t] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};                       \
      }                                                                                          \
      _Pragma("unroll") for (int j = 0; j < TN; ++j) _Pragma("unroll") for (int i = 0; i < TM; ++i) { \
        if (step == 0)                                                                           \
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                           \
              fb[j], fa[i], acc[j][i], 4, 4, (O0), (int)sw[j], (O0), (int)sx[i]);                \
        else                                                                                     \
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                           \
              fb[j], fa[i], acc[j][i], 4, 4, (O0) + 1, (int)sw[j], (O0) + 1, (int)sx[i]);        \
      }                                                                                          \
    }                                                                                            \
  }

  for (int st = 0; st < nst; st += 2) {
    // even stage st (LDS buffer 0, scale bytes 0 and 1 of chunk st/2);
    // registers hold stage st+1: park it in buffer 1, fetch stage st+2
#pragma unroll
    for (int i = 0; i < LA; ++i) *reinterpret_cast<u32x4*>(smem + STAGE + la[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < LB; ++i) *reinterpret_cast<u32x4*>(smem + STAGE + lb[i]) = rb[i];
    if (st + 2 < nst) {
#pragma unroll
      for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const u32x4*>(ga[i] + (st + 2) * 64);
#pragma unroll
      for (int i = 0; i < LB; ++i) rb[i] = *reinterpret_cast<const u32x4*>(gb[i] + (st + 2) * 64);
    }
    SVDQ_MX_COMPUTE(0, 0)
    __syncthreads();
    // odd stage st+1 (buffer 1, scale bytes 2 and 3)
    if (st + 2 < nst) {
#pragma unroll
      for (int i = 0; i < LA; ++i) *reinterpret_cast<u32x4*>(smem + la[i]) = ra[i];
#pragma unroll
      for (int i = 0; i < LB; ++i) *reinterpret_cast<u32x4*>(smem + lb[i]) = rb[i];
#pragma unroll
      for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const u32x4*>(ga[i] + (st + 3) * 64);
#pragma unroll
      for (int i = 0; i < LB; ++i) rb[i] = *reinterpret_cast<const u32x4*>(gb[i] + (st + 3) * 64);
    }
    SVDQ_MX_COMPUTE(1, 2)
    // next chunk's scale words become current; fetch the one after
    const int cn = min(st / 2 + 2, nch - 1);
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      sx[t] = sxn[t];
      sxn[t] = sxp[t][2 * cn];
    }
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      sw[t] = swn[t];
      swn[t] = swp[t][2 * cn];
    }
    __syncthreads();
  }
#undef SVDQ_MX_COMPUTE

  // epilogue: + (X_hat L1) L2 on bf16 MFMA (L2^T fragment as A, Z fragment as B)
  if (a.r32 > 0) {
    for (int c = 0; c < a.r32 / 16; ++c) {
      bf16x8 zf[TM], lf[TN];
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const int row = min(m0 + wm * WM + t * 32 + lr, M - 1);
        uint4 v = *reinterpret_cast<const uint4*>(a.z + (size_t)row * a.r32 + 16 * c + 8 * h);
        zf[t] = *reinterpret_cast<bf16x8*>(&v);
      }
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int col = min(n0 + wn * WN + t * 32 + lr, N - 1);
        uint4 v = *reinterpret_cast<const uint4*>(a.l2t + (size_t)col * a.r32 + 16 * c + 8 * h);
        lf[t] = *reinterpret_cast<bf16x8*>(&v);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf[j], zf[i], acc[j][i], 0, 0, 0);
    }
  }
  // + bias, bf16, 8-byte stores: lane holds token m = .. + lr and channels
  // n = .. + 8q + 4h + (0..3) for q = 0..3
#pragma unroll
  for (int j = 0; j < TN; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + wn * WN + j * 32 + 8 * q + 4 * h;
      if (n >= N) continue;
      const uint2 bw = *reinterpret_cast<const uint2*>(a.bias + n);
      const float b0 = bf16lo(bw.x), b1 = bf16hi(bw.x), b2 = bf16lo(bw.y), b3 = bf16hi(bw.y);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = m0 + wm * WM + i * 32 + lr;
        if (m >= M) continue;
        uint2 o;
        o.x = pack_bf16x2(acc[j][i][4 * q + 0] + b0, acc[j][i][4 * q + 1] + b1);
        o.y = pack_bf16x2(acc[j][i][4 * q + 2] + b2, acc[j][i][4 * q + 3] + b3);
        *reinterpret_cast<uint2*>(a.y + (size_t)m * N + n) = o;
      }
    }
  }
}

namespace {
constexpr int kBM = 256, kBN = 256, kWGM = 2, kWGN = 4;
constexpr size_t kLds = 2 * (size_t)(kBM + kBN) * G_PITCH;
}  // namespace

hipError_t prepare_gemm_mxfp4() {
  return hipFuncSetAttribute((const void*)gemm_mxfp4_kernel<kBM, kBN, kWGM, kWGN>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
}

hipError_t launch_gemm_mxfp4(const GemmArgs& a, hipStream_t st) {
  const int tm = (a.M + kBM - 1) / kBM, tn = (a.N + kBN - 1) / kBN;
  hipLaunchKernelGGL((gemm_mxfp4_kernel<kBM, kBN, kWGM, kWGN>), dim3(tm * tn),
                     dim3(64 * kWGM * kWGN), kLds, st, a, tm, tn);
  return hipGetLastError();
}

}  // namespace svdq
