// Kernel (2) of the forward for MXFP4 layers: Q4(X_hat) Q4(R)^T on the
// block-scaled FP4 MFMA, plus the epilogue that adds (X_hat L1) L2 and the
// bias before the single bf16 write of Y (aiflownews.com, "What SVDQuant
// actually does": two-branch computation, FP4 data type; "Nunchaku: the
// inference engine...": the branches share the output write).
//
// E2M1 operands and their E8M0 block scales go straight into
// v_mfma_scale_f32_32x32x64_f8f6f4: the hardware applies 2^(e_w + e_x) per
// 32-channel block and accumulates in fp32, so no dequantization runs on the
// vector ALUs. The weight fragment is operand A and the activation fragment
// operand B, so a lane's 16 results are 4 runs of 4 consecutive output
// channels of one token.
//
// Data path: codes and scale bytes of both operands are stored in fragment
// order (one 1 KiB block = one wave's MFMA operand), so every global->LDS
// transfer is a direct `global_load_lds_dwordx4` of a contiguous 1 KiB with
// no register staging, and every LDS fragment read is a contiguous,
// bank-conflict-free 1 KiB. A ring of NSTAGE K-stages (128 channels each)
// keeps NSTAGE-1 stages of loads in flight to cover L2-miss latency.
// The output tile is staged through the (then idle) ring so each wave writes
// Y in full 128-byte rows.
#include "svdq_gemm_common.h"
#include "svdq_internal.h"

namespace svdq {

namespace {
constexpr int kBM = 256, kBN = 256, kWGM = 2, kWGN = 4, kNW = kWGM * kWGN;
constexpr int kWM = kBM / kWGM, kWN = kBN / kWGN, kTM = kWM / 32, kTN = kWN / 32;
constexpr int kNStage = 4;
// one ring slot: A codes (8 blocks x 2 steps x 1 KiB), B codes, A scales, B scales
constexpr int kCodeA = 0, kCodeB = 16384, kScA = 32768, kScB = 33792, kSlot = 34816;
constexpr int kOutPitch = 136;                       // bytes per staged output row (128 + 8)
constexpr size_t kLds = (size_t)kNStage * kSlot;
static_assert(kLds >= (size_t)kNW * kWM * kOutPitch, "output staging must fit in the ring");
static_assert(kWM * 4 == kBM * 2 && kTM == 4 && kTN == 2, "layout below assumes 2x4 waves");

// Stage barrier of the ring: wait until at most `n` of this wave's global->LDS
// transfers are outstanding (they complete in issue order) and all its LDS reads
// have returned, then s_barrier. No memory fence: a fence would also wait for
// the later stages' transfers that are meant to stay in flight. The scheduling
// barriers keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier(int n) {
  __builtin_amdgcn_sched_barrier(0);
  // s_waitcnt: vmcnt = n (bits 3:0), expcnt = 7 (no wait), lgkmcnt = 0
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0070 | 0); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0070 | 5); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0070 | 10); break;
    default: __builtin_amdgcn_s_waitcnt(0x0070 | 0); break;
  }
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ lds_void* lds_ptr(uint8_t* p) { return (lds_void*)p; }
}  // namespace

__global__ __launch_bounds__(64 * kNW) void gemm_mxfp4_kernel(GemmArgs a, int tiles_m, int tiles_n) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / kWGN, wn = wave % kWGN;
  const TileMap tmap = map_tile(blockIdx.x, tiles_m, tiles_n, 8);
  const int m0 = tmap.tm * kBM, n0 = tmap.tn * kBN;
  const int M = a.M, N = a.N, K = a.K;
  const int MB = (M + 31) / 32, NB = N / 32;      // 32-row blocks of X (padded) and W
  const int KS = K / 64;                          // 64-channel steps
  const int nst = K / 128;                        // K-stages
  const int mb0 = m0 / 32, nb0 = n0 / 32;

  // ---- this wave's share of every stage's transfers: 4 code blocks + 1 scale dword ----
  const uint8_t* gsrc[4];
  int ldst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = wave * 4 + i;   // 0..15 A blocks, 16..31 B blocks; block (bl, step) = (q/2, q%2)
    if (q < 16) {
      const int b = min(mb0 + (q >> 1), MB - 1);
      gsrc[i] = a.qx + ((size_t)b * KS + (q & 1)) * 1024 + lane * 16;
      ldst[i] = kCodeA + q * 1024;
    } else {
      const int b = min(nb0 + ((q - 16) >> 1), NB - 1);
      gsrc[i] = a.qw + ((size_t)b * KS + (q & 1)) * 1024 + lane * 16;
      ldst[i] = kCodeB + (q - 16) * 1024;
    }
  }
  const uint8_t* ssrc;
  size_t sstride;
  int sdst;
  if (wave < 4) {   // A scale blocks mb0 + 2w, mb0 + 2w + 1
    const int b = min(mb0 + 2 * wave + (lane >> 5), MB - 1);
    ssrc = reinterpret_cast<const uint8_t*>(a.sx) + (size_t)b * 128 + (lane & 31) * 4;
    sstride = (size_t)MB * 128;
    sdst = kScA + wave * 256;
  } else {
    const int b = min(nb0 + 2 * (wave - 4) + (lane >> 5), NB - 1);
    ssrc = reinterpret_cast<const uint8_t*>(a.sw) + (size_t)b * 128 + (lane & 31) * 4;
    sstride = (size_t)NB * 128;
    sdst = kScB + (wave - 4) * 256;
  }

#define SVDQ_ISSUE(ST)                                                                             \
  {                                                                                                \
    uint8_t* slot = smem + ((ST) % kNStage) * kSlot;                                               \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                  \
        __builtin_amdgcn_global_load_lds(gsrc[i] + (size_t)(ST) * 2048, lds_ptr(slot + ldst[i]), 16, 0, 0); \
    __builtin_amdgcn_global_load_lds(ssrc + (size_t)(ST) * sstride, lds_ptr(slot + sdst), 4, 0, 0); \
  }

  f32x16 acc[kTN][kTM];
#pragma unroll
  for (int j = 0; j < kTN; ++j)
#pragma unroll
    for (int i = 0; i < kTM; ++i) acc[j][i] = f32x16{};

  // prologue: stages 0 .. NSTAGE-2 in flight
#pragma unroll
  for (int s = 0; s < kNStage - 1; ++s)
    if (s < nst) SVDQ_ISSUE(s)

  for (int st = 0; st < nst; ++st) {
    // this wave's transfers for stage st are done once at most min(NSTAGE-2, nst-1-st)
    // later stages (5 transfers each) are still outstanding
    const int later = min(kNStage - 2, nst - 1 - st);
    ring_barrier(5 * later);   // everyone's stage st landed; everyone finished stage st-1
    if (st + kNStage - 1 < nst) SVDQ_ISSUE(st + kNStage - 1)

    const uint8_t* slot = smem + (st % kNStage) * kSlot;
    uint32_t sa[kTM], sb[kTN];
#pragma unroll
    for (int t = 0; t < kTM; ++t)
      sa[t] = *reinterpret_cast<const uint16_t*>(slot + kScA + (wm * kTM + t) * 128 + lane * 2);
#pragma unroll
    for (int t = 0; t < kTN; ++t)
      sb[t] = *reinterpret_cast<const uint16_t*>(slot + kScB + (wn * kTN + t) * 128 + lane * 2);
#pragma unroll
    for (int step = 0; step < 2; ++step) {
      i32x8 fa[kTM], fb[kTN];
#pragma unroll
      for (int t = 0; t < kTM; ++t) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(slot + kCodeA + ((wm * kTM + t) * 2 + step) * 1024 + lane * 16);
        fa[t] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int t = 0; t < kTN; ++t) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(slot + kCodeB + ((wn * kTN + t) * 2 + step) * 1024 + lane * 16);
        fb[t] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
          if (step == 0)
            acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fb[j], fa[i], acc[j][i], 4, 4, 0, (int)sb[j], 0, (int)sa[i]);
          else
            acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fb[j], fa[i], acc[j][i], 4, 4, 1, (int)sb[j], 1, (int)sa[i]);
        }
    }
  }
#undef SVDQ_ISSUE

  // ---- epilogue: + (X_hat L1) L2 on bf16 MFMA (L2^T fragment as A, Z fragment as B) ----
  const int h = lane >> 5, lr = lane & 31;
  if (a.r32 > 0) {
    for (int c = 0; c < a.r32 / 16; ++c) {
      bf16x8 zf[kTM], lf[kTN];
#pragma unroll
      for (int t = 0; t < kTM; ++t) {
        const int row = min(m0 + wm * kWM + t * 32 + lr, M - 1);
        u32x4 v = *reinterpret_cast<const u32x4*>(a.z + (size_t)row * a.r32 + 16 * c + 8 * h);
        zf[t] = *reinterpret_cast<bf16x8*>(&v);
      }
#pragma unroll
      for (int t = 0; t < kTN; ++t) {
        const int col = min(n0 + wn * kWN + t * 32 + lr, N - 1);
        u32x4 v = *reinterpret_cast<const u32x4*>(a.l2t + (size_t)col * a.r32 + 16 * c + 8 * h);
        lf[t] = *reinterpret_cast<bf16x8*>(&v);
      }
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int i = 0; i < kTM; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf[j], zf[i], acc[j][i], 0, 0, 0);
    }
  }

  // ---- + bias, bf16; stage the wave's 128 x 64 tile in LDS, store full rows ----
  ring_barrier(0);   // the ring is free
  uint8_t* ot = smem + wave * (kWM * kOutPitch);
#pragma unroll
  for (int j = 0; j < kTN; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nl = j * 32 + 8 * q + 4 * h;             // channel within the wave tile
      const int n = min(n0 + wn * kWN + nl, N - 4);
      const u32x2 bw = *reinterpret_cast<const u32x2*>(a.bias + n);
      const float b0 = bf16lo(bw.x), b1 = bf16hi(bw.x), b2 = bf16lo(bw.y), b3 = bf16hi(bw.y);
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        u32x2 o;
        o.x = pack_bf16x2(acc[j][i][4 * q + 0] + b0, acc[j][i][4 * q + 1] + b1);
        o.y = pack_bf16x2(acc[j][i][4 * q + 2] + b2, acc[j][i][4 * q + 3] + b3);
        *reinterpret_cast<u32x2*>(ot + (i * 32 + lr) * kOutPitch + nl * 2) = o;
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int rsub = lane >> 3, chunk = lane & 7;
  const int ncol = n0 + wn * kWN + chunk * 8;
#pragma unroll 4
  for (int it = 0; it < kWM / 8; ++it) {
    const int rl = it * 8 + rsub;
    const int m = m0 + wm * kWM + rl;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ot + rl * kOutPitch + chunk * 16);
    if (m < M && ncol < N) *reinterpret_cast<u32x4*>(a.y + (size_t)m * N + ncol) = v;
  }
}

hipError_t prepare_gemm_mxfp4() {
  return hipFuncSetAttribute((const void*)gemm_mxfp4_kernel,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
}

hipError_t launch_gemm_mxfp4(const GemmArgs& a, hipStream_t st) {
  const int tm = (a.M + kBM - 1) / kBM, tn = (a.N + kBN - 1) / kBN;
  hipLaunchKernelGGL(gemm_mxfp4_kernel, dim3(tm * tn), dim3(64 * kNW), kLds, st, a, tm, tn);
  return hipGetLastError();
}

}  // namespace svdq
