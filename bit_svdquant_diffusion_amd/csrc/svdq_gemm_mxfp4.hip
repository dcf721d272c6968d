// Kernel (2) of the forward for MXFP4 layers: Q4(X_hat) Q4(R)^T on the
// block-scaled FP4 MFMA, plus the low-rank up-projection (X_hat L1) L2 and the
// bias, added before the single bf16 write of Y (aiflownews.com, "What
// SVDQuant actually does": two-branch computation, FP4 data type; "Nunchaku:
// the inference engine...": the branches share the output write).
//
// E2M1 operands and their E8M0 block scales go straight into
// v_mfma_scale_f32_32x32x64_f8f6f4: the hardware applies 2^(e_x + e_w) per
// 32-channel block and accumulates in fp32; no dequantization runs on the
// vector ALUs. The low-rank branch is r32/32 more "stages" of the same
// pipeline on v_mfma_f32_32x32x16_bf16 accumulating into the same registers.
//
// Data path. Every operand (4-bit codes, E8M0 bytes, Z = X_hat L1, L2^T) is
// stored in MFMA fragment order, one 1 KiB block per wave operand, so each
// global->LDS transfer is a direct `global_load_lds_dwordx4` of contiguous
// bytes and each LDS fragment read is a contiguous, conflict-free 1 KiB.
// Workgroups are persistent (one per CU) and walk their tiles; a ring of four
// LDS slots runs across tile boundaries with three stages in flight, so the
// next tile's first stages load while the current tile finishes and stores.
//
// Schedule. Eight waves, 2 (M) x 4 (N), each owning a 96 x 96 sub-tile of the
// 192 x 384 tile (3 x 3 blocks of 32 x 32). One workgroup barrier per stage.
// The second half (step 1) of each stage's MFMAs is issued right after the
// next barrier, so every wave enters each stage with matrix work queued while
// its LDS reads for the new stage are in flight.
#include "svdq_gemm_common.h"
#include "svdq_internal.h"

namespace svdq {

namespace {
constexpr int kBM = 192, kBN = 384, kWGM = 2, kWGN = 4, kNW = kWGM * kWGN;
constexpr int kWM = kBM / kWGM, kWN = kBN / kWGN, kTM = kWM / 32, kTN = kWN / 32;
constexpr int kMB = kBM / 32, kNBt = kBN / 32;     // 32-row blocks per tile: 6 (A), 12 (B)
constexpr int kNStage = 4;
// The 32 workgroups resident on one XCD take 8 tile-rows x 4 tile-columns:
// per K stage they share 8 A blocks of 12 KiB and 4 B blocks of 24 KiB, the
// split that minimizes the bytes the XCD's L2 must fetch for them.
constexpr int kGroupM = 8;
constexpr int kStores = 2 * 3 * 3;                 // 16-byte Y stores per wave per tile
// Transfers per stage: 36 fragment blocks of 1 KiB and 3 scale (or bias)
// transfers of up to 1 KiB, spread so that each SIMD (waves w and w + 4)
// issues 9 or 10 of them: wave w moves kFrag(w) fragment blocks starting at
// kFrag0(w), and waves 2, 3 and 6 one scale transfer each.
__host__ __device__ constexpr int kFrag(int w) { return (w & 2) ? 4 : 5; }
__host__ __device__ constexpr int kFrag0(int w) {
  return w == 0 ? 0 : w == 1 ? 5 : w == 2 ? 10 : w == 3 ? 14 : w == 4 ? 18 : w == 5 ? 23 : w == 6 ? 28 : 32;
}
__host__ __device__ constexpr int kScaleOp(int w) { return w == 2 ? 0 : (w == 3 ? 1 : (w == 6 ? 2 : -1)); }
__host__ __device__ constexpr int kOpsOf(int w) { return kFrag(w) + (kScaleOp(w) >= 0 ? 1 : 0); }
// one ring slot: A fragments (6 blocks x 2 steps x 1 KiB), B fragments (12 x 2 x 1 KiB),
// A scale bytes (6 x 128 B), B scale bytes (12 x 128 B)
constexpr int kCodeA = 0, kCodeB = kMB * 2 * 1024, kScA = kCodeB + kNBt * 2 * 1024;
constexpr int kScB = kScA + kMB * 128, kSlot = kScB + kNBt * 128;
constexpr size_t kLds = (size_t)kNStage * kSlot;
static_assert(kTM == 3 && kTN == 3, "schedule below assumes 3 x 3 blocks per wave");
static_assert(kLds <= 160 * 1024, "ring must fit in LDS");
static_assert(kFrag0(0) == 0 && kFrag0(1) == 5 && kFrag0(2) == 10 && kFrag0(3) == 14 && kFrag0(4) == 18 &&
              kFrag0(5) == 23 && kFrag0(6) == 28 && kFrag0(7) == 32 && kFrag0(7) + kFrag(7) == 2 * (kMB + kNBt),
              "fragment blocks partition");
static_assert(kMB * 128 == 768 && kNBt * 128 == 1536 && kBN * 2 == 768, "scale and bias transfer sizes");

// Ring barrier: wait until at most n of this wave's vector-memory operations
// are outstanding, and its LDS reads have returned, then s_barrier. Vector
// memory operations retire in issue order (loads and stores alike), so n =
// the number issued after the transfer being waited for. No memory fence (a
// fence would also drain the stages meant to stay in flight); scheduling
// barriers keep LDS accesses on their side.
#define SVDQ_VMCNT(n) (((n) & 15) | (((n) >> 4) << 14) | 0x0070)   /* expcnt 7, lgkmcnt 0 */
__device__ __forceinline__ void ring_barrier(int n) {
  __builtin_amdgcn_sched_barrier(0);
  switch (n) {
    case 4: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(5)); break;
    case 8: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(8)); break;
    case 10: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(10)); break;
    case 18: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(18)); break;
    case 22: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(22)); break;
    case 23: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(23)); break;
    case 26: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(26)); break;
    case 28: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(28)); break;
    default: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(0)); break;
  }
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ lds_void* lds_ptr(uint8_t* p) { return (lds_void*)p; }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};   // v_cvt_pk_bf16_f32: round to nearest even
  return *reinterpret_cast<uint32_t*>(&v);
}

struct Geo {
  int M, N, K, MB, NB, KS, nst, nlr, nstt, tiles_m, tiles_n;
};

// Ring-step transfers: direct global->LDS loads of 16 bytes per lane. A
// fragment block is 1 KiB (both 64-channel steps of a 4-bit stage, or both
// 16-column steps of Z and L2^T in a low-rank stage). The tile's scale bytes
// of a stage are contiguous in the stage-major scale layout: 768 A bytes (48
// lanes) and 1536 B bytes (64 + 32 lanes). In low-rank stages the three
// scale transfers move the tile's 384 bias values instead (48 lanes; the
// other two repeat it: same bytes to the same place). The number of
// transfers of a wave is the same in every stage. The source of every
// transfer is fixed per tile up to a per-stage offset, so each tile sets the
// sources once.
}  // namespace

__global__ __launch_bounds__(64 * kNW) void gemm_mxfp4_kernel(GemmArgs a, Geo g, int grid) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWGN, wn = wave % kWGN;
  const int h = lane >> 5, lr = lane & 31;
  const int ntiles = g.tiles_m * g.tiles_n;
  const int my_tiles = (int)blockIdx.x < ntiles ? (ntiles - 1 - (int)blockIdx.x) / grid + 1 : 0;
  const int total = my_tiles * g.nstt;   // ring steps of this workgroup

  // issue side: next ring step to load (tile-local index, stage, tile origin)
  // and this wave's per-tile transfer sources: fragment block k of the wave
  // from src[k] (4-bit) and src[5 + k] (low-rank); the scale transfer from
  // ssrc (4-bit) and bsrc (bias)
  const int nfrag = kFrag(wave), frag0 = kFrag0(wave), sop = kScaleOp(wave);
  const int nops = kOpsOf(wave);
  const int slanes = sop == 0 ? 48 : (sop == 1 ? 64 : 32);   // active lanes of the scale transfer
  int is_t = 0, is_s = 0;
  const uint8_t* src[10];
  const uint8_t* ssrc = nullptr;
  const uint8_t* bsrc = nullptr;
  int sstride = 0;   // bytes between stages of the scale transfer
  const int per_l = a.r32 / 16;
#define SVDQ_ISSUE(GS)                                                                              \
  {                                                                                                 \
    if (is_s == 0) {                                                                                \
      const TileMap tmi = map_tile((int)blockIdx.x + is_t * grid, g.tiles_m, g.tiles_n, kGroupM);   \
      const int mb0 = tmi.tm * kMB, nb0 = tmi.tn * kNBt;                                            \
      _Pragma("unroll") for (int k = 0; k < 5; ++k) {                                               \
        const int it = frag0 + k;                          /* fragment item 0..35 */               \
        const bool isA = it < 2 * kMB;                                                              \
        const int blk = isA ? (it >> 1) : ((it - 2 * kMB) >> 1);                                     \
        const size_t b = (size_t)min((isA ? mb0 : nb0) + blk, (isA ? g.MB : g.NB) - 1);             \
        src[k] = (isA ? a.qx : a.qw) + (b * g.KS + (it & 1)) * 1024 + lane * 16;                    \
        src[5 + k] = reinterpret_cast<const uint8_t*>(isA ? a.z : a.l2t) + (b * per_l + (it & 1)) * 1024 + lane * 16; \
      }                                                                                             \
      {                                                                                             \
        const bool isA = sop == 0;                                                                  \
        const int blk = (sop == 2 ? 8 : 0) + (lane >> 3);                                           \
        const int b = min((isA ? mb0 : nb0) + blk, (isA ? g.MB : g.NB) - 1);                        \
        ssrc = reinterpret_cast<const uint8_t*>(isA ? a.sx : a.sw) + (size_t)b * 128 + (lane & 7) * 16; \
        sstride = (isA ? g.MB : g.NB) * 128;                                                        \
        bsrc = reinterpret_cast<const uint8_t*>(a.bias + min(nb0 * 32 + 8 * lane, g.N - 8));        \
      }                                                                                             \
    }                                                                                               \
    uint8_t* slot_w = smem + ((GS) % kNStage) * kSlot;                                              \
    const bool lrs = is_s >= g.nst;                                                                 \
    const int sl = lrs ? is_s - g.nst : is_s;                                                       \
    if (lrs && a.r32 == 0) {                                                                        \
      /* no low-rank fragments: every transfer of the stage moves the bias */                      \
      _Pragma("unroll") for (int k = 0; k < 6; ++k)                                                 \
        if (k < nops && lane < 48) __builtin_amdgcn_global_load_lds(bsrc, lds_ptr(slot_w + kScA), 16, 0, 0); \
    } else {                                                                                        \
      _Pragma("unroll") for (int k = 0; k < 5; ++k) {                                               \
        if (k < nfrag) {                                                                            \
          const int it = frag0 + k;                                                                 \
          const int dst = it < 2 * kMB ? kCodeA + it * 1024 : kCodeB + (it - 2 * kMB) * 1024;       \
          __builtin_amdgcn_global_load_lds(src[(lrs ? 5 : 0) + k] + (size_t)sl * 2048, lds_ptr(slot_w + dst), 16, 0, 0); \
        }                                                                                           \
      }                                                                                             \
      if (sop >= 0 && lane < (lrs ? 48 : slanes)) {                                                 \
        if (lrs)                                                                                    \
          __builtin_amdgcn_global_load_lds(bsrc, lds_ptr(slot_w + kScA), 16, 0, 0);                 \
        else                                                                                        \
          __builtin_amdgcn_global_load_lds(ssrc + (size_t)sl * sstride,                             \
                                           lds_ptr(slot_w + (sop == 0 ? kScA : kScB + (sop == 2 ? 1024 : 0))), 16, 0, 0); \
      }                                                                                             \
    }                                                                                               \
    if (++is_s == g.nstt) {                                                                         \
      is_s = 0;                                                                                     \
      ++is_t;                                                                                       \
    }                                                                                               \
  }

  f32x16 acc[kTN][kTM];
  i32x4 f0a[kTM], f0b[kTN], f1a[kTM], f1b[kTN];
  uint32_t sa[kTM] = {0, 0, 0}, sb[kTN] = {0, 0, 0}, pa[kTM], pb[kTN];

#define SVDQ_READ(SLOT, STEP, FA, FB)                                                               \
  {                                                                                                 \
    _Pragma("unroll") for (int t = 0; t < kTM; ++t)                                                 \
        FA[t] = *reinterpret_cast<const i32x4*>((SLOT) + kCodeA + ((wm * kTM + t) * 2 + (STEP)) * 1024 + lane * 16); \
    _Pragma("unroll") for (int t = 0; t < kTN; ++t)                                                 \
        FB[t] = *reinterpret_cast<const i32x4*>((SLOT) + kCodeB + ((wn * kTN + t) * 2 + (STEP)) * 1024 + lane * 16); \
  }
  // MFMAs of one step, weight fragment as operand A and activation fragment as
  // operand B: 4-bit (scaled, opsel = step) or low-rank (bf16)
#define SVDQ_MFMA(LOWRANK, STEP, FA, FB, XA, XB)                                                    \
  {                                                                                                 \
    if constexpr (!(LOWRANK)) {                                                                     \
      _Pragma("unroll") for (int j = 0; j < kTN; ++j) _Pragma("unroll") for (int i = 0; i < kTM; ++i) \
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                               \
              i32x8{FB[j][0], FB[j][1], FB[j][2], FB[j][3], 0, 0, 0, 0},                              \
              i32x8{FA[i][0], FA[i][1], FA[i][2], FA[i][3], 0, 0, 0, 0}, acc[j][i], 4, 4, (STEP),     \
              (int)XB[j], (STEP), (int)XA[i]);                                                        \
    } else {                                                                                        \
      _Pragma("unroll") for (int j = 0; j < kTN; ++j) _Pragma("unroll") for (int i = 0; i < kTM; ++i) \
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, FB[j]),      \
                                                             __builtin_bit_cast(bf16x8, FA[i]), acc[j][i], 0, 0, 0); \
    }                                                                                               \
  }
  // One ring step. The deferred second half of the previous step's MFMAs goes
  // first, so the matrix pipe has work while this step's step-0 fragments
  // load; the step-1 fragments are read behind the step-0 MFMAs.
  // Waves 0-3 issue their transfers for ring step gs + 3 before their LDS
  // reads, waves 4-7 after their step-0 MFMAs, so each SIMD's two waves do
  // not stall on transfer issue at the same time. `stores_due` counts the
  // ring steps whose wait must also let the last tile's Y stores stay in
  // flight.
#define SVDQ_STEP(LOWRANK, LAST, DO_MFMA)                                                           \
  {                                                                                                 \
    ring_barrier(nops * min(kNStage - 2, total - 1 - gs) + (stores_due > 0 ? kStores : 0));         \
    if (stores_due > 0) --stores_due;                                                               \
    if (pending) {                                                                                  \
      SVDQ_MFMA(LOWRANK, 1, f1a, f1b, pa, pb)                                                       \
      pending = false;                                                                              \
    }                                                                                               \
    const bool more = gs + kNStage - 1 < total;                                                     \
    if (more && wave < 4) SVDQ_ISSUE(gs + kNStage - 1)                                              \
    const uint8_t* slot = smem + (gs % kNStage) * kSlot;                                            \
    if (DO_MFMA) {                                                                                  \
      if (!(LOWRANK)) {                                                                             \
        _Pragma("unroll") for (int t = 0; t < kTM; ++t)                                             \
            sa[t] = *reinterpret_cast<const uint16_t*>(slot + kScA + (wm * kTM + t) * 128 + lane * 2); \
        _Pragma("unroll") for (int t = 0; t < kTN; ++t)                                             \
            sb[t] = *reinterpret_cast<const uint16_t*>(slot + kScB + (wn * kTN + t) * 128 + lane * 2); \
      }                                                                                             \
      SVDQ_READ(slot, 0, f0a, f0b)                                                                  \
      SVDQ_MFMA(LOWRANK, 0, f0a, f0b, sa, sb)                                                       \
      SVDQ_READ(slot, 1, f1a, f1b)   /* used by the deferred MFMAs: loads behind step 0 */         \
      if (more && wave >= 4) SVDQ_ISSUE(gs + kNStage - 1)                                           \
      _Pragma("unroll") for (int t = 0; t < kTM; ++t) pa[t] = sa[t];                                \
      _Pragma("unroll") for (int t = 0; t < kTN; ++t) pb[t] = sb[t];                                \
      if (LAST) {                                                                                   \
        SVDQ_MFMA(LOWRANK, 1, f1a, f1b, pa, pb)                                                     \
      } else {                                                                                      \
        pending = true;                                                                             \
      }                                                                                             \
    } else if (more && wave >= 4) {                                                                 \
      SVDQ_ISSUE(gs + kNStage - 1)                                                                  \
    }                                                                                               \
    ++gs;                                                                                           \
  }

  bool pending = false;   // deferred step-1 MFMAs of the previous ring step
  int gs = 0, stores_due = 0;
  const int nlr = g.nstt - g.nst;
  // prologue: the first kNStage - 1 ring steps in flight
  for (int p = 0; p < kNStage - 1 && p < total; ++p) SVDQ_ISSUE(p)
  for (int ct = 0; ct < my_tiles; ++ct) {
    const TileMap tmc = map_tile((int)blockIdx.x + ct * grid, g.tiles_m, g.tiles_n, kGroupM);
    const int n0 = tmc.tn * kBN + wn * kWN;
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int i = 0; i < kTM; ++i) acc[j][i] = f32x16{};
    for (int s4 = 0; s4 < g.nst; ++s4) SVDQ_STEP(false, s4 == g.nst - 1, true)
    for (int l = 0; l < nlr; ++l) SVDQ_STEP(true, l == nlr - 1, a.r32 > 0)

    // + bias (from the last low-rank slot), bf16. The accumulator lane holds
    // token m0 + 32 i + lr and channels 32 j + 8 q + 4 h + (0..3); swapping the
    // packed pairs (q = 1, h = 0) <-> (q = 0, h = 1) and (q = 3, h = 0) <->
    // (q = 2, h = 1) between the lane halves leaves lane h with channels
    // 32 j + 8 h + (0..7) and 32 j + 16 + 8 h + (0..7): two 16-byte stores,
    // 32 contiguous bytes of one row per lane pair.
    const uint8_t* bslot = smem + ((gs - 1) % kNStage) * kSlot + kScA + wn * kWN * 2;
    // Y rows of this tile as a buffer resource: stores past its end are dropped
    const int ynrec = min(g.M - tmc.tm * kBM, kBM) * g.N * 2;
    const __amdgpu_buffer_rsrc_t yrs =
        __builtin_amdgcn_make_buffer_rsrc(a.y + (size_t)tmc.tm * kBM * g.N, 0, ynrec, 0x00020000);
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      float bv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 bw = *reinterpret_cast<const u32x2*>(bslot + (32 * j + 8 * q + 4 * h) * 2);
        bv[4 * q + 0] = bf16lo(bw.x);
        bv[4 * q + 1] = bf16hi(bw.x);
        bv[4 * q + 2] = bf16lo(bw.y);
        bv[4 * q + 3] = bf16hi(bw.y);
      }
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        uint32_t o[8];
#pragma unroll
        for (int p = 0; p < 8; ++p)
          o[p] = cvt_bf16x2(acc[j][i][2 * p] + bv[2 * p], acc[j][i][2 * p + 1] + bv[2 * p + 1]);
#pragma unroll
        for (int p = 0; p < 2; ++p) {   // (o[4p], o[4p+1]) is q = 2p, (o[4p+2], o[4p+3]) is q = 2p+1
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            const auto r = __builtin_amdgcn_permlane32_swap(o[4 * p + w], o[4 * p + 2 + w], false, false);
            o[4 * p + w] = r[0];
            o[4 * p + 2 + w] = r[1];
          }
        }
        // always issued (the ring waits count them); the resource drops rows
        // past M and a block past N is sent past the end
        const int col = n0 + 32 * j + 8 * h;
        const int off = col < g.N ? ((wm * kWM + 32 * i + lr) * g.N + col) * 2 : ynrec;
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{o[0], o[1], o[2], o[3]}, yrs, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{o[4], o[5], o[6], o[7]}, yrs, col < g.N ? off + 32 : ynrec, 0, 0);
      }
    }
    stores_due = kNStage - 1;
  }
#undef SVDQ_STEP
#undef SVDQ_READ
#undef SVDQ_MFMA
#undef SVDQ_ISSUE
#undef SVDQ_READ
#undef SVDQ_MFMA
}

hipError_t prepare_gemm_mxfp4() {
  return hipFuncSetAttribute((const void*)gemm_mxfp4_kernel,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
}

hipError_t launch_gemm_mxfp4(const GemmArgs& a, int num_cus, hipStream_t st) {
  Geo g;
  g.M = a.M;
  g.N = a.N;
  g.K = a.K;
  g.MB = (a.M + 31) / 32;
  g.NB = a.N / 32;
  g.KS = a.K / 64;
  g.nst = a.K / 128;
  g.nlr = a.r32 > 0 ? a.r32 / 32 : 1;   // at least one: the bias rides in a low-rank stage
  g.nstt = g.nst + g.nlr;
  g.tiles_m = (a.M + kBM - 1) / kBM;
  g.tiles_n = (a.N + kBN - 1) / kBN;
  const int ntiles = g.tiles_m * g.tiles_n;
  // persistent grid: one workgroup per CU, a multiple of 8 so each stays on its XCD's tiles
  int grid = num_cus > 0 ? num_cus : 256;
  if (grid > ntiles) grid = ntiles;
  hipLaunchKernelGGL(gemm_mxfp4_kernel, dim3(grid), dim3(64 * kNW), kLds, st, a, g, grid);
  return hipGetLastError();
}

}  // namespace svdq
