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
// global->LDS transfer is a direct `buffer_load_dwordx4 ... lds` of
// contiguous bytes and each LDS fragment read is a contiguous,
// conflict-free 1 KiB. (The buffer form with a 32-bit lane offset runs
// beside the other wave's MFMAs on a SIMD; the 64-bit-address global form
// measured mostly additive to them.)
// Workgroups are persistent (one per CU) and walk their tiles; a ring of four
// LDS slots runs across tile boundaries with three stages in flight, so the
// next tile's first stages load while the current tile finishes and stores.
//
// Schedule. Eight waves, 2 (M) x 4 (N), each owning a 96 x 96 sub-tile of the
// 192 x 384 tile (3 x 3 blocks of 32 x 32). One workgroup barrier per stage.
// The second half (step 1) of each stage's MFMAs is deferred past the next
// barrier and runs while that stage's first fragments load. The per-stage
// control is kept to a few scalar instructions (a uniform transfer count, one
// wait form, per-wave LDS read offsets fixed once): on a SIMD the issue of
// other instructions adds to the MFMA time rather than hiding under it.
#include "svdq_gemm_common.h"
#include "svdq_internal.h"
#include "svdq_layout.h"

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
// transfers of 1 KiB (the scale areas of a slot are padded to whole KiB, so
// every transfer uses all 64 lanes). Every wave issues kOps = 5 per stage:
// waves 0-2 four of the 12 A blocks and one scale (bias) transfer, waves 3-7
// five of the 24 B blocks (wave 7 repeats its last block: same bytes to the
// same place). Each wave reads a single operand.
constexpr int kOps = 5;
// LDS position p of a B block (0..11 in a tile) holds the tile's block
// bperm(p): odd wave columns take their three blocks in reverse. Two waves
// share a 128-byte line of a Y row (tile blocks 2 and 3, and 8 and 9); with
// the reversal both store their halves of it at the same epilogue step
// (j = 2), so the line is whole when it leaves L2. An involution; positions
// past the tile's blocks (scale and bias padding) map to themselves.
__host__ __device__ constexpr int bperm(int p) {
  return p < kNBt && ((p / kTN) & 1) ? p / kTN * kTN + (kTN - 1) - p % kTN : p;
}
static_assert(bperm(2) == 2 && bperm(3) == 5 && bperm(5) == 3 && bperm(8) == 8 && bperm(9) == 11 &&
                  bperm(11) == 9 && bperm(12) == 12,
              "shared lines (blocks 2|3, 8|9) at the same step of both waves");
__host__ __device__ constexpr int kItem(int w, int k) {   // fragment item 0..35 of transfer k of wave w
  return w < 3 ? 4 * w + k : (12 + 5 * (w - 3) + k < 36 ? 12 + 5 * (w - 3) + k : 35);
}
// one ring slot: A fragments (6 blocks x 2 steps x 1 KiB), B fragments (12 x 2 x 1 KiB),
// A scale bytes (6 x 128 B, padded to 1 KiB), B scale bytes (12 x 128 B, padded to 2 KiB);
// low-rank stages carry the bias in the A scale area
constexpr int kCodeA = 0, kCodeB = kMB * 2 * 1024, kScA = kCodeB + kNBt * 2 * 1024;
constexpr int kScB = kScA + 1024, kSlot = kScB + 2048;
constexpr size_t kLds = (size_t)kNStage * kSlot;
static_assert(kTM == 3 && kTN == 3, "schedule below assumes 3 x 3 blocks per wave");
static_assert(kLds <= 160 * 1024, "ring must fit in LDS");
static_assert((kNStage & (kNStage - 1)) == 0, "ring index is a mask");
static_assert(kItem(2, 3) == 2 * kMB - 1 && kItem(3, 0) == 2 * kMB && kItem(7, 3) == 2 * (kMB + kNBt) - 1,
              "fragment blocks partition");
static_assert(kCodeB == 2 * kMB * 1024, "fragment item it sits at it KiB");
static_assert(kMB * 128 <= 1024 && kNBt * 128 <= 2048 && kBN * 2 <= 1024, "scale and bias transfer sizes");

// Ring barrier: wait until at most n of this wave's vector-memory operations
// are outstanding, and its LDS reads have returned, then s_barrier. Vector
// memory operations retire in issue order (loads and stores alike), so n =
// the number issued after the transfer being waited for. No memory fence (a
// fence would also drain the stages meant to stay in flight); scheduling
// barriers keep LDS accesses on their side.
#define SVDQ_VMCNT(n) (((n) & 15) | (((n) >> 4) << 14) | 0x0070)   /* expcnt 7, lgkmcnt 0 */
// Every ring step issues the transfers of the step three ahead (past the
// end of the work they repeat the last tile's), so two later steps are
// always in flight: the wait is for all but 2 kOps of the wave's transfers,
// plus the last tile's Y stores while they are still counted.
// FUSE: the fused epilogue's stores instead, nstores of them (up to 48);
// a count past the cases waits for all outstanding operations.
template <bool FUSE>
__device__ __forceinline__ void ring_barrier(bool stores, int nstores) {
  __builtin_amdgcn_sched_barrier(0);
  if (!stores) {
    __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(2 * kOps));
  } else if constexpr (!FUSE) {
    __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(2 * kOps + kStores));
  } else {
#define SVDQ_FWAIT(k) \
  case k: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(2 * kOps + k)); break;
    switch (nstores) {
      SVDQ_FWAIT(18) SVDQ_FWAIT(21) SVDQ_FWAIT(24) SVDQ_FWAIT(27) SVDQ_FWAIT(30)
      SVDQ_FWAIT(33) SVDQ_FWAIT(36) SVDQ_FWAIT(39) SVDQ_FWAIT(42) SVDQ_FWAIT(45) SVDQ_FWAIT(48)
      default: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(0)); break;
    }
#undef SVDQ_FWAIT
  }
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}
static_assert(2 * kOps + kStores < 64 && 2 * kOps + 48 < 64, "vmcnt range");

// Word 3 of the buffer resources: 32-bit data format, no swizzle, no added
// thread id (untyped loads and stores ignore the rest).
constexpr int kRsrcWord3 = 0x00020000;

typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ lds_void* lds_ptr(uint8_t* p) { return (lds_void*)p; }


struct Geo {
  int M, N, K, MB, NB, KS, nst, nlr, nstt, tiles_m, tiles_n;   // N, K padded
  int ldy;   // Y's row stride and width (the layer's N)
};

// Ring-step transfers: direct global->LDS loads of 16 bytes per lane. A
// fragment block is 1 KiB (both 64-channel steps of a 4-bit stage, or both
// 16-column steps of Z and L2^T in a low-rank stage). The tile's scale bytes
// of a stage are contiguous in the stage-major scale layout: 768 A bytes and
// 1536 B bytes, moved as three full-wave transfers whose extra lanes read
// neighbouring (clamped, in-bounds) scale bytes into the padding. In
// low-rank stages those three transfers move the tile's 384 bias values
// instead. The source of every transfer is fixed per tile up to a per-stage
// offset, so each tile sets the sources once.
}  // namespace

// FUSE: the tile's output is the next layer's input (GELU between them):
// see fused_tile below.
template <bool FUSE>
__global__ __launch_bounds__(64 * kNW) void gemm_mxfp4_kernel(GemmArgs a, Geo g, int grid) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWGN, wn = wave % kWGN;
  const int h = lane >> 5, lr = lane & 31;
  const int ntiles = g.tiles_m * g.tiles_n;
  const int my_tiles = (int)blockIdx.x < ntiles ? (ntiles - 1 - (int)blockIdx.x) / grid + 1 : 0;

  // issue side: next ring step to load (tile-local index, stage). Transfers
  // are buffer loads into LDS. Per tile, the rows of the wave's operand that
  // the tile covers become a buffer resource (rcur: the 4-bit codes; rlow:
  // the low-rank fragments, which replace them for the low-rank stages), and
  // transfer k reads at lane offset vcur[k] from it, plus the stage offset
  // soffs. Waves 0-2 take their scale bytes from a per-tile resource at lane
  // offset soff plus the stage offset ssoffs (32 bits: the shape check keeps
  // K * ceil(M / 32) below 2^31), and the bias from the whole vector at lane
  // offset boff.
  const bool opA = wave < 3;   // this wave's operand: A (X side) or B (W side)
  const int per_l = a.r32 / 16;
  int is_t = 0, is_s = 0;
  __amdgpu_buffer_rsrc_t rcur = __builtin_amdgcn_make_buffer_rsrc(nullptr, 0, 0, 0), rlow = rcur;
  __amdgpu_buffer_rsrc_t rsc = rcur;    // scale bytes of the tile's first block
  uint32_t vcur[kOps], vlow[kOps], soffs = 0, ssoffs = 0;   // stage offsets: fragments, scale bytes
  int sstride = 0, soff = 0, boff = 0;  // scale bytes between stages; lane offsets of the scale and bias transfers
  const int sdst = wave == 0 ? kScA : kScB + (wave == 2 ? 1024 : 0);   // LDS offset of the scale transfer
#define SVDQ_ISSUE(GS)                                                                              \
  {                                                                                                 \
    if (is_s == 0) {                                                                                \
      const TileMap tmi = map_tile((int)blockIdx.x + min(is_t, my_tiles - 1) * grid, g.tiles_m, g.tiles_n, kGroupM); \
      const int mb0 = tmi.tm * kMB, nb0 = tmi.tn * kNBt;                                            \
      const int b0 = opA ? mb0 : nb0, nbl = opA ? min(g.MB - mb0, kMB) : min(g.NB - nb0, kNBt);    \
      rcur = __builtin_amdgcn_make_buffer_rsrc((void*)((opA ? a.qx : a.qw) + (size_t)b0 * g.KS * 1024), 0, \
                                               nbl * g.KS * 1024, kRsrcWord3);                      \
      rlow = __builtin_amdgcn_make_buffer_rsrc((void*)((opA ? a.z : a.l2t) + (size_t)b0 * per_l * 512), 0, \
                                               nbl * per_l * 1024, kRsrcWord3);                     \
      _Pragma("unroll") for (int k = 0; k < kOps; ++k) {                                            \
        const int it = kItem(wave, k) - (opA ? 0 : 2 * kMB);   /* item within the operand */       \
        const int bl = min(opA ? it >> 1 : bperm(it >> 1), nbl - 1);   /* block within the tile */ \
        vcur[k] = (uint32_t)((bl * g.KS + (it & 1)) * 1024 + lane * 16);                            \
        vlow[k] = (uint32_t)((bl * per_l + (it & 1)) * 1024 + lane * 16);                           \
      }                                                                                             \
      soffs = 0;                                                                                    \
      {                                                                                             \
        const bool isA = wave == 0;                                                                 \
        const int base = isA ? mb0 : nb0, lim = isA ? g.MB : g.NB;                                  \
        const int blk = (wave == 2 ? 8 : 0) + (lane >> 3);                                          \
        sstride = lim * 128;                                                                        \
        rsc = __builtin_amdgcn_make_buffer_rsrc(                                                    \
            (void*)(reinterpret_cast<const uint8_t*>(isA ? a.sx : a.sw) + (size_t)base * 128), 0,    \
            (g.nst - 1) * sstride + (lim - base) * 128, kRsrcWord3);                                \
        soff = (min(base + (isA ? blk : bperm(blk)), lim - 1) - base) * 128 + (lane & 7) * 16;      \
        ssoffs = 0;                                                                                 \
        boff = min(nb0 * 32 + 32 * bperm(lane >> 2) + 8 * (lane & 3), g.N - 8) * 2;                 \
      }                                                                                             \
    } else if (is_s == g.nst) {                                                                     \
      rcur = rlow;                                                                                  \
      _Pragma("unroll") for (int k = 0; k < kOps; ++k) vcur[k] = vlow[k];                           \
      soffs = 0;                                                                                    \
    }                                                                                               \
    uint8_t* slot_w = smem + ((GS) & (kNStage - 1)) * kSlot;                                              \
    _Pragma("unroll") for (int k = 0; k < kOps - 1; ++k)                                            \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rcur, lds_ptr(slot_w + kItem(wave, k) * 1024), 16, vcur[k], soffs, 0, 0); \
    if (!opA) {                                                                                     \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rcur, lds_ptr(slot_w + kItem(wave, kOps - 1) * 1024), 16, \
                                               vcur[kOps - 1], soffs, 0, 0);                        \
    } else if (is_s < g.nst) {                                                                      \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, lds_ptr(slot_w + sdst), 16, soff, ssoffs, 0, 0); \
      ssoffs += sstride;                                                                            \
    } else {                                                                                        \
      const __amdgpu_buffer_rsrc_t rbias = __builtin_amdgcn_make_buffer_rsrc((void*)a.bias, 0, g.N * 2, kRsrcWord3); \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rbias, lds_ptr(slot_w + sdst), 16, boff, 0, 0, 0);   \
    }                                                                                               \
    soffs += 2048;                                                                                  \
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
        FA[t] = *reinterpret_cast<const i32x4*>(smem + rd_a + (SLOT) + (2 * t + (STEP)) * 1024);     \
    _Pragma("unroll") for (int t = 0; t < kTN; ++t)                                                 \
        FB[t] = *reinterpret_cast<const i32x4*>(smem + rd_b + (SLOT) + (2 * t + (STEP)) * 1024);     \
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
  // One ring step. This step's step-0 fragments (and scale bytes) are read
  // first; the deferred second half of the previous step's MFMAs runs while
  // they load, then the step-0 MFMAs, with the step-1 fragments read behind
  // them for the next step's deferred half. Waves 0-3 issue their transfers
  // for ring step gs + 3 right after the barrier, waves 4-7 after their
  // step-0 MFMAs, so each SIMD's two waves do not issue at the same time.
  // `stores_due` counts the ring steps whose wait must also let the last
  // tile's Y stores stay in flight.
#define SVDQ_STEP(LOWRANK, LAST, DO_MFMA)                                                           \
  {                                                                                                 \
    ring_barrier<FUSE>(stores_due > 0, nstores);                                                    \
    if (stores_due > 0) --stores_due;                                                               \
    if (wave < 4) SVDQ_ISSUE(gs + kNStage - 1)                                                      \
    const uint32_t slot = (gs & (kNStage - 1)) * kSlot;                                                   \
    if (DO_MFMA) {                                                                                  \
      if (!(LOWRANK)) {                                                                             \
        _Pragma("unroll") for (int t = 0; t < kTM; ++t)                                             \
            sa[t] = *reinterpret_cast<const uint16_t*>(smem + rs_a + slot + t * 128);                \
        _Pragma("unroll") for (int t = 0; t < kTN; ++t)                                             \
            sb[t] = *reinterpret_cast<const uint16_t*>(smem + rs_b + slot + t * 128);                \
      }                                                                                             \
      SVDQ_READ(slot, 0, f0a, f0b)                                                                  \
    }                                                                                               \
    if (pending) {                                                                                  \
      SVDQ_MFMA(LOWRANK, 1, f1a, f1b, pa, pb)                                                       \
      pending = false;                                                                              \
    }                                                                                               \
    if (DO_MFMA) {                                                                                  \
      SVDQ_MFMA(LOWRANK, 0, f0a, f0b, sa, sb)                                                       \
      SVDQ_READ(slot, 1, f1a, f1b)                                                                  \
      if (wave >= 4) SVDQ_ISSUE(gs + kNStage - 1)                                                   \
      _Pragma("unroll") for (int t = 0; t < kTM; ++t) pa[t] = sa[t];                                \
      _Pragma("unroll") for (int t = 0; t < kTN; ++t) pb[t] = sb[t];                                \
      if (LAST) {                                                                                   \
        SVDQ_MFMA(LOWRANK, 1, f1a, f1b, pa, pb)                                                     \
      } else {                                                                                      \
        pending = true;                                                                             \
      }                                                                                             \
    } else if (wave >= 4) {                                                                         \
      SVDQ_ISSUE(gs + kNStage - 1)                                                                  \
    }                                                                                               \
    ++gs;                                                                                           \
  }

  bool pending = false;   // deferred step-1 MFMAs of the previous ring step
  int gs = 0, stores_due = 0;
  // stores of one tile's epilogue per wave (the same in every wave)
  const int nstores = FUSE ? kTM * kTN * 2 + kTM * (a.nxt_r32 / 32) : kStores;
  const int nlr = g.nstt - g.nst;
  // this wave's LDS read offsets within a slot: fragment blocks and scale bytes
  const uint32_t rd_a = kCodeA + wm * kTM * 2048 + lane * 16, rd_b = kCodeB + wn * kTN * 2048 + lane * 16;
  const uint32_t rs_a = kScA + wm * kTM * 128 + lane * 2, rs_b = kScB + wn * kTN * 128 + lane * 2;
  // FUSE: instead of Y, this wave's 96 x 96 of GELU(bf16(acc + bias)) (a bf16
  // value, as a separate GELU over bf16 Y would give) becomes the next MXFP4
  // layer's input, smoothed by its mu: first the partial X_hat L1 over the
  // tile's 384 channels on bf16 MFMAs (each wave its 96 channels; the four
  // wave columns' partials added in column order through LDS, in the ring
  // slot the tile's last step used, by all eight waves, one 16-byte store per
  // lane), then each token's three 32-channel blocks quantized by the stage-1
  // quantizer: E8M0 scale byte and E2M1 codes in the stage-1 fragment order
  // (the two lanes of a token trade 4-channel runs so that each stores 8
  // contiguous bytes). Every store is issued by every wave (lanes past M, or
  // not holding a scale, aim past the end of their buffer): kTM kTN 2 + kTM
  // r32 / 32 of them, which the next ring waits count.
  auto fused_tile = [&](int tm, int tn, const uint8_t* bslot, uint8_t* zslot) {
    const int nr = a.nxt_r32, Kd = g.N, rows32 = g.MB * 32;
    const int m0t = tm * kBM;
    float* zred = reinterpret_cast<float*>(zslot);   // [wave column][wave row][16][64]
    const uint32_t zbytes = (uint32_t)((size_t)g.tiles_n * g.M * nr * 4);
    const uint32_t qbytes = (uint32_t)((size_t)rows32 * Kd / 2);
    const uint32_t sbytes = (uint32_t)((size_t)(Kd / 128) * g.MB * 128);
    // mu and L1 of the next layer through buffer resources: a lane offset
    // plus wave-uniform offsets, so their addresses take few registers
    const __amdgpu_buffer_rsrc_t rmu = __builtin_amdgcn_make_buffer_rsrc((void*)a.nxt_mu, 0, Kd * 4, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rl1 =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.nxt_l1s, 0, (uint32_t)Kd * (nr > 0 ? nr : 1) * 2, kRsrcWord3);
    // the Z reduction's share of thread tid: wave row zr, token ztk of the
    // block, ranks zc .. zc + 3; in the 32 x 32 accumulator layout that is
    // register 4 (ztk / 8) + ztk % 4 of lanes zc + 32 ((ztk / 4) % 2) + (0..3)
    const int zr = tid >> 8, ztk = (tid >> 3) & 31, zc = 4 * (tid & 7);
    const int zoff = ((zr * 16 + 4 * (ztk / 8) + ztk % 4) * 64) + zc + 32 * ((ztk / 4) % 2);
    // one 32-token block at a time (acc of the later blocks stays live)
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      // GELU(bf16(acc + bias)) as packed bf16 pairs: hb[j][p] holds
      // accumulator values 2 p and 2 p + 1 of block (j, i)
      uint32_t hb[kTN][8];
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x2 bw = *reinterpret_cast<const u32x2*>(bslot + (32 * j + 8 * q + 4 * h) * 2);
          const uint32_t y0 = cvt_bf16x2(acc[j][i][4 * q + 0] + bf16lo(bw.x), acc[j][i][4 * q + 1] + bf16hi(bw.x));
          const uint32_t y1 = cvt_bf16x2(acc[j][i][4 * q + 2] + bf16lo(bw.y), acc[j][i][4 * q + 3] + bf16hi(bw.y));
          hb[j][2 * q] = cvt_bf16x2(gelu_f32(bf16lo(y0)), gelu_f32(bf16hi(y0)));
          hb[j][2 * q + 1] = cvt_bf16x2(gelu_f32(bf16lo(y1)), gelu_f32(bf16hi(y1)));
        }
      // x_hat of values 8 m .. 8 m + 7 of block j (channels 32 cb + 16 m +
      // 4 h + (0..3, 8..11)): the bf16 GELU times the next layer's mu
      auto xhat8 = [&](int j, int m, int cb, float* o) {
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          const f32x4 m4 = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(rmu, 16 * h, (32 * cb + 16 * m + 8 * qq) * 4, 0));
          const uint32_t p0 = hb[j][4 * m + 2 * qq], p1 = hb[j][4 * m + 2 * qq + 1];
          o[4 * qq + 0] = bf16lo(p0) * m4[0];
          o[4 * qq + 1] = bf16hi(p0) * m4[1];
          o[4 * qq + 2] = bf16lo(p1) * m4[2];
          o[4 * qq + 3] = bf16hi(p1) * m4[3];
        }
      };
      for (int rb = 0; rb < nr / 32; ++rb) {
        // A: the token's x_hat of channels 32 cb + 16 m + 4 h + (0..3, 8..11)
        // as bf16; B: the same channels' L1 rows for rank 32 rb + lr, 8
        // bytes per 4 channels of the stage-1 layout [K/256][4][r32/16][2]
        // [64][8]: channel k = 32 cb + 16 m + 8 u + 4 h, column col sits at
        // element (((k/256 4 + (k%256)/64) r32/16 + col/16) 2 + u) 512 +
        // (16 ((k%64)/16) + col%16) 8 + 4 h
        const uint32_t lane_off = ((lr / 16) * 1024 + (lr % 16) * 8 + 4 * h) * 2;
        f32x16 zacc = f32x16{};
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
          const int cb = tn * kNBt + bperm(wn * kTN + j);
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            u32x2 bl[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int sel = (((cb / 8) * 4 + (cb % 8) / 2) * (nr / 16) + 2 * rb) * 1024 + u * 512 +
                              (32 * (cb % 2) + 16 * m) * 8;
              bl[u] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rl1, lane_off, sel * 2, 0));
            }
            float x8[8];
            xhat8(j, m, cb, x8);
            const u32x4 av = u32x4{cvt_bf16x2(x8[0], x8[1]), cvt_bf16x2(x8[2], x8[3]), cvt_bf16x2(x8[4], x8[5]),
                                   cvt_bf16x2(x8[6], x8[7])};
            zacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                           __builtin_bit_cast(bf16x8, u32x4{bl[0][0], bl[0][1], bl[1][0], bl[1][1]}),
                                                           zacc, 0, 0, 0);
          }
        }
        // the slot's fragments (first time) or the last block's partials are read
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 16; ++e) zred[(((wn * kWGM + wm) * 16 + e) * 64) + lane] = zacc[e];
        __syncthreads();
        f32x4 zs = *reinterpret_cast<const f32x4*>(zred + zoff);
#pragma unroll
        for (int c = 1; c < kWGN; ++c) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(zred + c * (kWGM * 16 * 64) + zoff);
#pragma unroll
          for (int e = 0; e < 4; ++e) zs[e] += v[e];
        }
        const int tz = m0t + zr * kWM + 32 * i + ztk;
        const uint32_t zo = tz < g.M ? (uint32_t)((((size_t)tn * g.M + tz) * nr + 32 * rb + zc) * 4) : zbytes;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, zs),
                                               __builtin_amdgcn_make_buffer_rsrc(a.nxt_zpart, 0, zbytes, kRsrcWord3),
                                               zo, 0, 0);
      }
      // each token's three 32-channel blocks: E8M0 scale byte and E2M1 codes
      const int t = m0t + wm * kWM + 32 * i + lr;   // the lane's token
      const bool live = t < g.M;                    // rows past M stay unwritten, as stage 1 leaves them
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        const int cb = tn * kNBt + bperm(wn * kTN + j);
        float v[16];
        xhat8(j, 0, cb, v);
        xhat8(j, 1, cb, v + 8);
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[e]));
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));   // the block's other 16 channels
        const int ex = mx_exponent(amax);
        // runs r = 2 q + h of 4 channels: A holds runs h and 2 + h, B runs
        // 4 + h and 6 + h; after the swap lane h holds runs 4h .. 4h + 3
        const uint32_t ca = e2m1x8_codes(v, ex), cbw = e2m1x8_codes(v + 8, ex);
        const auto sw = __builtin_amdgcn_permlane32_swap(ca, cbw, false, false);
        const uint32_t w0 = (sw[0] & 0xFFFFu) | (sw[1] << 16), w1 = (sw[0] >> 16) | (sw[1] & 0xFFFF0000u);
        const uint32_t qo = live ? (uint32_t)f_code_byte(Kd, t, 32 * cb + 16 * h) : qbytes;
        const uint32_t so = live && h == 0 ? (uint32_t)f_scale_index(rows32, t, cb) : sbytes;
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{w0, w1}, __builtin_amdgcn_make_buffer_rsrc(a.nxt_qx, 0, qbytes, kRsrcWord3),
                                              qo, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b8((unsigned char)(ex + 127),
                                             __builtin_amdgcn_make_buffer_rsrc(a.nxt_sx, 0, sbytes, kRsrcWord3), so, 0, 0);
      }
    }
  };
  // prologue: the first kNStage - 1 ring steps in flight
  for (int p = 0; p < kNStage - 1; ++p) SVDQ_ISSUE(p)
  for (int ct = 0; ct < my_tiles; ++ct) {
    const TileMap tmc = map_tile((int)blockIdx.x + ct * grid, g.tiles_m, g.tiles_n, kGroupM);
    const int n0 = tmc.tn * kBN;
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int i = 0; i < kTM; ++i) acc[j][i] = f32x16{};
    for (int s4 = 0; s4 < g.nst; ++s4) SVDQ_STEP(false, s4 == g.nst - 1, true)
    for (int l = 0; l < nlr; ++l) SVDQ_STEP(true, l == nlr - 1, a.r32 > 0)
    // (every tile's last step runs its deferred MFMAs itself: saying so here
    // leaves the deferred operands dead over the epilogue)
    pending = false;

    const uint8_t* bslot = smem + ((gs - 1) & (kNStage - 1)) * kSlot + kScA + wn * kWN * 2;
    if constexpr (FUSE) {
      fused_tile(tmc.tm, tmc.tn, bslot, smem + ((gs - 1) & (kNStage - 1)) * kSlot);
    } else {
      // + bias (from the last low-rank slot), bf16. The accumulator lane holds
      // token m0 + 32 i + lr and channels 32 j + 8 q + 4 h + (0..3); swapping the
      // packed pairs (q = 1, h = 0) <-> (q = 0, h = 1) and (q = 3, h = 0) <->
      // (q = 2, h = 1) between the lane halves leaves lane h with channels
      // 32 j + 8 h + (0..7) and 32 j + 16 + 8 h + (0..7): two 16-byte stores,
      // 32 contiguous bytes of one row per lane pair.
      // Y rows of this tile as a buffer resource: stores past its end are dropped
      const int ynrec = min(g.M - tmc.tm * kBM, kBM) * g.ldy * 2;
      const __amdgpu_buffer_rsrc_t yrs =
          __builtin_amdgcn_make_buffer_rsrc(a.y + (size_t)tmc.tm * kBM * g.ldy, 0, ynrec, kRsrcWord3);
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
          // past M, and an 8-channel run past the layer's N is sent past the end
          const int col = n0 + 32 * bperm(wn * kTN + j) + 8 * h;
          const int off = ((wm * kWM + 32 * i + lr) * g.ldy + col) * 2;
          __builtin_amdgcn_raw_buffer_store_b128(u32x4{o[0], o[1], o[2], o[3]}, yrs, col < g.ldy ? off : ynrec, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b128(u32x4{o[4], o[5], o[6], o[7]}, yrs, col + 16 < g.ldy ? off + 32 : ynrec,
                                                 0, 0);
        }
      }
    }
    stores_due = kNStage - 1;
  }
  // the transfers issued past the end must land before the workgroup's LDS goes
  __builtin_amdgcn_s_waitcnt(0);
#undef SVDQ_STEP
#undef SVDQ_READ
#undef SVDQ_MFMA
#undef SVDQ_ISSUE
#undef SVDQ_READ
#undef SVDQ_MFMA
}

hipError_t prepare_gemm_mxfp4() {
  const hipError_t e = hipFuncSetAttribute((const void*)gemm_mxfp4_kernel<false>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void*)gemm_mxfp4_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)kLds);
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
  g.ldy = a.ldy;
  const int ntiles = g.tiles_m * g.tiles_n;
  // persistent grid: one workgroup per CU, a multiple of 8 so each stays on its XCD's tiles
  int grid = num_cus > 0 ? num_cus : 256;
  if (grid > ntiles) grid = ntiles;
  if (a.nxt_qx != nullptr)
    hipLaunchKernelGGL(gemm_mxfp4_kernel<true>, dim3(grid), dim3(64 * kNW), kLds, st, a, g, grid);
  else
    hipLaunchKernelGGL(gemm_mxfp4_kernel<false>, dim3(grid), dim3(64 * kNW), kLds, st, a, g, grid);
  return hipGetLastError();
}

}  // namespace svdq
