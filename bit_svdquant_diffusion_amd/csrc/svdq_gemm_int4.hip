// Kernel (2) of the forward for INT4 layers: Q4(X_hat) Q4(R)^T with per-group
// dequantization, plus the low-rank up-projection (X_hat L1) L2 and the bias,
// added before the single bf16 write of Y (aiflownews.com, "What SVDQuant
// actually does": the two-branch computation; "Nunchaku: the inference
// engine...": the branches share the output write).
//
// Integer part. The stored codes are 4-bit (one 1 KiB fragment per 32 rows
// and 64-channel group, lane 32h + r holding the 32 channels 32h + [0, 32)
// of row r). Every INT4 code lies in [-7, 7], and each of those integers is
// exact in FP6 E2M3, so before the GEMM a small kernel copies both operands'
// codes into the workspace as FP6 fields, and one group of a 32 x 32 block
// is one v_mfma_scale_f32_32x32x64_f8f6f4 on FP6 operands with unit E8M0
// scales: the products are small integers and the group sum P (|P| <= 49 *
// 64) comes out exactly, as an fp32 value.
//
// Dequantization. The per-output scale s_w[n] * s_x[m] of the group is an
// outer product, so it comes from the matrix unit as well: one two-block
// v_mfma_f32_32x32x1_2b_f32 gives it for two 32 x 32 blocks. That leaves one
// vector instruction per output and group, acc += P * s, in fp32.
//
// Data path and schedule follow the MXFP4 kernel: persistent workgroups (one
// per CU) walk 128 x 256 tiles; direct buffer loads into LDS of 16 bytes per
// lane (a lane's 24 FP6 bytes in two parts) fill a ring of LDS slots across
// tile boundaries; eight waves, 2 (M) x
// 4 (N), each own 64 x 64 (2 x 2 blocks of 32 x 32); one workgroup barrier
// per 128-channel stage (two groups). The low-rank branch is r32/32 more
// stages on v_mfma_f32_32x32x16_bf16 into the same accumulators.
//
// Work split. Whole rounds of tiles go one per workgroup. The tiles left
// after them (less than one round's worth) are cut into their K stages and dealt out
// as equal contiguous runs of (tile, stage) pairs, so every workgroup ends at
// the same time. Each XCD deals its own share of those tiles (the ones the
// tile map gives it) over its own workgroups, which keeps their operand
// panels in that XCD's L2. A run's part of a tile is a piece (a run that
// covers a whole tile just finishes it). Every piece writes its fp32 partial
// to its own workspace slot and then takes a ticket from the tile's counter;
// the piece that takes the last ticket adds all the tile's partials in piece
// (K) order, so the result does not depend on which piece came last, resets
// the counter and finishes the tile (low-rank product, bias, Y) with direct
// loads. No workgroup ever waits for another, so nothing assumes that the
// grid's workgroups run at the same time. Stage 1 clears the counters before
// every GEMM; the finishers leave them at zero as well.
#include "svdq_gemm_common.h"
#include "svdq_internal.h"
#include "svdq_layout.h"

#include <algorithm>

namespace svdq {

namespace {
constexpr int kBM = 128, kBN = 256, kWGM = 2, kWGN = 4, kNW = kWGM * kWGN;
constexpr int kWM = kBM / kWGM, kWN = kBN / kWGN, kTM = kWM / 32, kTN = kWN / 32;
constexpr int kMB = kBM / 32, kNBt = kBN / 32;     // 32-row blocks per tile: 4 (A), 8 (B)
constexpr int kGroupM = 8;
constexpr int kStores = 2 * kTN * kTM;             // 16-byte Y stores per wave per tile
// Transfers per stage, five per wave: op o = 5 w + k (k = 0..4).
// - 4-bit stage: ops 0..35 move the 36 FP6 fragment parts of 1 KiB (12 row
//   blocks x [group 0 heads, group 1 heads, both groups' tails]), op 36 the A
//   scales, ops 37 and 38 the two halves of the B scales, op 39 repeats op 38.
// - low-rank stage: ops 0..23 move the 24 bf16 fragments of Z and L2^T
//   (1 KiB each), the others copies of the bias transfer.
// Every wave thus issues the same count in every stage, so the ring waits
// have one form.
constexpr int kOps = 5;
constexpr int kParts4 = 3 * (kMB + kNBt);    // 4-bit fragment parts per stage
constexpr int kPartsLr = 2 * (kMB + kNBt);   // low-rank fragments per stage
// one ring slot: A codes (4 blocks x 3 KiB), B codes (8 x 3 KiB), A scales
// fp32 [2 groups][128], B scales fp32 [2 groups][256]; a low-rank stage puts
// its Z fragments at kCodeA and its L2^T fragments at kCodeB, 2 KiB per
// block, and the bias at kScA
constexpr int kCodeA = 0, kCodeB = kMB * 3 * 1024, kScA = kCodeB + kNBt * 3 * 1024;
constexpr int kScB = kScA + 2 * kBM * 4, kSlot = kScB + 2 * kBN * 4;
// ring slots: four, or three in the fused epilogue's launch, whose LDS also
// holds the cross-wave sum of the next layer's partial Z (the partials of all
// eight waves for one 32-token block and 32-rank block)
__host__ __device__ constexpr int ring_slots(bool fuse) { return fuse ? 3 : 4; }
constexpr size_t kZred = (size_t)kWGN * kWGM * 16 * 64 * 4;
constexpr size_t kLds = (size_t)ring_slots(false) * kSlot;
constexpr size_t kLdsFuse = (size_t)ring_slots(true) * kSlot + kZred;
static_assert(kLds <= 160 * 1024 - 256 && kLdsFuse <= 160 * 1024 - 256, "ring (and Z reduction) fit in LDS");
static_assert(kTM == 2 && kTN == 2, "schedule below assumes 2 x 2 blocks per wave");
static_assert(kNW * kOps == kParts4 + 4 && kPartsLr <= kParts4, "ops per stage partition");
static_assert(kParts4 == (kNW - 1) * kOps + 1, "the scale ops are ops 1..4 of the last wave");
static_assert(2 * kBM * 4 == 1024 && 2 * kBN * 4 == 2048 && kBN * 2 <= 1024,
              "one A and two B scale transfers of 64 lanes; the bias fits the A scale area");

// Ring barrier: wait until at most n of this wave's vector-memory operations
// are outstanding and its LDS reads have returned, then s_barrier (the same
// rule as the MXFP4 kernel: operations retire in issue order, so n = the
// number issued after the transfer being waited for).
#define SVDQ_VMCNT(n) (((n) & 15) | (((n) >> 4) << 14) | 0x0070)   /* expcnt 7, lgkmcnt 0 */
// `steady`: the step has two ring steps in flight after it and no stores
// counted, so n = C. Tested first, on its own flag: a test of n itself is
// folded by the compiler into the search through the cases, which every step
// would then walk.
template <int C>
__device__ __forceinline__ void ring_barrier(bool steady, int n) {
  __builtin_amdgcn_sched_barrier(0);
#define SVDQ_WAIT_CASE(k) \
  case k: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(k)); break;
  if (steady) {
    __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(C));
  } else switch (n < 24 ? n : 24) {   // a larger n waits for 24: longer than needed, never shorter
    SVDQ_WAIT_CASE(1) SVDQ_WAIT_CASE(2) SVDQ_WAIT_CASE(3) SVDQ_WAIT_CASE(4) SVDQ_WAIT_CASE(5) SVDQ_WAIT_CASE(6)
    SVDQ_WAIT_CASE(7) SVDQ_WAIT_CASE(8) SVDQ_WAIT_CASE(9) SVDQ_WAIT_CASE(10) SVDQ_WAIT_CASE(11) SVDQ_WAIT_CASE(12)
    SVDQ_WAIT_CASE(13) SVDQ_WAIT_CASE(14) SVDQ_WAIT_CASE(15) SVDQ_WAIT_CASE(16) SVDQ_WAIT_CASE(17)
    SVDQ_WAIT_CASE(18) SVDQ_WAIT_CASE(19) SVDQ_WAIT_CASE(20) SVDQ_WAIT_CASE(21) SVDQ_WAIT_CASE(22)
    SVDQ_WAIT_CASE(23) SVDQ_WAIT_CASE(24)
    default: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(0)); break;
  }
#undef SVDQ_WAIT_CASE
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ lds_void* lds_ptr(uint8_t* p) { return (lds_void*)p; }


struct Geo {
  int M, N, K, MB, NB, KS, nst, nstt, tiles_m, tiles_n, act_rows;   // N, K padded
  int r32;
  int ldy;   // Y's row stride and width (the layer's N)
  int tm_off, tn_off;   // group-sum hook: the window's first tile
  // whole tiles (indices below sk_base, a multiple of 8: rounds * grid),
  // then the sk_tiles tiles from index sk_base: tile index sk_base + 8 m + x
  // goes to XCD x, whose workgroups share its (tile, stage) pairs
  int rounds, sk_base, sk_tiles;
};
constexpr int kPartFloats = kBM * kBN;   // one fp32 partial tile
constexpr int kMinRun = 6;               // fewest stages per run of the split (when there are that many)
static_assert(kPartFloats * 4 == kSplitPartBytes, "workspace slot size");
static_assert(kSplitPieces == 2, "a run holds at most two pieces: its first and its last segment");
}  // namespace

// DEBUG_P: instead of dequantizing, write every group sum P (exact int32) of
// the outputs inside the window [m0, m0 + mc) x [n0, n0 + nc) to p, over the
// window's tiles only, with the same FP6 copies, transfers and MFMAs.
// FUSE: the tile's output is the next layer's input (GELU between them): see
// fused_tile below. Not combined with DEBUG_P.
template <bool DEBUG_P, bool FUSE>
__global__ __launch_bounds__(64 * kNW) void gemm_int4_kernel(GemmArgs a, Geo g, int grid) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWGN, wn = wave % kWGN;
  const int h = lane >> 5, lr = lane & 31;
  const int ntiles = g.tiles_m * g.tiles_n;
  const int wg = (int)blockIdx.x;
  const int nlr = g.nstt - g.nst;
  auto tile_of = [&](int t) -> TileMap {
    if (DEBUG_P) return TileMap{g.tm_off + t % g.tiles_m, g.tn_off + t / g.tiles_m};
    return map_tile(t, g.tiles_m, g.tiles_n, kGroupM);
  };
  // whole tiles wg + k * grid for k < ncl, then the run [u0, u1) of this
  // XCD's (tile m, stage) pairs, u = m nst + stage; a segment is one tile's
  // part of the run: stages [ka, kb)
  const int ncl = wg < g.sk_base ? (g.sk_base - 1 - wg) / grid + 1 : 0;
  const int xcd = wg & 7, kx = wg >> 3;   // XCD and index among its workgroups
  const int xtiles = DEBUG_P ? 0 : (g.sk_tiles > xcd ? (g.sk_tiles - xcd + 7) / 8 : 0);
  const long long xunits = (long long)xtiles * g.nst;
  // runs of this XCD: at most its workgroups, at least kMinRun stages each
  const int xruns = (int)min((long long)(grid >> 3), max(1LL, xunits / kMinRun));
  auto run_begin = [&](int k) -> long long { return (long long)k * xunits / xruns; };
  const long long u0 = (xtiles > 0 && kx < xruns) ? run_begin(kx) : 0;
  const long long u1 = (xtiles > 0 && kx < xruns) ? run_begin(kx + 1) : 0;
  // a segment: tile idx, its stages [ka, kb); whole (all K stages) or a
  // piece, m the tile's index among this XCD's split tiles
  struct Seg {
    int idx, ka, kb, m;
    bool whole;
  };
  auto seg_at = [&](int k, long long u) -> Seg {
    if (k < ncl) return Seg{wg + k * grid, 0, g.nst, -1, true};
    const int m = (int)(u / g.nst), ka = (int)(u - (long long)m * g.nst);
    const int kb = (int)min((long long)g.nst, ka + (u1 - u));
    return Seg{g.sk_base + 8 * m + xcd, ka, kb, m, ka == 0 && kb == g.nst};
  };
  // the run holding unit u of this XCD
  auto run_of = [&](long long u) -> int { return (int)min((long long)xruns - 1, ((u + 1) * xruns - 1) / xunits); };
  auto seg_len = [&](const Seg& sg) { return sg.kb - sg.ka + (sg.whole && !DEBUG_P ? nlr : 0); };
  int total = 0;   // ring steps of this workgroup
  {
    int k = 0;
    for (long long u = u0; k < ncl || u < u1; ++k) {
      const Seg sg = seg_at(k, u);
      total += seg_len(sg);
      if (k >= ncl) u += sg.kb - sg.ka;
    }
  }

  // issue side: next ring step to load (step is_s of segment is_k), and this
  // wave's per-tile transfer sources as byte offsets from uniform bases: op
  // 5 w + k from src[k] in a 4-bit stage (a fragment part, or for the last
  // wave's ops 1..4 its lane's scale entries) and from src[kOps + k] in a
  // low-rank stage; the bias from bsrc
  constexpr int NS = ring_slots(FUSE);
  const int nops = kOps;
  int is_k = 0, is_s = 0, is_ka = 0, is_nk = 0, is_len = 0;   // segment, step in it, its stages
  long long is_u = u0;
  uint32_t src[2 * kOps], bsrc = 0;
  const int per_l = a.r32 / 16;
  const uint32_t sstr_a = 2u * g.act_rows * 4, sstr_b = 2u * g.N * 4;   // scale bytes per stage
  // every source as a buffer resource over the whole operand: a transfer is
  // one buffer load into LDS with the lane's 32-bit offset and the stage as
  // a scalar offset (the API keeps the FP6 activation codes below 4 GiB)
  auto rsrc = [](const void* p, uint64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)(uint32_t)min(bytes, (uint64_t)0xFFFFFFFFu),
                                             0x00020000);
  };
  const __amdgpu_buffer_rsrc_t rqx = rsrc(a.qx6, (uint64_t)g.MB * g.KS * 1536);
  const __amdgpu_buffer_rsrc_t rqw = rsrc(a.qw6, (uint64_t)g.NB * g.KS * 1536);
  const __amdgpu_buffer_rsrc_t rz = rsrc(a.z, (uint64_t)g.MB * per_l * 1024);
  const __amdgpu_buffer_rsrc_t rl2 = rsrc(a.l2t, (uint64_t)g.NB * per_l * 1024);
  const __amdgpu_buffer_rsrc_t rsx = rsrc(a.sx, (uint64_t)g.KS * g.act_rows * 4);
  const __amdgpu_buffer_rsrc_t rsw = rsrc(a.sw, (uint64_t)g.KS * g.N * 4);
  const __amdgpu_buffer_rsrc_t rbias = rsrc(a.bias, (uint64_t)g.N * 2);
#define SVDQ_ISSUE(GS)                                                                              \
  {                                                                                                 \
    if (is_s == 0) {                                                                                \
      const Seg sg_ = seg_at(is_k, is_u);                                                           \
      is_ka = sg_.ka;                                                                               \
      is_nk = sg_.kb - sg_.ka;                                                                      \
      is_len = seg_len(sg_);                                                                        \
      const TileMap tmi = tile_of(sg_.idx);                                                         \
      const int mb0 = tmi.tm * kMB, nb0 = tmi.tn * kNBt;                                            \
      _Pragma("unroll") for (int k = 0; k < kOps; ++k) {                                            \
        const int o = kOps * wave + k;                                                              \
        if (o < kParts4) {                                                                          \
          /* part o % 3 of row block o / 3 (A), or of (o - 12) / 3 (B) */                          \
          const bool isA = o < 3 * kMB;                                                             \
          const int q = isA ? o : o - 3 * kMB;                                                      \
          const uint32_t b = (uint32_t)min((isA ? mb0 : nb0) + q / 3, (isA ? g.MB : g.NB) - 1);     \
          src[k] = (b * (uint32_t)g.nst * 3 + q % 3) * 1024 + lane * 16;                            \
        } else {                                                                                    \
          /* scales: entry e = 4 lane (+ 256 for the second B half) of [2 groups][T] */            \
          const int sop = min(o - kParts4, 2);                                                      \
          const bool isA = sop == 0;                                                                \
          const int T = isA ? kBM : kBN;                                                            \
          const int e = (sop == 2 ? 256 : 0) + 4 * lane;                                            \
          const int gg = e >= T ? 1 : 0, idx = e - gg * T;                                          \
          const int lim = isA ? g.act_rows : g.N;                                                   \
          const int row = min((isA ? mb0 : nb0) * 32 + idx, lim - 4);                               \
          src[k] = (uint32_t)(gg * lim + row) * 4;                                                  \
        }                                                                                           \
        if (o < kPartsLr) {                                                                         \
          /* 16-column step o % 2 of row block o / 2 (Z), or of (o - 8) / 2 (L2^T) */              \
          const bool isA = o < 2 * kMB;                                                             \
          const int q = isA ? o : o - 2 * kMB;                                                      \
          const uint32_t b = (uint32_t)min((isA ? mb0 : nb0) + (q >> 1), (isA ? g.MB : g.NB) - 1);  \
          src[kOps + k] = (b * per_l + (q & 1)) * 1024 + lane * 16;                                 \
        }                                                                                           \
      }                                                                                             \
      bsrc = (uint32_t)min(nb0 * 32 + 8 * lane, g.N - 8) * 2;                                       \
    }                                                                                               \
    uint8_t* slot_w = smem + ((GS) % NS) * kSlot;                                                   \
    const bool lrs = is_s >= is_nk;                                                                 \
    const int sl = lrs ? is_s - is_nk : is_ka + is_s;                                               \
    if (lrs) {                                                                                      \
      if (a.r32 > 0 && wave * kOps < kPartsLr) {                                                    \
        /* Z / L2^T fragments below op 24, copies of the bias from there */                        \
        _Pragma("unroll") for (int k = 0; k < kOps; ++k) {                                          \
          const int o = kOps * wave + k;                                                            \
          if (o < kPartsLr) {                                                                       \
            const bool isA = o < 2 * kMB;                                                           \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(isA ? rz : rl2,                                \
                                                     lds_ptr(slot_w + (isA ? kCodeA + o * 1024 : kCodeB + (o - 2 * kMB) * 1024)), \
                                                     16, src[kOps + k], sl * 2048, 0, 0);           \
          } else if (lane < 32) {                                                                   \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rbias, lds_ptr(slot_w + kScA), 16, bsrc, 0, 0, 0); \
          }                                                                                         \
        }                                                                                           \
      } else {                                                                                      \
        _Pragma("unroll") for (int k = 0; k < kOps; ++k) if (lane < 32)                             \
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rbias, lds_ptr(slot_w + kScA), 16, bsrc, 0, 0, 0); \
      }                                                                                             \
    } else if (wave < kNW - 1) {                                                                    \
      /* five fragment parts; part o lands at o KiB (the B area follows the A area) */             \
      _Pragma("unroll") for (int k = 0; k < kOps; ++k) {                                            \
        const int o = kOps * wave + k;                                                              \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(o < 3 * kMB ? rqx : rqw, lds_ptr(slot_w + kCodeA + o * 1024), 16, \
                                                 src[k], sl * 3072, 0, 0);                          \
      }                                                                                             \
    } else {                                                                                        \
      /* the last fragment part, the A scales, both B scale halves, the second again */            \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rqw, lds_ptr(slot_w + kCodeA + (kParts4 - 1) * 1024), 16, src[0], \
                                               sl * 3072, 0, 0);                                    \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsx, lds_ptr(slot_w + kScA), 16, src[1], sl * sstr_a, 0, 0); \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, lds_ptr(slot_w + kScB), 16, src[2], sl * sstr_b, 0, 0); \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, lds_ptr(slot_w + kScB + 1024), 16, src[3], sl * sstr_b, 0, 0); \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, lds_ptr(slot_w + kScB + 1024), 16, src[4], sl * sstr_b, 0, 0); \
    }                                                                                               \
    if (++is_s == is_len) {                                                                         \
      is_s = 0;                                                                                     \
      if (is_k >= ncl) is_u += is_nk;                                                               \
      ++is_k;                                                                                       \
    }                                                                                               \
  }

  f32x16 acc[kTN][kTM];

  // The two groups of a stage are eight units u = (group u / 4, block
  // j = (u / 2) % 2, i = u % 2). A unit is one block-scaled MFMA on the FP6
  // codes with unit E8M0 scales, which gives the group's P exactly in fp32
  // (integer products, |P| <= 49 * 64), every other unit one fp32 MFMA for
  // the scale outer product of two blocks, and the dequant acc += P s of
  // its 16 outputs per lane (or, DEBUG_P, the group-sum writes). Units are
  // software-pipelined within the wave: the MFMAs of unit u + 1 are issued
  // before the vector work of unit u.
  // ring step being computed; ring steps still to absorb the last epilogue's
  // stores, and how many stores that epilogue issued (the same in every wave)
  int gs = 0, stores_due = 0;
  const int nstores = FUSE ? kTM * (2 + (a.nxt_r32 > 0 ? a.nxt_r32 / 32 : 0)) : kStores;
  i32x8 xo[2][kTM], wo[2][kTN];   // FP6 operands: six dwords of 32 fields, two unused
  float sxv[2][kTM], swv[2][kTN];
  f32x16 pf[2];
  f32x16 sc[2][2];   // [block pair (u / 2) % 2][i]
  auto mfma_unit = [&](int u) {
    const int gg = u >> 2, j = (u >> 1) & 1, i = u & 1;
    pf[u & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wo[gg][j], xo[gg][i], f32x16{}, 2, 2, 0, 127, 0, 127);
    if (!DEBUG_P && i == 0) {
      // scales of blocks (j, 0) and (j, 1) in one two-block outer product:
      // block b = lane / 32 takes the 32 channel scales of block row j and
      // the 32 token scales of block column i = b; output block b in
      // registers 16 b .. 16 b + 15, each in the 32 x 32 accumulator layout
      const f32x32 r = __builtin_amdgcn_mfma_f32_32x32x1f32(swv[gg][j], h ? sxv[gg][1] : sxv[gg][0], f32x32{}, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sc[(u >> 1) & 1][0][e] = r[e];
        sc[(u >> 1) & 1][1][e] = r[16 + e];
      }
    }
  };
  auto valu_unit = [&](int u, int st, int m0t, int n0t) {
    const int gg = u >> 2, j = (u >> 1) & 1, i = u & 1;
    const f32x16& p = pf[u & 1];
    if constexpr (DEBUG_P) {
      const int tok = m0t + wm * kWM + 32 * i + lr;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int ch = n0t + wn * kWN + 32 * j + 8 * (e >> 2) + 4 * h + (e & 3);
        if (tok >= a.m0 && tok < a.m0 + a.mc && ch >= a.n0 && ch < a.n0 + a.nc)
          if (2 * st + gg < a.ldk / 64)   // the layer's groups (not the padding)
            a.p[((size_t)(tok - a.m0) * a.nc + (ch - a.n0)) * (a.ldk / 64) + 2 * st + gg] = (int)p[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][i][e] = __builtin_fmaf(p[e], sc[(u >> 1) & 1][i][e], acc[j][i][e]);
    }
  };
  // One stage: the FP6 operands and scales of both groups are read from LDS
  // up front (a lane's 24 bytes: its 16-byte head and its 8-byte tail);
  // then eight pipeline steps, each its own scheduling region: the MFMAs of
  // unit u + 1 spread over the 16 vector instructions of unit u.
  auto stage_compute = [&](const uint8_t* slot, int st, int m0t, int n0t) {
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
#pragma unroll
      for (int t = 0; t < kTM; ++t) {
        const int ba = wm * kTM + t;
        const i32x4 hd = *reinterpret_cast<const i32x4*>(slot + kCodeA + (ba * 3 + gg) * 1024 + lane * 16);
        const u32x2 tl = *reinterpret_cast<const u32x2*>(slot + kCodeA + (ba * 3 + 2) * 1024 + gg * 512 + lane * 8);
        xo[gg][t] = i32x8{hd[0], hd[1], hd[2], hd[3], (int)tl[0], (int)tl[1], 0, 0};
        sxv[gg][t] = *reinterpret_cast<const float*>(slot + kScA + gg * (kBM * 4) + (wm * kWM + 32 * t + lr) * 4);
      }
#pragma unroll
      for (int t = 0; t < kTN; ++t) {
        const int bb = wn * kTN + t;
        const i32x4 hd = *reinterpret_cast<const i32x4*>(slot + kCodeB + (bb * 3 + gg) * 1024 + lane * 16);
        const u32x2 tl = *reinterpret_cast<const u32x2*>(slot + kCodeB + (bb * 3 + 2) * 1024 + gg * 512 + lane * 8);
        wo[gg][t] = i32x8{hd[0], hd[1], hd[2], hd[3], (int)tl[0], (int)tl[1], 0, 0};
        swv[gg][t] = *reinterpret_cast<const float*>(slot + kScB + gg * (kBN * 4) + (wn * kWN + 32 * t + lr) * 4);
      }
    }
    mfma_unit(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u + 1 < 8) mfma_unit(u + 1);
      valu_unit(u, st, m0t, n0t);
      if (u + 1 < 8) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // acc + bias, bf16 write of the wave's 64 x 64 (the MXFP4 kernel's
  // epilogue). Lane h of the accumulator holds channels 32 j + 8 q + 4 h +
  // (0..3) of token m0 + 32 i + lr; after swapping the packed pairs (q = 1,
  // h = 0) <-> (q = 0, h = 1) and (q = 3, h = 0) <-> (q = 2, h = 1), each
  // lane stores two 16-byte runs of one row.
  auto store_tile = [&](int m0t, int n0, const float (&bv)[kTN][16]) {
    const int ynrec = min(g.M - m0t, kBM) * g.ldy * 2;
    const __amdgpu_buffer_rsrc_t yrs =
        __builtin_amdgcn_make_buffer_rsrc(a.y + (size_t)m0t * g.ldy, 0, ynrec, 0x00020000);
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        uint32_t o[8];
#pragma unroll
        for (int p = 0; p < 8; ++p)
          o[p] = cvt_bf16x2(acc[j][i][2 * p] + bv[j][2 * p], acc[j][i][2 * p + 1] + bv[j][2 * p + 1]);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            const auto r = __builtin_amdgcn_permlane32_swap(o[4 * p + w], o[4 * p + 2 + w], false, false);
            o[4 * p + w] = r[0];
            o[4 * p + 2 + w] = r[1];
          }
        }
        // always issued (the ring waits count them); the resource drops rows
        // past M, and an 8-channel run past the layer's N is sent past the end
        const int col = n0 + 32 * j + 8 * h;
        const int off = ((wm * kWM + 32 * i + lr) * g.ldy + col) * 2;
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{o[0], o[1], o[2], o[3]}, yrs, col < g.ldy ? off : ynrec, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{o[4], o[5], o[6], o[7]}, yrs, col + 16 < g.ldy ? off + 32 : ynrec,
                                               0, 0);
      }
    }
  };
  // FUSE: instead of Y, this wave's 64 x 64 of GELU(bf16(acc + bias)) (a bf16
  // value, as a separate GELU over bf16 Y would give) becomes the next
  // layer's input, smoothed by its mu: first the partial X_hat L1 over the
  // tile's 256 channels on bf16 MFMAs (each wave its 64 channels; the four
  // wave columns' partials added in column order through LDS by all eight
  // waves, one 16-byte store per lane), then one 64-channel group per token
  // quantized by the stage-1 quantizer, codes in the stage-1 fragment order
  // (lane h keeps block j = h: the two lanes of a token trade the other
  // block's 4-channel runs) and scales. Every store is issued by every wave
  // (lanes past M or not holding a scale aim past the end of their buffer),
  // kTM * (2 + r32 / 32) of them, which the next ring waits count.
  auto fused_tile = [&](int m0t, int n0, int tn) {
    const int grp = n0 / 64, nr = a.nxt_r32;
    // acc (+ bias, added by the caller) -> the next layer's smoothed input, in place
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 m4 = *reinterpret_cast<const f32x4*>(a.nxt_mu + n0 + 32 * j + 8 * q + 4 * h);
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const uint32_t yb = cvt_bf16x2(acc[j][i][4 * q + e], acc[j][i][4 * q + e + 1]);   // Y as bf16
            const uint32_t gb = cvt_bf16x2(gelu_f32(bf16lo(yb)), gelu_f32(bf16hi(yb)));
            acc[j][i][4 * q + e] = bf16lo(gb) * m4[e];
            acc[j][i][4 * q + e + 1] = bf16hi(gb) * m4[e + 1];
          }
      }
    if (nr > 0) {
      // zred [wave column][wave row][16][64]: one 32-token block's partials
      float* zred = reinterpret_cast<float*>(smem + (size_t)NS * kSlot);
      const uint32_t zbytes = (uint32_t)((size_t)g.tiles_n * g.M * nr * 4);
      const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(a.nxt_zpart, 0, zbytes, 0x00020000);
      // the reduction's share of thread tid: wave row zr, token ztk of the
      // block, ranks zc .. zc + 3; in the 32 x 32 accumulator layout that is
      // register 4 (ztk / 8) + ztk % 4 of lanes zc + 32 ((ztk / 4) % 2) + (0..3)
      const int zr = tid >> 8, ztk = (tid >> 3) & 31, zc = 4 * (tid & 7);
      const int zoff = ((zr * 16 + 4 * (ztk / 8) + ztk % 4) * 64) + zc + 32 * ((ztk / 4) % 2);
      for (int rb = 0; rb < nr / 32; ++rb) {
        // B: L1 rows of channels n0 + 32 j + 16 m + 8 u + 4 h + (0..3) for
        // rank 32 rb + lr, gathered from the stage-1 layout (8 bytes per 4 channels)
        u32x4 bw[kTN][2];
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            u32x2 bl[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int k = n0 + 32 * j + 16 * m + 8 * u + 4 * h, col = 32 * rb + lr;
              const size_t li = (((((size_t)(k / 256) * 4 + (k % 256) / 64) * (nr / 16) + col / 16) * 2 + (k % 16) / 8) * 64 +
                                 16 * ((k % 64) / 16) + col % 16) * 8 + k % 8;
              bl[u] = *reinterpret_cast<const u32x2*>(a.nxt_l1s + li);
            }
            bw[j][m] = u32x4{bl[0][0], bl[0][1], bl[1][0], bl[1][1]};
          }
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
          // A: the token's channels 32 j + 16 m + 4 h + (0..3, 8..11), that
          // is acc[j][i][8 m .. 8 m + 7], as bf16
          f32x16 zacc = f32x16{};
#pragma unroll
          for (int j = 0; j < kTN; ++j)
#pragma unroll
            for (int m = 0; m < 2; ++m) {
              const f32x16& v = acc[j][i];
              const u32x4 av = u32x4{cvt_bf16x2(v[8 * m + 0], v[8 * m + 1]), cvt_bf16x2(v[8 * m + 2], v[8 * m + 3]),
                                     cvt_bf16x2(v[8 * m + 4], v[8 * m + 5]), cvt_bf16x2(v[8 * m + 6], v[8 * m + 7])};
              zacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                             __builtin_bit_cast(bf16x8, bw[j][m]), zacc, 0, 0, 0);
            }
          if (rb + i > 0) __syncthreads();   // the last block's reads are done
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
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, zs), zrs, zo, 0, 0);
        }
      }
    }
    const uint32_t qbytes = (uint32_t)((size_t)(g.MB * 32) * (g.N / 2));
    const uint32_t sbytes = (uint32_t)((size_t)(g.N / 64) * g.act_rows * 4);
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(a.nxt_qx, 0, qbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(a.nxt_sx, 0, sbytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int t = m0t + wm * kWM + 32 * i + lr;   // the lane's token
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(acc[j][i][e]));
      amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));   // the token's other 32 channels
      const float sc = amax / 7.0f;
      uint32_t c[kTN][2];
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = acc[j][i][e];
        int4_codes16(v, sc, c[j][0], c[j][1]);
      }
      const uint32_t o0 = __shfl_xor(h ? c[0][0] : c[1][0], 32), o1 = __shfl_xor(h ? c[0][1] : c[1][1], 32);
      const uint32_t m0 = h ? c[1][0] : c[0][0], m1 = h ? c[1][1] : c[0][1];
      // runs of channels 8k .. 8k + 3 are lane 0's, 8k + 4 .. 8k + 7 lane 1's
      const uint32_t ev0 = h ? o0 : m0, od0 = h ? m0 : o0, ev1 = h ? o1 : m1, od1 = h ? m1 : o1;
      const u32x4 out = u32x4{(ev0 & 0xFFFFu) | (od0 << 16), (ev0 >> 16) | (od0 & 0xFFFF0000u),
                              (ev1 & 0xFFFFu) | (od1 << 16), (ev1 >> 16) | (od1 & 0xFFFF0000u)};
      // rows past M stay unwritten, as stage 1 leaves them
      const bool live = t < g.M;
      const uint32_t qo = live ? (uint32_t)((((size_t)(t / 32) * (g.N / 64) + grp) * 64 + 32 * h + t % 32) * 16) : qbytes;
      const uint32_t so = live && h == 0 ? (uint32_t)(((size_t)grp * g.act_rows + t) * 4) : sbytes;
      __builtin_amdgcn_raw_buffer_store_b128(out, qrs, qo, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), srs, so, 0, 0);
    }
  };
  __shared__ int ticket_last;   // the workgroup took a tile's last ticket

  // prologue: the first NS - 1 ring steps in flight
  for (int p = 0; p < NS - 1 && p < total; ++p) SVDQ_ISSUE(p)
  // this lane's 16 float4 of a partial tile in a workspace slot
  auto part_at = [&](int slot_wg, int f) -> float* {
    return a.part + (size_t)slot_wg * kPartFloats + ((size_t)(wave * 16 + f) * 64 + lane) * 4;
  };
  int ck = 0;
  for (long long cu = u0; ck < ncl || cu < u1; ++ck) {
    const Seg sg = seg_at(ck, cu);
    if (ck >= ncl) cu += sg.kb - sg.ka;
    const TileMap tmc = tile_of(sg.idx);
    const int m0t = tmc.tm * kBM, n0t = tmc.tn * kBN;
    const int n0 = n0t + wn * kWN;
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int i = 0; i < kTM; ++i) acc[j][i] = f32x16{};
    for (int st = sg.ka; st < sg.kb; ++st) {
      ring_barrier<kOps * (NS - 2)>(!DEBUG_P && stores_due == 0 && total - 1 - gs >= NS - 2,
                                    DEBUG_P ? 0 : nops * min(NS - 2, total - 1 - gs) + (stores_due > 0 ? nstores : 0));
      if (stores_due > 0) --stores_due;
      if (gs + NS - 1 < total) SVDQ_ISSUE(gs + NS - 1)
      stage_compute(smem + (gs % NS) * kSlot, st, m0t, n0t);
      ++gs;
    }
    if constexpr (DEBUG_P) continue;
    if (!FUSE && !sg.whole) {   // (FUSE launches take whole tiles only)
      // a piece: publish the partial in this run's slot for it (its first
      // segment, else its last), then take the tile's ticket
      const int myslot = kSplitPieces * wg + (ck == ncl ? 0 : 1);
#pragma unroll
      for (int f = 0; f < 16; ++f) {
        const f32x16& v = acc[f >> 3][(f >> 2) & 1];
        *reinterpret_cast<f32x4*>(part_at(myslot, f)) = f32x4{v[4 * (f & 3)], v[4 * (f & 3) + 1], v[4 * (f & 3) + 2], v[4 * (f & 3) + 3]};
      }
      __builtin_amdgcn_s_waitcnt(0);   // every wave's stores (and transfers) have landed ...
      __syncthreads();                  // ... before one release covers them all
      const int k0 = run_of((long long)sg.m * g.nst), k1 = run_of((long long)(sg.m + 1) * g.nst - 1);
      uint32_t* ctr = a.flags + (sg.idx - g.sk_base);
      if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const uint32_t t = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = t + 1 == (uint32_t)(k1 - k0 + 1);
        if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ticket_last = last ? 1 : 0;
      }
      __syncthreads();
      if (!ticket_last) continue;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      // the last piece: the tile's partials in piece order. A run's piece is
      // its first segment when the run starts inside this tile (or at its
      // first stage), else its last segment.
      for (int k = k0; k <= k1; ++k) {
        const int slot = kSplitPieces * (xcd + 8 * k) + (run_begin(k) >= (long long)sg.m * g.nst ? 0 : 1);
#pragma unroll
        for (int f = 0; f < 16; ++f) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(part_at(slot, f));
          f32x16& d = acc[f >> 3][(f >> 2) & 1];
#pragma unroll
          for (int e = 0; e < 4; ++e) d[4 * (f & 3) + e] = k == k0 ? v[e] : d[4 * (f & 3) + e] + v[e];
        }
      }
      // + (X_hat L1) L2 from fragments loaded straight from memory, in the
      // ring's order of 16-column steps, then the bias
      const int per_l = g.r32 / 16;
      for (int c = 0; c < per_l; ++c) {
        i32x4 fa[kTM], fb[kTN];
#pragma unroll
        for (int t = 0; t < kTM; ++t) {
          const int b = min(tmc.tm * kMB + wm * kTM + t, g.MB - 1);
          fa[t] = *reinterpret_cast<const i32x4*>(a.z + ((size_t)(b * per_l + c) * 64 + lane) * 8);
        }
#pragma unroll
        for (int t = 0; t < kTN; ++t) {
          const int b = min(tmc.tn * kNBt + wn * kTN + t, g.NB - 1);
          fb[t] = *reinterpret_cast<const i32x4*>(a.l2t + ((size_t)(b * per_l + c) * 64 + lane) * 8);
        }
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
          for (int i = 0; i < kTM; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fb[j]),
                                                                __builtin_bit_cast(bf16x8, fa[i]), acc[j][i], 0, 0, 0);
      }
      float bv[kTN][16];
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = min(n0 + 32 * j + 8 * q + 4 * h, g.N - 4);
          const u32x2 bw = *reinterpret_cast<const u32x2*>(a.bias + ch);
          bv[j][4 * q + 0] = bf16lo(bw.x);
          bv[j][4 * q + 1] = bf16hi(bw.x);
          bv[j][4 * q + 2] = bf16lo(bw.y);
          bv[j][4 * q + 3] = bf16hi(bw.y);
        }
      __builtin_amdgcn_s_waitcnt(0);   // no transfer is in flight: the next ring waits stay exact
      store_tile(m0t, n0, bv);
      stores_due = NS - 1;
      continue;
    }
    for (int l = 0; l < nlr; ++l) {
      ring_barrier<kOps * (NS - 2)>(stores_due == 0 && total - 1 - gs >= NS - 2,
                                    nops * min(NS - 2, total - 1 - gs) + (stores_due > 0 ? nstores : 0));
      if (stores_due > 0) --stores_due;
      const bool more = gs + NS - 1 < total;
      if (more && wave < 4) SVDQ_ISSUE(gs + NS - 1)
      const uint8_t* slot = smem + (gs % NS) * kSlot;
      if (a.r32 > 0) {
#pragma unroll
        for (int step = 0; step < 2; ++step) {
          i32x4 fa[kTM], fb[kTN];
#pragma unroll
          for (int t = 0; t < kTM; ++t)
            fa[t] = *reinterpret_cast<const i32x4*>(slot + kCodeA + ((wm * kTM + t) * 2 + step) * 1024 + lane * 16);
#pragma unroll
          for (int t = 0; t < kTN; ++t)
            fb[t] = *reinterpret_cast<const i32x4*>(slot + kCodeB + ((wn * kTN + t) * 2 + step) * 1024 + lane * 16);
#pragma unroll
          for (int j = 0; j < kTN; ++j)
#pragma unroll
            for (int i = 0; i < kTM; ++i)
              acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fb[j]),
                                                                  __builtin_bit_cast(bf16x8, fa[i]), acc[j][i], 0, 0, 0);
        }
      }
      if (more && wave >= 4) SVDQ_ISSUE(gs + NS - 1)
      ++gs;
    }

    // + bias (from the last low-rank slot), bf16 write
    const uint8_t* bslot = smem + ((gs - 1) % NS) * kSlot + kScA + wn * kWN * 2;
    float bv[kTN][16];
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 bw = *reinterpret_cast<const u32x2*>(bslot + (32 * j + 8 * q + 4 * h) * 2);
        bv[j][4 * q + 0] = bf16lo(bw.x);
        bv[j][4 * q + 1] = bf16hi(bw.x);
        bv[j][4 * q + 2] = bf16lo(bw.y);
        bv[j][4 * q + 3] = bf16hi(bw.y);
      }
    if constexpr (FUSE) {
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[j][i][e] += bv[j][e];
      fused_tile(m0t, n0, tmc.tn);
    } else {
      store_tile(m0t, n0, bv);
    }
    stores_due = NS - 1;
  }
#undef SVDQ_ISSUE
}

// The tiled GEMM's FP6 copy of 4-bit codes. Nibble fragment (row block b,
// group f): 1 KiB, lane l's 16 bytes holding channels 32 h + [0, 32) with the
// even channel in the low nibble. Its FP6 form is lane l's 24 bytes of 32
// E2M3 fields (field i at bit 6 i: channel 32 h + i), the first 16 bytes in
// part f % 2 and the last 8 in part 2 at (f % 2) 512 + 8 l, of the 3 KiB of
// (b, stage f / 2). The codes, sign-extended and converted to fp32 (exact
// small integers), go through v_cvt_scalef32_2xpk16_fp6_f32 with scale 1,
// which is exact for them (every integer in [-7, 7] is an E2M3 value) and
// puts element i of its first operand in field 2 i and of its second in
// field 2 i + 1: the even and the odd channels. One thread per lane and
// fragment: workgroup (x, y) takes row block x (X's row blocks first, then
// W's) and its groups 4 y .. 4 y + 3, a wave per group.
__global__ __launch_bounds__(256) void expand_fp6_kernel(const uint8_t* __restrict__ qx, uint8_t* __restrict__ x6,
                                                         int mbx, const uint8_t* __restrict__ qw,
                                                         uint8_t* __restrict__ w6, int KS) {
  const int lane = threadIdx.x & 63;
  const bool isx = (int)blockIdx.x < mbx;
  const size_t b = isx ? blockIdx.x : blockIdx.x - mbx;
  const int f = 4 * blockIdx.y + (threadIdx.x >> 6);
  const u32x4 in = *reinterpret_cast<const u32x4*>((isx ? qx : qw) + ((b * KS + f) * 64 + lane) * 16);
  f32x16 ev, od;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    ev[j] = (float)(int)__builtin_amdgcn_sbfe((int)in[j >> 2], 8 * (j & 3), 4);
    od[j] = (float)(int)__builtin_amdgcn_sbfe((int)in[j >> 2], 8 * (j & 3) + 4, 4);
  }
  const auto w = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 1.0f);
  uint8_t* dst = (isx ? x6 : w6) + (b * (KS / 2) + (f >> 1)) * 3072;
  *reinterpret_cast<u32x4*>(dst + (f & 1) * 1024 + lane * 16) = u32x4{w[0], w[1], w[2], w[3]};
  *reinterpret_cast<u32x2*>(dst + 2048 + (f & 1) * 512 + lane * 8) = u32x2{w[4], w[5]};
}

hipError_t prepare_gemm_int4() {
  hipError_t e = hipFuncSetAttribute((const void*)gemm_int4_kernel<false, false>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)gemm_int4_kernel<false, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)kLdsFuse);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void*)gemm_int4_kernel<true, false>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
}

hipError_t launch_gemm_int4(const GemmArgs& a, int num_cus, hipStream_t st) {
  Geo g;
  g.M = a.M;
  g.N = a.N;
  g.K = a.K;
  g.MB = (a.M + 31) / 32;
  g.NB = a.N / 32;
  g.KS = a.K / 64;
  g.nst = a.K / 128;
  g.act_rows = (a.M + 15) / 16 * 16;
  g.r32 = a.r32;
  g.ldy = a.ldy;
  g.tm_off = g.tn_off = 0;
  int grid = num_cus > 0 ? num_cus : 256;
  // the FP6 copies of both operands' codes, then the GEMM on them
  if (a.qx6 == nullptr || a.qw6 == nullptr) return hipErrorInvalidValue;
  hipLaunchKernelGGL(expand_fp6_kernel, dim3(g.MB + g.NB, g.KS / 4), dim3(256), 0, st, a.qx, a.qx6, g.MB, a.qw,
                     a.qw6, g.KS);
  if (a.p) {
    // group-sum hook: only the tiles that hold the window, no low-rank stages
    g.nstt = g.nst;
    g.tm_off = a.m0 / kBM;
    g.tn_off = a.n0 / kBN;
    g.tiles_m = (a.m0 + a.mc + kBM - 1) / kBM - g.tm_off;
    g.tiles_n = (a.n0 + a.nc + kBN - 1) / kBN - g.tn_off;
    const int ntiles = g.tiles_m * g.tiles_n;
    if (grid > ntiles) grid = ntiles;
    g.rounds = 0;
    g.sk_base = ntiles;   // whole tiles only
    g.sk_tiles = 0;
    hipLaunchKernelGGL((gemm_int4_kernel<true, false>), dim3(grid), dim3(64 * kNW), kLds, st, a, g, grid);
    return hipGetLastError();
  }
  const int nlr = a.r32 > 0 ? a.r32 / 32 : 1;   // at least one: the bias rides in a low-rank stage
  g.nstt = g.nst + nlr;
  g.tiles_m = (a.M + kBM - 1) / kBM;
  g.tiles_n = (a.N + kBN - 1) / kBN;
  const int ntiles = g.tiles_m * g.tiles_n;
  if (grid > kSplitSlots) grid = kSplitSlots;
  if (grid >= 8) {
    grid &= ~7;   // every XCD holds the same number of workgroups
    // every whole round; the remainder is split. (Splitting the last whole
    // round as well measured no faster and read more: runs that start
    // mid-tile fall out of K step with their XCD's other workgroups.)
    g.rounds = ntiles / grid;
    g.sk_base = g.rounds * grid;
    g.sk_tiles = ntiles - g.sk_base;
  } else {
    g.rounds = (ntiles + grid - 1) / grid;
    g.sk_base = ntiles;   // whole tiles only
    g.sk_tiles = 0;
  }
  if (a.nxt_qx != nullptr) {
    // whole tiles only: the epilogue's registers on top of the split's
    // finisher would spill in the main loop
    if (grid > ntiles) grid = ntiles;
    g.rounds = (ntiles + grid - 1) / grid;
    g.sk_base = ntiles;
    g.sk_tiles = 0;
    hipLaunchKernelGGL((gemm_int4_kernel<false, true>), dim3(grid), dim3(64 * kNW), kLdsFuse, st, a, g, grid);
  } else
    hipLaunchKernelGGL((gemm_int4_kernel<false, false>), dim3(grid), dim3(64 * kNW), kLds, st, a, g, grid);
  return hipGetLastError();
}

// Z = bf16 of the tile partials [tiles_n][M][r32] added in tile order, in
// the stage-1 fragment order; the next layer's split counters cleared
__global__ void fused_zsum_kernel(const float* __restrict__ zpart, int tiles_n, int M, int r32,
                                  uint16_t* __restrict__ z, uint32_t* __restrict__ flags, int nflags) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < nflags) flags[idx] = 0u;
  if (idx >= M * r32) return;
  const int t = idx / r32, col = idx - t * r32;
  float s = zpart[idx];
  for (int c = 1; c < tiles_n; ++c) s += zpart[(size_t)c * M * r32 + idx];
  z[(((size_t)(t / 32) * (r32 / 16) + col / 16) * 64 + 32 * ((col % 16) / 8) + t % 32) * 8 + col % 8] = (uint16_t)f2bf(s);
}

hipError_t launch_fused_zsum(const float* zpart, int tiles_n, int M, int r32, uint16_t* z, uint32_t* flags,
                             int nflags, hipStream_t st) {
  const int n = std::max(M * r32, nflags);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fused_zsum_kernel, dim3((n + 255) / 256), dim3(256), 0, st, zpart, tiles_n, M, r32, z, flags,
                     nflags);
  return hipGetLastError();
}

__global__ void gelu_bf16_kernel(uint16_t* __restrict__ y, size_t n8) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  u32x4 v = reinterpret_cast<u32x4*>(y)[i];
#pragma unroll
  for (int d = 0; d < 4; ++d) v[d] = cvt_bf16x2(gelu_f32(bf16lo(v[d])), gelu_f32(bf16hi(v[d])));
  reinterpret_cast<u32x4*>(y)[i] = v;
}

hipError_t launch_gelu_bf16(uint16_t* y, size_t n, hipStream_t st) {
  const size_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  hipLaunchKernelGGL(gelu_bf16_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, y, n8);
  return hipGetLastError();
}

}  // namespace svdq
