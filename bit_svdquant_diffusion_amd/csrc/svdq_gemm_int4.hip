// Kernel (2) of the forward for INT4 layers: Q4(X_hat) Q4(R)^T with per-group
// dequantization, plus the low-rank up-projection (X_hat L1) L2 and the bias,
// added before the single bf16 write of Y (aiflownews.com, "What SVDQuant
// actually does": the two-branch computation; "Nunchaku: the inference
// engine...": the branches share the output write).
//
// Integer part. Codes are stored in the same fragment order as the MXFP4
// path: one 1 KiB block per 32 rows and 64-channel group, lane 32h + r holding
// the 32 channels 32h + [0, 32) of row r. Widened in registers to int8 as
// 16*q ((w << 4) & 0xF0F0F0F0 for the even channels, w & 0xF0F0F0F0 for the
// odd ones), one group of a 32 x 32 block is two v_mfma_i32_32x32x32_i8 (even
// channels, then odd channels into the same accumulator), giving 256 * P
// exactly in int32.
//
// Dequantization. The per-output scale s_w[n] * s_x[m] / 256 of the group is
// an outer product, so it comes from the matrix unit as well: one two-block
// v_mfma_f32_32x32x1_2b_f32 gives it for two 32 x 32 blocks. That leaves two
// vector instructions per output and group, acc += float(256 P) * s, in fp32.
//
// Data path and schedule follow the MXFP4 kernel: persistent workgroups (one
// per CU) walk 128 x 256 tiles; direct buffer loads into LDS of 16 bytes per
// lane fill a ring of LDS slots across tile boundaries; eight waves, 2 (M) x
// 4 (N), each own 64 x 64 (2 x 2 blocks of 32 x 32); one workgroup barrier
// per 128-channel stage (two groups). The low-rank branch is r32/32 more
// stages on v_mfma_f32_32x32x16_bf16 into the same accumulators.
//
// Work split. Whole rounds of tiles go one per workgroup. The tiles left
// after them (between one and two rounds' worth, or all of them when there
// are fewer tiles than workgroups) are cut into their K stages and dealt out
// as equal contiguous runs of (tile, stage) pairs, so every workgroup ends at
// the same time. Each XCD deals its own share of those tiles (the ones the
// tile map gives it) over its own workgroups, which keeps their operand
// panels in that XCD's L2. A tile cut between runs belongs to the workgroup
// holding its first stage; that piece is the last of its run. The other
// pieces come first in their runs: each writes its fp32 partial to its own
// workspace slot and raises its flag; the owner adds the partials in
// workgroup order (the result does not depend on timing), clears the flags,
// and finishes the tile (low-rank stages, bias, Y). Stage 1 clears the flags
// before every GEMM.
#include "svdq_gemm_common.h"
#include "svdq_internal.h"
#include "svdq_layout.h"

namespace svdq {

namespace {
constexpr int kBM = 128, kBN = 256, kWGM = 2, kWGN = 4, kNW = kWGM * kWGN;
constexpr int kWM = kBM / kWGM, kWN = kBN / kWGN, kTM = kWM / 32, kTN = kWN / 32;
constexpr int kMB = kBM / 32, kNBt = kBN / 32;     // 32-row blocks per tile: 4 (A), 8 (B)
constexpr int kNStage = 4;
constexpr int kGroupM = 8;
constexpr int kStores = 2 * kTN * kTM;             // 16-byte Y stores per wave per tile
// Transfers per stage: 24 fragment blocks of 1 KiB (3 per wave, from 3 w)
// and 3 scale transfers of 1 KiB (A, then two of B) on waves 1, 2 and 3, or,
// in low-rank stages, copies of the bias transfer. Each SIMD (waves w and
// w + 4) issues 6 or 7 transfers per stage.
constexpr int kFragPerWave = 3;
__host__ __device__ constexpr int kScaleOp(int w) { return (w >= 1 && w <= 3) ? w - 1 : -1; }
__host__ __device__ constexpr int kOpsOf(int w) { return kFragPerWave + (kScaleOp(w) >= 0 ? 1 : 0); }
// one ring slot: A codes (4 blocks x 2 groups x 1 KiB), B codes (8 x 2 x 1 KiB),
// A scales fp32 [2 groups][128], B scales fp32 [2 groups][256]
constexpr int kCodeA = 0, kCodeB = kMB * 2 * 1024, kScA = kCodeB + kNBt * 2 * 1024;
constexpr int kScB = kScA + 2 * kBM * 4, kSlot = kScB + 2 * kBN * 4;
constexpr size_t kLds = (size_t)kNStage * kSlot;
static_assert(kTM == 2 && kTN == 2, "schedule below assumes 2 x 2 blocks per wave");
static_assert(kLds <= 160 * 1024, "ring must fit in LDS");
static_assert(kNW * kFragPerWave == 2 * (kMB + kNBt), "fragment blocks partition");
static_assert(2 * kBM * 4 == 1024 && 2 * kBN * 4 == 2048 && kBN * 2 <= 1024,
              "one A and two B scale transfers of 64 lanes; the bias fits the A scale area");

// Ring barrier: wait until at most n of this wave's vector-memory operations
// are outstanding and its LDS reads have returned, then s_barrier (the same
// rule as the MXFP4 kernel: operations retire in issue order, so n = the
// number issued after the transfer being waited for).
#define SVDQ_VMCNT(n) (((n) & 15) | (((n) >> 4) << 14) | 0x0070)   /* expcnt 7, lgkmcnt 0 */
__device__ __forceinline__ void ring_barrier(int n) {
  __builtin_amdgcn_sched_barrier(0);
  switch (n) {
    case 3: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(4)); break;
    case 6: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(6)); break;
    case 8: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(8)); break;
    case 11: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(11)); break;
    case 12: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(12)); break;
    case 14: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(14)); break;
    case 16: __builtin_amdgcn_s_waitcnt(SVDQ_VMCNT(16)); break;
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

// int8 operands of one 32-channel half of a group: 16*q of the even channels
// (lo) and of the odd channels (hi) of a 16-byte fragment
__device__ __forceinline__ void widen(const i32x4& w, i32x4& lo, i32x4& hi) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    lo[d] = (int)(((uint32_t)w[d] << 4) & 0xF0F0F0F0u);
    hi[d] = (int)((uint32_t)w[d] & 0xF0F0F0F0u);
  }
}

struct Geo {
  int M, N, K, MB, NB, KS, nst, nstt, tiles_m, tiles_n, act_rows;
  int tm_off, tn_off;   // group-sum hook: the window's first tile
  // whole tiles (indices below sk_base, a multiple of 8: rounds * grid),
  // then the sk_tiles tiles from index sk_base: tile index sk_base + 8 m + x
  // goes to XCD x, whose workgroups share its (tile, stage) pairs
  int rounds, sk_base, sk_tiles;
};
constexpr int kPartFloats = kBM * kBN;   // one fp32 partial tile
constexpr int kMinRun = 6;               // fewest stages per run of the split (when there are that many)
static_assert(kPartFloats * 4 == kSplitPartBytes, "workspace slot size");
}  // namespace

// DEBUG_P: instead of dequantizing, write every group sum P (exact int32) of
// the outputs inside the window [m0, m0 + mc) x [n0, n0 + nc) to p, over the
// window's tiles only, with the same transfers, widening and MFMAs.
template <bool DEBUG_P>
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
  struct Seg {
    int idx, ka, kb;
    bool owner;
  };
  auto seg_at = [&](int k, long long u) -> Seg {
    if (k < ncl) return Seg{wg + k * grid, 0, g.nst, true};
    const int m = (int)(u / g.nst), ka = (int)(u - (long long)m * g.nst);
    const int kb = (int)min((long long)g.nst, ka + (u1 - u));
    return Seg{g.sk_base + 8 * m + xcd, ka, kb, ka == 0};
  };
  auto seg_len = [&](const Seg& sg) { return sg.kb - sg.ka + (sg.owner && !DEBUG_P ? nlr : 0); };
  int total = 0;   // ring steps of this workgroup
  {
    int k = 0;
    for (long long u = u0; k < ncl || u < u1; ++k) {
      const Seg sg = seg_at(k, u);
      total += seg_len(sg);
      if (k >= ncl) u += sg.kb - sg.ka;
    }
  }

  // issue side: next ring step to load (step is_s of segment is_k)
  // and this wave's per-tile transfer sources as byte offsets from uniform
  // bases: fragment item 3 w + k from src[k] (4-bit) and src[3 + k]
  // (low-rank); the scale transfer from ssrc plus the stage times sstride;
  // the bias from bsrc
  const int frag0 = kFragPerWave * wave, sop = kScaleOp(wave);
  const int nops = kOpsOf(wave);
  int is_k = 0, is_s = 0, is_ka = 0, is_nk = 0, is_len = 0;   // segment, step in it, its stages
  long long is_u = u0;
  uint32_t src[2 * kFragPerWave], ssrc = 0, bsrc = 0, sstride = 0;
  const int per_l = a.r32 / 16;
  // every source as a buffer resource over the whole operand: a transfer is
  // one buffer load into LDS with the lane's 32-bit offset and the stage as
  // a scalar offset (the API keeps the codes below 4 GiB)
  auto rsrc = [](const void* p, uint64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)(uint32_t)min(bytes, (uint64_t)0xFFFFFFFFu),
                                             0x00020000);
  };
  const __amdgpu_buffer_rsrc_t rqx = rsrc(a.qx, (uint64_t)g.MB * g.KS * 1024);
  const __amdgpu_buffer_rsrc_t rqw = rsrc(a.qw, (uint64_t)g.NB * g.KS * 1024);
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
      _Pragma("unroll") for (int k = 0; k < kFragPerWave; ++k) {                                    \
        const int it = frag0 + k;                          /* fragment item 0..23 */               \
        const bool isA = it < 2 * kMB;                                                              \
        const int blk = isA ? (it >> 1) : ((it - 2 * kMB) >> 1);                                     \
        const uint32_t b = (uint32_t)min((isA ? mb0 : nb0) + blk, (isA ? g.MB : g.NB) - 1);         \
        src[k] = (b * g.KS + (it & 1)) * 1024 + lane * 16;                                          \
        src[kFragPerWave + k] = (b * per_l + (it & 1)) * 1024 + lane * 16;                          \
      }                                                                                             \
      if (sop >= 0) {                                                                               \
        /* entry e = 4 lane (+ 256 for the second B transfer) of [2 groups][T] */                  \
        const bool isA = sop == 0;                                                                  \
        const int T = isA ? kBM : kBN;                                                              \
        const int e = (sop == 2 ? 256 : 0) + 4 * lane;                                              \
        const int gg = e >= T ? 1 : 0, idx = e - gg * T;                                            \
        const int lim = isA ? g.act_rows : g.N;                                                     \
        const int row = min((isA ? mb0 : nb0) * 32 + idx, lim - 4);                                 \
        ssrc = (uint32_t)(gg * lim + row) * 4;                                                      \
        sstride = (uint32_t)(2 * lim * 4);                                                          \
      }                                                                                             \
      bsrc = (uint32_t)min(nb0 * 32 + 8 * lane, g.N - 8) * 2;                                       \
    }                                                                                               \
    uint8_t* slot_w = smem + ((GS) % kNStage) * kSlot;                                              \
    const bool lrs = is_s >= is_nk;                                                                 \
    const int sl = lrs ? is_s - is_nk : is_ka + is_s;                                               \
    if (lrs && a.r32 == 0) {                                                                        \
      /* no low-rank fragments: every transfer of the stage moves the bias */                      \
      _Pragma("unroll") for (int k = 0; k < kFragPerWave + 1; ++k)                                  \
        if (k < nops && lane < 32) __builtin_amdgcn_raw_ptr_buffer_load_lds(rbias, lds_ptr(slot_w + kScA), 16, bsrc, 0, 0, 0); \
    } else {                                                                                        \
      _Pragma("unroll") for (int k = 0; k < kFragPerWave; ++k) {                                    \
        const int it = frag0 + k;                                                                   \
        const bool isA = it < 2 * kMB;                                                              \
        const int dst = isA ? kCodeA + it * 1024 : kCodeB + (it - 2 * kMB) * 1024;                  \
        const __amdgpu_buffer_rsrc_t rs = lrs ? (isA ? rz : rl2) : (isA ? rqx : rqw);                \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr(slot_w + dst), 16, src[(lrs ? kFragPerWave : 0) + k], \
                                                 sl * 2048, 0, 0);                                  \
      }                                                                                             \
      if (sop >= 0) {                                                                               \
        if (lrs) {                                                                                  \
          if (lane < 32) __builtin_amdgcn_raw_ptr_buffer_load_lds(rbias, lds_ptr(slot_w + kScA), 16, bsrc, 0, 0, 0); \
        } else {                                                                                    \
          __builtin_amdgcn_raw_ptr_buffer_load_lds(sop == 0 ? rsx : rsw,                            \
                                                   lds_ptr(slot_w + (sop == 0 ? kScA : kScB + 1024 * (sop - 1))), 16, \
                                                   ssrc, sl * sstride, 0, 0);                       \
        }                                                                                           \
      }                                                                                             \
    }                                                                                               \
    if (++is_s == is_len) {                                                                         \
      is_s = 0;                                                                                     \
      if (is_k >= ncl) is_u += is_nk;                                                               \
      ++is_k;                                                                                       \
    }                                                                                               \
  }

  f32x16 acc[kTN][kTM];

  // The two groups of a stage are eight units u = (group u / 4, block
  // j = (u / 2) % 2, i = u % 2). A unit is two i8 MFMAs for 256 P, one fp32
  // MFMA for the scale outer product, and the dequant of its 16 outputs per
  // lane (or, DEBUG_P, the group-sum writes). Units are software-pipelined
  // within the wave: the MFMAs of unit u + 1 are issued before the vector
  // work of unit u, so the matrix pipe and the vector ALU run side by side.
  int gs = 0, stores_due = 0;   // ring step being computed; ring steps still to absorb Y stores
  i32x4 alo[2][kTM], ahi[2][kTM], blo[2][kTN], bhi[2][kTN];
  float sxv[2][kTM], swv[2][kTN];
  i32x16 pp[2];
  f32x16 sc[2][2];   // [block pair (u / 2) % 2][i]
  auto mfma_unit = [&](int u) {
    const int gg = u >> 2, j = (u >> 1) & 1, i = u & 1;
    i32x16 p = __builtin_amdgcn_mfma_i32_32x32x32_i8(blo[gg][j], alo[gg][i], i32x16{}, 0, 0, 0);
    pp[u & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bhi[gg][j], ahi[gg][i], p, 0, 0, 0);
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
    const i32x16& p = pp[u & 1];
    if constexpr (DEBUG_P) {
      const int tok = m0t + wm * kWM + 32 * i + lr;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int ch = n0t + wn * kWN + 32 * j + 8 * (e >> 2) + 4 * h + (e & 3);
        if (tok >= a.m0 && tok < a.m0 + a.mc && ch >= a.n0 && ch < a.n0 + a.nc)
          a.p[((size_t)(tok - a.m0) * a.nc + (ch - a.n0)) * (g.K / 64) + 2 * st + gg] = p[e] / 256;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][i][e] = __builtin_fmaf((float)p[e], sc[(u >> 1) & 1][i][e], acc[j][i][e]);
    }
  };
  // One stage: raw fragments and scales of both groups are read from LDS up
  // front; then eight pipeline steps, each its own scheduling region: the 3
  // MFMAs of unit u + 1 spread over the ~32 vector instructions of unit u
  // (step 2 also widens group 1, which unit 4 needs).
  auto stage_compute = [&](const uint8_t* slot, int st, int m0t, int n0t) {
    i32x4 ra[2][kTM], rb[2][kTN];
    float rsx[2][kTM], rsw[2][kTN];
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
#pragma unroll
      for (int t = 0; t < kTM; ++t) {
        ra[gg][t] = *reinterpret_cast<const i32x4*>(slot + kCodeA + ((wm * kTM + t) * 2 + gg) * 1024 + lane * 16);
        rsx[gg][t] = *reinterpret_cast<const float*>(slot + kScA + gg * (kBM * 4) + (wm * kWM + 32 * t + lr) * 4);
      }
#pragma unroll
      for (int t = 0; t < kTN; ++t) {
        rb[gg][t] = *reinterpret_cast<const i32x4*>(slot + kCodeB + ((wn * kTN + t) * 2 + gg) * 1024 + lane * 16);
        rsw[gg][t] = *reinterpret_cast<const float*>(slot + kScB + gg * (kBN * 4) + (wn * kWN + 32 * t + lr) * 4);
      }
    }
    // int8 operands; the token scale carries the 1/256 of the widened codes
    auto widen_group = [&](int gg) {
#pragma unroll
      for (int t = 0; t < kTM; ++t) {
        widen(ra[gg][t], alo[gg][t], ahi[gg][t]);
        sxv[gg][t] = rsx[gg][t] * (1.0f / 256.0f);
      }
#pragma unroll
      for (int t = 0; t < kTN; ++t) {
        widen(rb[gg][t], blo[gg][t], bhi[gg][t]);
        swv[gg][t] = rsw[gg][t];
      }
    };
    widen_group(0);
    mfma_unit(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u == 2) widen_group(1);
      if (u + 1 < 8) mfma_unit(u + 1);
      valu_unit(u, st, m0t, n0t);
      if (u == 2) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 28, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 28, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 40, 0);
      } else if (u + 1 < 8) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 14, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // prologue: the first kNStage - 1 ring steps in flight
  for (int p = 0; p < kNStage - 1 && p < total; ++p) SVDQ_ISSUE(p)
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
      ring_barrier(DEBUG_P ? 0 : nops * min(kNStage - 2, total - 1 - gs) + (stores_due > 0 ? kStores : 0));
      if (stores_due > 0) --stores_due;
      if (gs + kNStage - 1 < total) SVDQ_ISSUE(gs + kNStage - 1)
      stage_compute(smem + (gs % kNStage) * kSlot, st, m0t, n0t);
      ++gs;
    }
    if constexpr (DEBUG_P) continue;
    if (!sg.owner) {
      // a later piece of a tile (the first segment of this run): publish the
      // partial in this workgroup's slot, then its flag
#pragma unroll
      for (int f = 0; f < 16; ++f) {
        const f32x16& v = acc[f >> 3][(f >> 2) & 1];
        *reinterpret_cast<f32x4*>(part_at(wg, f)) = f32x4{v[4 * (f & 3)], v[4 * (f & 3) + 1], v[4 * (f & 3) + 2], v[4 * (f & 3) + 3]};
      }
      __builtin_amdgcn_s_waitcnt(0);   // every store of every wave has landed ...
      __syncthreads();                  // ... before the flag is raised
      if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_store(a.flags + wg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      continue;
    }
    if (ck >= ncl && sg.kb < g.nst) {
      // the first piece of a tile that later runs continued: add their
      // partials in workgroup order (the flags bound the wait; they are set
      // early in those runs, so it is normally already over)
      const long long tile_end = (long long)((sg.idx - g.sk_base - xcd) / 8 + 1) * g.nst;
      for (int k = kx + 1; k < xruns && run_begin(k) < tile_end; ++k) {
        const int w = xcd + 8 * k;   // the workgroup of that run
        if (tid == 0) {
          for (int spin = 0; spin < (1 << 22) && __hip_atomic_load(a.flags + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u; ++spin)
            __builtin_amdgcn_s_sleep(2);
          __hip_atomic_store(a.flags + w, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
        for (int f = 0; f < 16; ++f) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(part_at(w, f));
          f32x16& d = acc[f >> 3][(f >> 2) & 1];
#pragma unroll
          for (int e = 0; e < 4; ++e) d[4 * (f & 3) + e] += v[e];
        }
      }
    }
    for (int l = 0; l < nlr; ++l) {
      ring_barrier(nops * min(kNStage - 2, total - 1 - gs) + (stores_due > 0 ? kStores : 0));
      if (stores_due > 0) --stores_due;
      const bool more = gs + kNStage - 1 < total;
      if (more && wave < 4) SVDQ_ISSUE(gs + kNStage - 1)
      const uint8_t* slot = smem + (gs % kNStage) * kSlot;
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
      if (more && wave >= 4) SVDQ_ISSUE(gs + kNStage - 1)
      ++gs;
    }

    // + bias (from the last low-rank slot), bf16 write: the MXFP4 kernel's
    // epilogue. Lane h of the accumulator holds channels 32 j + 8 q + 4 h +
    // (0..3) of token m0 + 32 i + lr; after swapping the packed pairs (q = 1,
    // h = 0) <-> (q = 0, h = 1) and (q = 3, h = 0) <-> (q = 2, h = 1), each
    // lane stores two 16-byte runs of one row.
    const uint8_t* bslot = smem + ((gs - 1) % kNStage) * kSlot + kScA + wn * kWN * 2;
    const int ynrec = min(g.M - m0t, kBM) * g.N * 2;
    const __amdgpu_buffer_rsrc_t yrs =
        __builtin_amdgcn_make_buffer_rsrc(a.y + (size_t)m0t * g.N, 0, ynrec, 0x00020000);
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
        for (int p = 0; p < 2; ++p) {
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
#undef SVDQ_ISSUE
}

hipError_t prepare_gemm_int4() {
  hipError_t e = hipFuncSetAttribute((const void*)gemm_int4_kernel<false>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void*)gemm_int4_kernel<true>,
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
  g.tm_off = g.tn_off = 0;
  int grid = num_cus > 0 ? num_cus : 256;
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
    hipLaunchKernelGGL(gemm_int4_kernel<true>, dim3(grid), dim3(64 * kNW), kLds, st, a, g, grid);
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
    // whole rounds while at least one more round's worth of tiles remains
    g.rounds = ntiles / grid > 1 ? ntiles / grid - 1 : 0;
    g.sk_base = g.rounds * grid;
    g.sk_tiles = ntiles - g.sk_base;
  } else {
    g.rounds = (ntiles + grid - 1) / grid;
    g.sk_base = ntiles;   // whole tiles only
    g.sk_tiles = 0;
  }
  hipLaunchKernelGGL(gemm_int4_kernel<false>, dim3(grid), dim3(64 * kNW), kLds, st, a, g, grid);
  return hipGetLastError();
}

}  // namespace svdq
