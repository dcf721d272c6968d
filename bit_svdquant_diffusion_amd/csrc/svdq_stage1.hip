// Kernel (1) of the forward: one read of X feeds three steps.
//   - smoothing: x_hat = fl32(x * mu_k) (aiflownews.com, "What SVDQuant actually
//     does": activation outliers are moved into the weights, so the runtime
//     divides X by lambda; mu = 1/lambda is stored);
//   - per-token 4-bit quantization of x_hat (INT4 per 64 channels, or MXFP4
//     per 32 channels);
//   - the low-rank down-projection Z = x_hat L1 on bf16 MFMA, with x_hat
//     rounded to bf16 (same page: the low-rank branch stays in a 16-bit
//     format, and both branches read the same smoothed input).
//
// Work split: a workgroup owns 16 TH tokens (TH = 1 or 2 halves of 16) and
// walks K in steps of 256 channels; wave w = 4 th + q takes the 64-channel
// quarter q of every step for the 16 tokens of half th, so a wave's quarter
// holds exactly one INT4 group (two MXFP4 blocks) per token. The two halves
// share each step's L1 fragments (each half loads half of them), which halves
// the L1 bytes per token. Lane (r = l%16, j = l/16) holds token r of its half
// and channels 16j .. 16j+15 of the quarter. Per step a wave
//   1. finds its quarter of X (16 tokens x 128 bytes), of mu and of L1 in
//      LDS, moved there by direct global->LDS transfers issued D steps ahead
//      into a ring of D + 1 slots (with two halves, a workgroup barrier after
//      the wait makes the other half's L1 transfers visible). Vector-memory
//      operations retire in issue order, so each wait names exactly the
//      operations issued after what it waits for; no register load is
//      outstanding across a wait (a register load would make the compiler
//      drain every transfer in flight);
//   2. reads its 16 values of x, multiplies by mu (x_hat = fl32(x mu));
//   3. quantizes: the group (block) absolute maximum is combined across the 4
//      (2) lanes that share it with lane swaps; codes are stored as 8 bytes;
//   4. accumulates Z on 16x16x32 bf16 MFMAs (two per 16 columns of L1).
// X lands in LDS through direct global->LDS transfers whose per-lane source
// addresses lay each token's 128 bytes out with its 16-byte chunks XOR-
// swizzled by the token index, so the read-back is free of bank conflicts.
// The four partial Z tiles are summed in LDS in wave order (deterministic)
// and stored as bf16.
#include <type_traits>

#include "svdq_device.h"
#include "svdq_internal.h"
#include "svdq_layout.h"

namespace svdq {

constexpr int S1_ROWS = 16;
constexpr int S1_STEP = 256;                 // channels per step
constexpr int S1_WAVES = 4;                  // one 64-channel quarter each
constexpr int S1_XQ = S1_ROWS * 64 * 2;      // bytes of one wave's X quarter (2 KiB)

typedef __attribute__((address_space(3))) void s1_lds_void;
// s_waitcnt operand: vmcnt n (n < 64), expcnt and lgkmcnt not waited on
#define S1_VMCNT(n) (((n) & 15) | (((n) >> 4) << 14) | 0x0070 | 0x0f00)

// Ring slot: X of the 4 TH waves, mu of the step, then each quarter's 2 NCB
// L1 fragments of 1 KiB. Depth: a single half with 16 KiB of L1 or less per
// step fits two workgroups per CU (80 KiB each), otherwise one workgroup per
// CU; at most 7 steps. Vector-memory operations of one step and wave, in
// issue order: the ring transfers D steps ahead (2 X, 1 mu, 2 NCB / TH L1),
// then the two stores (codes, scale; every wave issues them, lanes past M
// repeating the identical values of token M - 1). After step i's transfers
// are issued, what follows them when step i waits is: in the first D steps,
// the later prologue transfers and the whole steps before i; afterwards, the
// stores of step i - D and the D - 1 steps between. The largest count must
// fit the 63 operations a wave can have outstanding.
template <int NCB, int TH> struct S1Cfg {
  static constexpr int kL1PerWave = 2 * NCB / TH;
  static constexpr int kX = 3 + kL1PerWave, kSt = 2;
  static constexpr int kPerStep = kX + kSt;
  static constexpr int kMu = TH * S1_WAVES * S1_XQ;   // offset of the step's mu
  static constexpr int kL1 = kMu + S1_STEP * 4;       // offset of the step's L1 fragments
  static constexpr int kSlot = kL1 + S1_WAVES * 2 * NCB * 1024;
  static constexpr int kBudget = (TH == 1 && NCB <= 2 ? 80 : 160) * 1024;
  static constexpr int kDepthL = kBudget / kSlot - 1;
  static constexpr int kDepthV = 1 + (61 - kSt) / kPerStep;
  static constexpr int kDepth = kDepthL < kDepthV ? (kDepthL < 7 ? kDepthL : 7) : (kDepthV < 7 ? kDepthV : 7);
  static constexpr int count(int i) {   // operations issued after step i's transfers
    return i < kDepth ? kX * (kDepth - 1 - i) + i * kPerStep : kSt + (kDepth - 1) * kPerStep;
  }
  static_assert(TH == 1 || NCB % 2 == 0, "two halves split the L1 fragments evenly");
  static_assert(kDepth >= 1, "ring needs two slots");
  static_assert(count(kDepth) <= 62, "wait count out of range");
};

// max over the lanes l and l ^ 16 (and l ^ 32): each swap returns, between
// its two results, the lane's own value and its partner's
__device__ __forceinline__ float s1_max16(float a) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return __builtin_fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float s1_max32(float a) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return __builtin_fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}


template <int FMT, int NCB, int TH>
__global__ __launch_bounds__(64 * S1_WAVES * TH) void stage1_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ mu, const uint16_t* __restrict__ l1s,
    uint8_t* __restrict__ qx, void* __restrict__ sx, uint16_t* __restrict__ z, float* __restrict__ zp, int M,
    int K, int XK, uint32_t* __restrict__ flags, int nflags, int ps, int npieces, int grid, int split) {
  using Cfg = S1Cfg<NCB, TH>;
  constexpr int D = Cfg::kDepth;
  constexpr int r32 = NCB * 16;
  constexpr int FPW = Cfg::kL1PerWave;
  constexpr int TG = S1_ROWS * TH;   // tokens per group
  constexpr int NT = 64 * S1_WAVES * TH;
  static_assert(NCB == 0 || TH * S1_WAVES * NCB * 4 * 64 * 4 <= Cfg::kSlot, "Z reduction fits a ring slot");
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = wave & 3, th = wave >> 2;   // quarter and token half
  const int nsteps = K / S1_STEP;
  const int npc = (nsteps + ps - 1) / ps;   // K pieces (of ps steps) per token group
  const int Mp = (M + 15) / 16 * 16;   // row stride of the INT4 scales
  const int MB = (M + 31) / 32;        // 32-row blocks (MXFP4 fragment order)

  // the INT4 GEMM that follows on the stream expects its split flags clear
  if (blockIdx.x == 0)
    for (int f = threadIdx.x; f < nflags; f += NT) flags[f] = 0u;

  const int r = lane & 15, j = lane >> 4;
  // X transfer d (0, 1) of this lane: 16-byte unit u = 64 d + lane of the
  // quarter, token u / 8, chunk (u % 8) ^ ((token / 2) % 8)
  const int tA = lane >> 3, tB = 8 + (lane >> 3);
  // read-back of chunks 2j, 2j+1 of token r
  const int rd0 = (r * 8 + ((2 * j) ^ ((r >> 1) & 7))) * 16;
  const int rd1 = (r * 8 + ((2 * j + 1) ^ ((r >> 1) & 7))) * 16;

  // This workgroup's pieces (token group g = p / npc, K piece p % npc) and
  // the steps they hold, walked as one sequence. Without `split` the grid is
  // one workgroup per group and holds all its pieces.
  const int pb = (int)((int64_t)npieces * blockIdx.x / grid), pe = (int)((int64_t)npieces * (blockIdx.x + 1) / grid);
  int T = 0;
  for (int p = pb; p < pe; ++p) T += min(ps, nsteps - (p % npc) * ps);

  // issue cursor: piece ip (group ig, piece ic in it), step is (absolute),
  // its end. The cursors advance by increments: a group's rows are set up
  // only when the group changes. The transfers are buffer loads into LDS: X
  // through a resource over the half's 16 rows, mu and L1 through resources
  // over the whole vectors; each lane's offset is fixed per group and the
  // step adds a scalar offset (no per-transfer address arithmetic).
  int ip = pb, ig = pb / npc, ic = pb - (pb / npc) * npc, is = 0, iend = 0, iu = 0;
  __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)x, 0, 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t rmu = __builtin_amdgcn_make_buffer_rsrc((void*)mu, 0, XK * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rl1 = __builtin_amdgcn_make_buffer_rsrc((void*)l1s, 0, K * NCB * 32, 0x00020000);
  int vA = 0, vB = 0;   // the lane's X offsets (bytes) in the half's rows
  const int vmu = (q * 64 + lane) * 4;
  auto issue_group = [&]() {
    // rows past M read row M - 1 (a half wholly past M reads it throughout).
    // X's rows are XK channels; the steps run over K >= XK, and the reads of
    // channels past XK (zeroed after the read) stay inside the resource,
    // which ends with X's last row, or read zeros past it.
    const int m0 = ig * TG + th * S1_ROWS, m0c = min(m0, M - 1);
    rx = __builtin_amdgcn_make_buffer_rsrc((void*)(x + (size_t)m0c * XK), 0, (min(M, m0c + S1_ROWS) - m0c) * XK * 2,
                                           0x00020000);
    vA = ((min(m0 + tA, M - 1) - m0c) * XK + q * 64 + ((lane & 7) ^ ((tA >> 1) & 7)) * 8) * 2;
    vB = ((min(m0 + tB, M - 1) - m0c) * XK + q * 64 + ((lane & 7) ^ ((tB >> 1) & 7)) * 8) * 2;
  };
  is = ic * ps;
  iend = min(is + ps, nsteps);
  issue_group();
  // compute cursor: piece cp (group cg, piece cc in it), step cs, its end;
  // the lane's token m (a lane past M holds token M - 1's values, its X rows
  // being clamped, and stores them again, so every store always issues)
  int cp = pb, cg = ig, cc = ic, cs = is, cend = iend, m = 0;
  f32x4 zacc[NCB > 0 ? NCB : 1];   // this piece's partial Z of the wave's quarter
  f32x4 zrun[NCB > 0 ? NCB : 1];   // the sum over the group's pieces so far (whole-group mode)
#pragma unroll
  for (int c = 0; c < NCB; ++c) zrun[c] = f32x4{};
  // Stores as buffer stores: the codes through a resource over the group
  // half's 32-row block (every lane's m lies in it, rows past M included),
  // the scales through one over the whole scale area; each lane's offset is
  // fixed per group and the step adds a scalar offset.
  __amdgpu_buffer_rsrc_t rcode = rx;
  int vcode = 0, vsx = 0;
  const __amdgpu_buffer_rsrc_t rsx = __builtin_amdgcn_make_buffer_rsrc(
      sx, 0, FMT == SVDQ_FMT_INT4_G64 ? (K / 64) * Mp * 4 : (K / 128) * MB * 128, 0x00020000);
  auto compute_group = [&]() {
    m = min(cg * TG + th * S1_ROWS + r, M - 1);
    const int rb = min(cg * TG + th * S1_ROWS, M - 1) / 32;
    rcode = __builtin_amdgcn_make_buffer_rsrc(qx + (size_t)rb * (K / 64) * 1024, 0, K * 16, 0x00020000);
    vcode = (32 * (j >> 1) + m % 32) * 16 + (j & 1) * 8;
    // INT4: fp32 [K/64][Mp]; MXFP4: the byte of 32-channel block
    // kb = k0 / 32 + j / 2, k0 = 256 cs + 64 q, at ((kb / 4) MB + m / 32) 128
    // + (32 (kb % 2) + m % 32) 2 + (kb / 2) % 2, whose step part is 256 MB cs
    vsx = FMT == SVDQ_FMT_INT4_G64 ? m * 4
                                   : ((q >> 1) * MB + m / 32) * 128 + (32 * (j >> 1) + m % 32) * 2 + (q & 1);
  };
  compute_group();
#pragma unroll
  for (int c = 0; c < NCB; ++c) zacc[c] = f32x4{};
  // the next piece of the compute cursor (cs is already its first step)
  auto compute_next = [&]() {
    if (++cc == npc) {
      cc = 0;
      cs = 0;
      ++cg;
      compute_group();
    }
    cend = min(cs + ps, nsteps);
#pragma unroll
    for (int c = 0; c < NCB; ++c) zacc[c] = f32x4{};
  };

  // ring transfers of the next step of the issue cursor; past the last step
  // they re-read the first bytes of X and mu into the slot, so every step
  // issues the same number
#define S1_ISSUE()                                                                                 \
  {                                                                                                \
    const int st_ = iu < T ? is : 0;   /* past the last step: step 0 of the current rows */        \
    uint8_t* slot_ = smem + (iu % (D + 1)) * Cfg::kSlot;                                           \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (s1_lds_void*)(slot_ + wave * S1_XQ), 16, vA, st_ * S1_STEP * 2, 0, 0);        \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (s1_lds_void*)(slot_ + wave * S1_XQ + 1024), 16, vB, st_ * S1_STEP * 2, 0, 0); \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rmu, (s1_lds_void*)(slot_ + Cfg::kMu + q * 256), 4, vmu, st_ * S1_STEP * 4, 0, 0); \
    _Pragma("unroll") for (int f_ = th * FPW; f_ < (th + 1) * FPW; ++f_)                           \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl1, (s1_lds_void*)(slot_ + Cfg::kL1 + (q * 2 * NCB + f_) * 1024), 16,   \
                                               ((q * NCB * 2 + f_) * 64 + lane) * 16, st_ * S1_WAVES * NCB * 2048, 0, 0); \
    if (iu < T && ++is == iend && ++ip < pe) {                                                     \
      if (++ic == npc) {                                                                           \
        ic = 0;                                                                                    \
        is = 0;                                                                                    \
        ++ig;                                                                                      \
        issue_group();                                                                             \
      }                                                                                            \
      iend = min(is + ps, nsteps);                                                                 \
    }                                                                                              \
    ++iu;                                                                                          \
  }
#define S1_WAIT_CASE(k)                                                                            \
  case k: __builtin_amdgcn_s_waitcnt(S1_VMCNT(Cfg::count(k < D ? k : D))); break;

#pragma unroll
  for (int d = 0; d < D; ++d) S1_ISSUE()

  // One step of the walk. The first D steps wait for counts that depend on
  // the step; every later step waits for the same count, so the walk runs
  // them in a second copy of the body whose wait is a constant.
  auto step = [&](const int i, auto steady) {
        // 1. step i's transfers have landed once only the operations issued
        //    after them are outstanding (a finished piece's partial-Z stores
        //    only add to those: the wait gets longer, never shorter)
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(steady)::value) {
          __builtin_amdgcn_s_waitcnt(S1_VMCNT(Cfg::count(D)));
        } else {
          switch (i) {
            S1_WAIT_CASE(0) S1_WAIT_CASE(1) S1_WAIT_CASE(2) S1_WAIT_CASE(3)
            S1_WAIT_CASE(4) S1_WAIT_CASE(5) S1_WAIT_CASE(6) S1_WAIT_CASE(7)
            default: __builtin_amdgcn_s_waitcnt(S1_VMCNT(0)); break;
          }
        }
        // both halves' L1 transfers are in: the other half's become visible
        // at the barrier, which also means every wave is done reading the
        // slot that the transfers below refill
        if constexpr (TH > 1) __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        uint8_t* slot = smem + (i % (D + 1)) * Cfg::kSlot;
        u32x4 l1v[NCB > 0 ? 2 * NCB : 1];
#pragma unroll
        for (int f = 0; f < 2 * NCB; ++f)
          l1v[f] = *reinterpret_cast<const u32x4*>(slot + Cfg::kL1 + (q * 2 * NCB + f) * 1024 + lane * 16);
        const u32x4 xa = *reinterpret_cast<const u32x4*>(slot + wave * S1_XQ + rd0);
        const u32x4 xb = *reinterpret_cast<const u32x4*>(slot + wave * S1_XQ + rd1);
        const float* mus = reinterpret_cast<const float*>(slot + Cfg::kMu + q * 256) + 16 * j;
        f32x4 muv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) muv[t] = *reinterpret_cast<const f32x4*>(mus + 4 * t);
        // the slot of step i + D is the one read at step i - 1: its reads are
        // complete (they were waited on before their use)
        __builtin_amdgcn_sched_barrier(0);
        S1_ISSUE()
        __builtin_amdgcn_sched_barrier(0);
        const int k0 = cs * S1_STEP + q * 64;   // first channel of the quarter
        // a quarter past the layer's channels (padding up to whole steps) is zero
        // (an all-ones or all-zeros mask ANDed into the products: a select per
        // value would be compiled into branches that copy the whole array)
        const uint32_t live = k0 < XK ? 0xFFFFFFFFu : 0u;
        float xh[16];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const f32x4 mv = muv[t];
          const u32x4& xw = t < 2 ? xa : xb;
          const uint32_t w0 = xw[(t & 1) * 2], w1 = xw[(t & 1) * 2 + 1];
          xh[4 * t + 0] = __uint_as_float(__float_as_uint(bf16lo(w0) * mv.x) & live);
          xh[4 * t + 1] = __uint_as_float(__float_as_uint(bf16hi(w0) * mv.y) & live);
          xh[4 * t + 2] = __uint_as_float(__float_as_uint(bf16lo(w1) * mv.z) & live);
          xh[4 * t + 3] = __uint_as_float(__float_as_uint(bf16hi(w1) * mv.w) & live);
        }

        // 3. Z += bf16(x_hat) L1: MFMA t takes channels 16j + 8t .. +7 of each lane
        if constexpr (NCB > 0) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const u32x4 av = u32x4{cvt_bf16x2(xh[8 * t + 0], xh[8 * t + 1]), cvt_bf16x2(xh[8 * t + 2], xh[8 * t + 3]),
                                   cvt_bf16x2(xh[8 * t + 4], xh[8 * t + 5]), cvt_bf16x2(xh[8 * t + 6], xh[8 * t + 7])};
#pragma unroll
            for (int c = 0; c < NCB; ++c)
              zacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                               __builtin_bit_cast(bf16x8, l1v[2 * c + t]), zacc[c], 0, 0, 0);
          }
        }


        // 4. quantize
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(xh[e]));
        amax = s1_max16(amax);                   // the lane pair 16 channels apart
        uint32_t c0, c1;
        if constexpr (FMT == SVDQ_FMT_INT4_G64) {
          amax = s1_max32(amax);                 // the 4 lanes of the 64-channel group
          const float sc = amax / 7.0f;          // IEEE-rounded division
          int4_codes16(xh, sc, c0, c1);
          if (j == 0) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), rsx, vsx, (cs * 4 + q) * Mp * 4, 0);
        } else {
          const int e = mx_exponent(amax);       // block b = j / 2 of the quarter
          c0 = e2m1x8_codes(xh, e);
          c1 = e2m1x8_codes(xh + 8, e);
          if ((j & 1) == 0) {
            // fragment-order scale byte of 32-channel block kb = k0/32 + j/2:
            // stage kb/4, step (kb%4)/2, half kb%2
            __builtin_amdgcn_raw_buffer_store_b8((unsigned char)(e + 127), rsx, vsx, cs * MB * 256, 0);
          }
        }
        {
          // fragment order: 64-channel step k0/64 of row block m/32; channels
          // 32h .. 32h+31 at lane 32h + m%32, 16 channels = 8 bytes
          __builtin_amdgcn_raw_buffer_store_b64(u32x2{c0, c1}, rcode, vcode, (cs * 4 + q) * 1024, 0);
        }


        // 5. end of a piece: add the wave's partial Z to the group's running
        //    sum, or store it (raw accumulators) for the piece-sum kernel
        if (++cs == cend) {
          if constexpr (NCB > 0) {
            if (split) {
              f32x4* dst = reinterpret_cast<f32x4*>(zp) + ((size_t)cp * (S1_WAVES * TH) + wave) * NCB * 64 + lane;
#pragma unroll
              for (int c = 0; c < NCB; ++c) dst[c * 64] = zacc[c];
            } else {
#pragma unroll
              for (int c = 0; c < NCB; ++c) zrun[c] = cc == 0 ? zacc[c] : zrun[c] + zacc[c];
            }
          }
          ++cp;
          if (cp < pe) compute_next();
        }
  };
  const int T0 = T < D ? T : D;
  for (int i = 0; i < T0; ++i) step(i, std::false_type{});
  for (int i = T0; i < T; ++i) step(i, std::true_type{});
#undef S1_ISSUE
#undef S1_WAIT_CASE
  // the transfers issued past the last step still write the ring
  __builtin_amdgcn_s_waitcnt(S1_VMCNT(0));

  if constexpr (NCB > 0) {
    if (split) return;
    // whole-group mode: add the four quarters' sums in wave order and store bf16
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
#pragma unroll
      for (int e = 0; e < 4; ++e) red[((wave * NCB + c) * 4 + e) * 64 + lane] = zrun[c][e];
    }
    __syncthreads();
    constexpr int per = NCB * 4 * 64;   // one wave's partial tile
    for (int idx = threadIdx.x; idx < TH * per; idx += NT) {
      const int h = idx / per, rem = idx - h * per;
      float acc = 0.f;
      for (int w = 0; w < S1_WAVES; ++w) acc += red[(h * S1_WAVES + w) * per + rem];
      // 16x16 result layout: lane l, reg e -> row 4(l/16) + e, column l%16
      const int l = rem & 63, e = (rem >> 6) & 3, c = rem >> 8;
      const int row = cg * TG + h * S1_ROWS + 4 * (l >> 4) + e;
      const int col = 16 * c + (l & 15);
      if (row < M)   // fragment order: (row block, 16-column step, lane 32h + row%32, element)
        z[((((size_t)(row / 32) * (r32 / 16) + col / 16) * 64 + 32 * ((col % 16) / 8) + row % 32) * 8) + col % 8] =
            (uint16_t)f2bf(acc);
    }
  }
}

// Z = bf16 of the sum, over the four quarters in wave order, of each
// quarter's sum over the K pieces in piece order (the whole-group path's
// additions, in its order), stored in fragment order: (row block, 16-column
// step, lane 32h + row%32, element). zp holds, per token group and piece,
// each wave's raw accumulators [wave][16-column block][lane][4]. Four lanes
// per element, one per quarter, each load all pieces of their quarter at
// once; lane 0 of the four then adds the quarter sums in order.
__global__ __launch_bounds__(256) void zsum_kernel(const float* __restrict__ zp, uint16_t* __restrict__ z, int M,
                                                   int r32, int npc, int th_n) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t idx = t >> 2;   // output element; the four lanes of a quad share it
  const int qq = (int)(t & 3);
  if (idx >= (int64_t)M * r32) return;
  const int row = (int)(idx / r32), col = (int)(idx - (int64_t)row * r32);
  const int tg = S1_ROWS * th_n, ncb = r32 / 16;
  const int g = row / tg, h = (row % tg) / S1_ROWS, rr = row % S1_ROWS;
  const int n = col / 16, l = (rr / 4) * 16 + col % 16, e = rr % 4;
  const size_t pstride = (size_t)(S1_WAVES * th_n) * ncb * 256;   // next piece of the group
  const size_t base = ((size_t)(g * npc) * (S1_WAVES * th_n) + h * S1_WAVES + qq) * ncb * 256 + ((size_t)n * 64 + l) * 4 + e;
  float v[kS1Pieces];
#pragma unroll
  for (int c = 0; c < kS1Pieces; ++c) v[c] = zp[base + (size_t)min(c, npc - 1) * pstride];
  float sum = v[0];
#pragma unroll
  for (int c = 1; c < kS1Pieces; ++c)
    if (c < npc) sum += v[c];
  const int q0 = (int)(threadIdx.x & 60u);   // lane of quarter 0 of this quad
  const float s0 = __shfl(sum, q0), s1 = __shfl(sum, q0 + 1), s2 = __shfl(sum, q0 + 2), s3 = __shfl(sum, q0 + 3);
  if (qq != 0) return;
  float acc = 0.f;
  acc += s0;
  acc += s1;
  acc += s2;
  acc += s3;
  z[((((size_t)(row / 32) * (r32 / 16) + col / 16) * 64 + 32 * ((col % 16) / 8) + row % 32) * 8) + col % 8] =
      (uint16_t)f2bf(acc);
}

template <int FMT, int NCB, int TH>
static size_t lds_bytes() {
  using Cfg = S1Cfg<NCB, TH>;
  return (size_t)(Cfg::kDepth + 1) * Cfg::kSlot;
}

// With at least half as many token groups as CUs, one workgroup per group
// walks all of K. With fewer, the groups' K pieces are dealt over the CUs
// (each CU then streams fewer steps) and a second kernel adds the partials.
template <int FMT, int NCB, int TH>
static hipError_t launch_t(const Stage1Args& a, int num_cus, hipStream_t st) {
  constexpr int TG = S1_ROWS * TH;
  const int groups = (a.M + TG - 1) / TG, npc = s1_pieces(a.K), ps = s1_piece_steps(a.K);
  const int cus = num_cus > 0 ? num_cus : 256;
  const size_t lds = lds_bytes<FMT, NCB, TH>();
  const int per_cu = lds <= 80 * 1024 ? 2 : 1;   // workgroups that fit one CU's LDS
  const bool split = NCB > 0 && npc > 1 && 2 * groups < cus && (int64_t)groups * TG <= kS1SplitRows;
  const int grid = split ? min(groups * npc, cus * per_cu) : groups;
  hipLaunchKernelGGL((stage1_kernel<FMT, NCB, TH>), dim3(grid), dim3(64 * S1_WAVES * TH), lds, st, a.x, a.mu,
                     a.l1s, a.qx, a.sx, a.z, a.zp, a.M, a.K, a.xk, a.flags, a.nflags, ps, groups * npc, grid,
                     split ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !split) return e;
  hipLaunchKernelGGL(zsum_kernel, dim3((unsigned)(((int64_t)a.M * a.r32 * 4 + 255) / 256)), dim3(256), 0, st, a.zp,
                     a.z, a.M, a.r32, npc, TH);
  return hipGetLastError();
}

// Two token halves per workgroup halve the L1 bytes but also the number of
// workgroups. MXFP4 quantization is cheap, so that pays from 2048 tokens on;
// the INT4 quantizer's vector work wants every CU, so INT4 takes two halves
// only once 32-token workgroups fill the 256 CUs, and only for long K: at
// K = 3072 one half per workgroup (two workgroups per CU) is the faster up
// to 16384 tokens at least, at K = 12288 two halves are.
constexpr int kTwoHalvesMinM[2] = {8192, 2048};   // INT4, MXFP4
constexpr int kTwoHalvesMinKInt4 = 6144;

template <int FMT>
static hipError_t launch_fmt(const Stage1Args& a, int cus, hipStream_t st) {
  const bool two = FMT == SVDQ_FMT_MXFP4_G32 ? a.M >= kTwoHalvesMinM[1]
                                             : a.M >= kTwoHalvesMinM[0] && a.K >= kTwoHalvesMinKInt4;
  switch (a.r32) {
    case 0: return two ? launch_t<FMT, 0, 2>(a, cus, st) : launch_t<FMT, 0, 1>(a, cus, st);
    case 32: return two ? launch_t<FMT, 2, 2>(a, cus, st) : launch_t<FMT, 2, 1>(a, cus, st);
    case 64: return two ? launch_t<FMT, 4, 2>(a, cus, st) : launch_t<FMT, 4, 1>(a, cus, st);
    case 96: return launch_t<FMT, 6, 1>(a, cus, st);
    case 128: return launch_t<FMT, 8, 1>(a, cus, st);
    default: return hipErrorInvalidValue;
  }
}

template <int FMT, int NCB, int TH>
static hipError_t prepare_t() {
  return hipFuncSetAttribute((const void*)stage1_kernel<FMT, NCB, TH>, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)lds_bytes<FMT, NCB, TH>());
}

template <int FMT>
static hipError_t prepare_fmt() {
  const hipError_t e[8] = {prepare_t<FMT, 0, 1>(), prepare_t<FMT, 2, 1>(), prepare_t<FMT, 4, 1>(),
                           prepare_t<FMT, 6, 1>(), prepare_t<FMT, 8, 1>(), prepare_t<FMT, 0, 2>(),
                           prepare_t<FMT, 2, 2>(), prepare_t<FMT, 4, 2>()};
  for (hipError_t x : e)
    if (x != hipSuccess) return x;
  return hipSuccess;
}

hipError_t prepare_stage1() {
  const hipError_t e = prepare_fmt<SVDQ_FMT_INT4_G64>();
  return e != hipSuccess ? e : prepare_fmt<SVDQ_FMT_MXFP4_G32>();
}

hipError_t launch_stage1(const Stage1Args& a, int num_cus, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  if (a.fmt == SVDQ_FMT_INT4_G64) return launch_fmt<SVDQ_FMT_INT4_G64>(a, num_cus, st);
  return launch_fmt<SVDQ_FMT_MXFP4_G32>(a, num_cus, st);
}

}  // namespace svdq
