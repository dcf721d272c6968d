// Kernel (2) for layers with few tokens: INT4 with M <= 256 and with 769
// to 1024 tokens (unless the channel blocks overfill one round of CUs), MXFP4
// with M <= 256. The same sums as the tiled kernels of each format
// (aiflownews.com, "What SVDQuant actually does": the two-branch computation;
// "Nunchaku: the inference engine...": the branches share the output write):
// - INT4: per 64-channel group the exact int32 sum P of code products,
//   dequantized by s_w[n] s_x[m] and accumulated in fp32 in group order;
// - MXFP4: per 32-channel block the E2M1 products scaled by both E8M0 scales
//   inside the block-scaled MFMA, accumulated in fp32 in K order;
// then (X_hat L1) L2 and the bias before the bf16 write of Y.
//
// With few tokens the layer's bytes are mostly the 4-bit weights (pages:
// inference is memory-bound), so every CU streams its own slice of them
// once, straight into registers: a workgroup owns one 32-channel block of W
// and a K share (the shares of a block leave fp32 partials that a second
// kernel adds in order). Its waves split K or, with four token blocks or
// more, the tokens. The activation codes are small and come from L2.
//
// INT4, per 64-channel group and 32-token block: two v_mfma_i32_32x32x32_i8
// on nibbles widened to 16 q (even, then odd channels: 256 P exactly) and,
// per two token blocks, one two-block v_mfma_f32_32x32x1f32 for the scale
// outer product s_w[n] * s_x[m]; the 1/256 is applied once at the end.
// MXFP4, per 128-channel stage and 32-token block: two
// v_mfma_scale_f32_32x32x64_f8f6f4 (its two 64-channel steps).
#include "svdq_device.h"
#include "svdq_internal.h"
#include "svdq_layout.h"

namespace svdq {

namespace {

// int8 operands of one 32-channel half of a group: 16*q of the even channels
// (lo) and of the odd channels (hi) of a 16-byte fragment
__device__ __forceinline__ void sm_widen(const i32x4& w, i32x4& lo, i32x4& hi) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    lo[d] = (int)(((uint32_t)w[d] << 4) & 0xF0F0F0F0u);
    hi[d] = (int)((uint32_t)w[d] & 0xF0F0F0F0u);
  }
}

// Accumulator lane layout (32 x 32 block, channels as rows, tokens as
// columns): lane l, register e -> channel 8 (e / 4) + 4 (l / 32) + e % 4,
// token l % 32. bf16 out: after the lane-half swap of the packed pairs
// (q = 1, h = 0) <-> (q = 0, h = 1) and (q = 3, h = 0) <-> (q = 2, h = 1),
// lane h holds channels 8 h + (0..7) and 16 + 8 h + (0..7) of its token.
// Y has ldy channels per row; 8-channel runs past them are not stored.
__device__ __forceinline__ void sm_store_block(const f32x16& v, uint16_t* y, int M, int ldy, int n0, int m, int h) {
  uint32_t o[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) o[p] = cvt_bf16x2(v[2 * p], v[2 * p + 1]);
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const auto r = __builtin_amdgcn_permlane32_swap(o[4 * p + w], o[4 * p + 2 + w], false, false);
      o[4 * p + w] = r[0];
      o[4 * p + 2 + w] = r[1];
    }
  }
  if (m < M) {
    u32x4* dst = reinterpret_cast<u32x4*>(y + (size_t)m * ldy + n0 + 8 * h);
    if (n0 + 8 * h < ldy) dst[0] = u32x4{o[0], o[1], o[2], o[3]};
    if (n0 + 16 + 8 * h < ldy) dst[2] = u32x4{o[4], o[5], o[6], o[7]};
  }
}
}  // namespace

// Workgroup b: channel block nb = b / splits, K share sp = b % splits. The
// NW waves form TT token parts by NW / TT K parts: wave w takes the token
// blocks w % TT, w % TT + TT, ... and the K units [g0, g1) of K part w / TT
// (a unit: an INT4 group of 64 channels, an MXFP4 stage of 128).
// MB is the most token blocks the instance serves; the layer has
// mb = ceil(M / 32) of them. part (splits > 1): sums [sp][token block][channel
// block][64 lanes][16].
// DEBUG_P (INT4 only): the same loads, widening and i8 MFMAs, but each group's
// exact sum P = (256 P) / 256 of the outputs inside the window [m0, m0 + mc)
// x [n0, n0 + nc) is written to a.p ([mc][nc][K/64] int32) instead of being
// dequantized; no epilogue.
template <int FMT, int MB, int TT, int PD, int NW, bool DEBUG_P>
__global__ __launch_bounds__(64 * NW) void gemm_small_kernel(GemmArgs a, int splits, float* part) {
  constexpr bool FP4 = FMT == SVDQ_FMT_MXFP4_G32;
  constexpr int FPU = FP4 ? 2 : 1;          // 64-channel fragments per K unit
  constexpr int KK = NW / TT;               // waves along K
  constexpr int MBW = (MB + TT - 1) / TT;   // token blocks per wave
  constexpr int NP = (MBW + 1) / 2;         // INT4: two-block scale products per group
  constexpr int NX = FP4 ? MBW : NP;        // activation scale registers per unit
  __shared__ __align__(16) float red[KK][KK > 1 ? MB : 1][16][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ti = wave % TT, ki = wave / TT;
  const int h = lane >> 5, lr = lane & 31;
  const int KS = a.K / 64, KU = KS / FPU, N = a.N, NB = N / 32;
  const int nb = blockIdx.x / splits, sp = blockIdx.x - nb * splits;
  const int s0 = (int)((int64_t)KU * sp / splits), s1 = (int)((int64_t)KU * (sp + 1) / splits);
  const int g0 = s0 + (s1 - s0) * ki / KK, g1 = s0 + (s1 - s0) * (ki + 1) / KK;
  const int act_rows = (a.M + 15) / 16 * 16;   // row stride of s_x
  const int mb = (a.M + 31) / 32;

  // Sources as buffer resources (no per-load address arithmetic): fragment
  // block (row block b, 64-channel step f) at ((b * KS + f) * 64 + lane) * 16
  // bytes, the unit's offset as the scalar offset. INT4 scales: s_w [K/64][N],
  // s_x [K/64][act_rows] fp32. MXFP4 scales: E8M0 bytes, per 128-channel
  // stage, 32-row block and lane the two steps' bytes (s_w [K/128][N/32][64],
  // s_x [K/128][mb][64]). Token blocks past the layer's and rows past M are
  // clamped to the last ones (their results are dropped).
  const __amdgpu_buffer_rsrc_t rqw =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.qw + (size_t)nb * KS * 1024), 0, KS * 1024, 0x00020000);
  const __amdgpu_buffer_rsrc_t rqx = __builtin_amdgcn_make_buffer_rsrc((void*)a.qx, 0, mb * KS * 1024, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsw =
      FP4 ? __builtin_amdgcn_make_buffer_rsrc((void*)a.sw, 0, KU * NB * 128, 0x00020000)
          : __builtin_amdgcn_make_buffer_rsrc((void*)((const float*)a.sw + nb * 32), 0, (KS - 1) * N * 4 + 128, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.sx, 0, FP4 ? KU * mb * 128 : KS * act_rows * 4, 0x00020000);
  auto blk = [&](int j) { return min(ti + TT * min(j, MBW - 1), mb - 1); };   // the wave's j-th token block
  // lane offsets of the activation scales: INT4, the lane's token row in
  // pair p's block (lanes 32 h + r: block 2 p + h); MXFP4, block j's bytes
  int sxo[NX];
#pragma unroll
  for (int p = 0; p < NX; ++p)
    sxo[p] = FP4 ? (blk(p) * 64 + lane) * 2 : min(blk(2 * p + h) * 32 + lr, a.M - 1) * 4;

  f32x16 acc[MBW];
#pragma unroll
  for (int j = 0; j < MBW; ++j) acc[j] = f32x16{};

  // The epilogue's operands (the first two 16-column steps of Z and L2^T,
  // the bias) do not depend on the main loop. When a wave finishes at most
  // two blocks they are loaded before it, so their latency hides under it.
  constexpr int FB = KK == 1 ? MBW : (MB + NW - 1) / NW;   // blocks this wave finishes
  constexpr bool PRE = FB <= 2;
  const int r32 = a.r32, nlr = r32 / 16;
  const i32x4* lf = reinterpret_cast<const i32x4*>(a.l2t) + (size_t)nb * nlr * 64 + lane;
  // the wave's i-th finished block (not past the last one)
  auto fin_block = [&](int i) { return min(KK == 1 ? ti + TT * i : wave + NW * i, mb - 1); };
  i32x4 zpre[PRE ? FB : 1][2], lpre[2];
  u32x2 bpre[4];
  if (PRE && sp == 0) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
      if (st < nlr) lpre[st] = lf[st * 64];
#pragma unroll
    for (int i = 0; i < (PRE ? FB : 1); ++i) {
      const i32x4* zf = reinterpret_cast<const i32x4*>(a.z) + (size_t)fin_block(i) * nlr * 64 + lane;
#pragma unroll
      for (int st = 0; st < 2; ++st)
        if (st < nlr) zpre[i][st] = zf[st * 64];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) bpre[q] = *reinterpret_cast<const u32x2*>(a.bias + nb * 32 + 8 * q + 4 * h);
  }

  // PD + 1 units of operands in registers, loads running PD units ahead.
  // No arithmetic touches a loaded value before its unit's turn (a scale
  // multiply at the load would make the wave wait for the load it has just
  // issued): the 1/256 of the widened INT4 codes is applied once at the end,
  // which is exact (a power of two) for these normal-range sums.
  i32x4 fb[PD + 1][FPU], fa[PD + 1][MBW][FPU];
  uint32_t fw[PD + 1], fx[PD + 1][NX];   // scales: fp32 bits (INT4) or two E8M0 bytes (MXFP4)
  auto load = [&](int slot, int g) {
    const int gg = min(g, g1 - 1);   // past the end: repeat the last unit (not multiplied)
#pragma unroll
    for (int f = 0; f < FPU; ++f)
      fb[slot][f] =
          __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rqw, lane * 16, (gg * FPU + f) * 1024, 0));
#pragma unroll
    for (int j = 0; j < MBW; ++j)
#pragma unroll
      for (int f = 0; f < FPU; ++f)
        fa[slot][j][f] = __builtin_bit_cast(
            i32x4, __builtin_amdgcn_raw_buffer_load_b128(rqx, lane * 16, (blk(j) * KS + gg * FPU + f) * 1024, 0));
    if constexpr (FP4) {
      fw[slot] = __builtin_amdgcn_raw_buffer_load_b16(rsw, lane * 2, (gg * NB + nb) * 128, 0);
#pragma unroll
      for (int j = 0; j < MBW; ++j) fx[slot][j] = __builtin_amdgcn_raw_buffer_load_b16(rsx, sxo[j], gg * mb * 128, 0);
    } else {
      fw[slot] = __builtin_amdgcn_raw_buffer_load_b32(rsw, lr * 4, gg * N * 4, 0);
#pragma unroll
      for (int p = 0; p < NP; ++p) fx[slot][p] = __builtin_amdgcn_raw_buffer_load_b32(rsx, sxo[p], gg * act_rows * 4, 0);
    }
  };
  // unit u of the ring holds K unit (group) grp
  auto mult = [&](int u, int grp) {
    if constexpr (FP4) {
      // weight fragment as operand A (channels as rows), the scale bytes of
      // step f selected by opsel f
#pragma unroll
      for (int j = 0; j < MBW; ++j) {
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            i32x8{fb[u][0][0], fb[u][0][1], fb[u][0][2], fb[u][0][3], 0, 0, 0, 0},
            i32x8{fa[u][j][0][0], fa[u][j][0][1], fa[u][j][0][2], fa[u][j][0][3], 0, 0, 0, 0}, acc[j], 4, 4, 0,
            (int)fw[u], 0, (int)fx[u][j]);
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            i32x8{fb[u][1][0], fb[u][1][1], fb[u][1][2], fb[u][1][3], 0, 0, 0, 0},
            i32x8{fa[u][j][1][0], fa[u][j][1][1], fa[u][j][1][2], fa[u][j][1][3], 0, 0, 0, 0}, acc[j], 4, 4, 1,
            (int)fw[u], 1, (int)fx[u][j]);
      }
    } else {
      i32x4 blo, bhi;
      sm_widen(fb[u][0], blo, bhi);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        // lanes 32 h + r: the channel scales times the token scales of the
        // pair's block 2 p + h; output block 2 p + bb in registers 16 bb .. + 15
        const f32x32 r = __builtin_amdgcn_mfma_f32_32x32x1f32(__builtin_bit_cast(float, fw[u]),
                                                             __builtin_bit_cast(float, fx[u][p]), f32x32{}, 0, 0, 0);
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const int j = 2 * p + bb;
          if (j < MBW) {
            i32x4 alo, ahi;
            sm_widen(fa[u][j][0], alo, ahi);
            i32x16 pp = __builtin_amdgcn_mfma_i32_32x32x32_i8(blo, alo, i32x16{}, 0, 0, 0);
            pp = __builtin_amdgcn_mfma_i32_32x32x32_i8(bhi, ahi, pp, 0, 0, 0);
            if constexpr (DEBUG_P) {
              // token (ti + TT j) 32 + lr, channel nb 32 + 8 (e / 4) + 4 h + e % 4;
              // surplus parts (a clamped, repeated block) write nothing
              const int tok = (ti + TT * j) * 32 + lr;
              if (ti + TT * j < mb && tok >= a.m0 && tok < a.m0 + a.mc && tok < a.M) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                  const int ch = nb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                  if (ch >= a.n0 && ch < a.n0 + a.nc && grp < a.ldk / 64)
                    a.p[((size_t)(tok - a.m0) * a.nc + (ch - a.n0)) * (a.ldk / 64) + grp] = pp[e] / 256;
                }
              }
            } else {
#pragma unroll
              for (int e = 0; e < 16; ++e) acc[j][e] = __builtin_fmaf((float)pp[e], r[16 * bb + e], acc[j][e]);
            }
          }
        }
      }
    }
  };
  const int n = g1 - g0;
  if (n > 0) {
    // the prologue's loads stay in slot order (scheduling barriers), so each
    // slot's wait counts the same in the first round as in later ones
#pragma unroll
    for (int d = 0; d < PD; ++d) {
      load(d, g0 + d);
      __builtin_amdgcn_sched_barrier(0);
    }
    // whole rounds: slot u holds group g + u; each step refills the slot
    // used last with the group PD later
    const int rounds = n / (PD + 1);
    int g = g0;
    for (int it = 0; it < rounds; ++it, g += PD + 1) {
#pragma unroll
      for (int u = 0; u <= PD; ++u) {
        load((u + PD) % (PD + 1), g + u + PD);
        mult(u, g + u);
        __builtin_amdgcn_sched_barrier(0);   // keep each step's loads at its start
      }
    }
    // the remaining groups already sit in slots 0 .. rem - 1
    const int rem = n - rounds * (PD + 1);
#pragma unroll
    for (int u = 0; u < PD; ++u)
      if (u < rem) mult(u, g + u);
  }
  if constexpr (DEBUG_P) return;

  // block b, the wave's i-th finished block
  auto finish = [&](int b, int i, f32x16 v) {
    if constexpr (!FP4) {
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] *= 1.0f / 256.0f;
    }
    if (sp == 0) {
      // + (X_hat L1) L2 on bf16 MFMA (Z and L2^T in 16-column fragment order) + bias
      const i32x4* zf = reinterpret_cast<const i32x4*>(a.z) + (size_t)b * nlr * 64 + lane;
      int st = 0;
      if constexpr (PRE) {
#pragma unroll
        for (; st < 2; ++st)
          if (st < nlr)
            v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, lpre[st]),
                                                        __builtin_bit_cast(bf16x8, zpre[i][st]), v, 0, 0, 0);
      }
      for (; st < nlr; ++st)
        v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, lf[st * 64]),
                                                    __builtin_bit_cast(bf16x8, zf[st * 64]), v, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 bw = PRE ? bpre[q] : *reinterpret_cast<const u32x2*>(a.bias + nb * 32 + 8 * q + 4 * h);
        v[4 * q + 0] += bf16lo(bw.x);
        v[4 * q + 1] += bf16hi(bw.x);
        v[4 * q + 2] += bf16lo(bw.y);
        v[4 * q + 3] += bf16hi(bw.y);
      }
    }
    if (splits == 1) {
      sm_store_block(v, a.y, a.M, a.ldy, nb * 32, b * 32 + lr, h);
    } else {
      f32x4* dst = reinterpret_cast<f32x4*>(part) + ((((size_t)sp * mb + b) * NB + nb) * 64 + lane) * 4;
#pragma unroll
      for (int c = 0; c < 4; ++c) dst[c] = f32x4{v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]};
    }
  };
  if constexpr (KK == 1) {
#pragma unroll
    for (int j = 0; j < MBW; ++j)
      if (ti + TT * j < mb) finish(ti + TT * j, j, acc[j]);
  } else {
    // the K parts' sums, added in K-part order
#pragma unroll
    for (int j = 0; j < MBW; ++j) {
      const int b = ti + TT * j;
      if (b < mb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) red[ki][b][e][lane] = acc[j][e];
      }
    }
    __syncthreads();
    for (int b = wave, i = 0; b < mb; b += NW, ++i) {
      f32x16 v;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < KK; ++k) s += red[k][b][e][lane];
        v[e] = s;
      }
      finish(b, i, v);
    }
  }
}

// Y = bf16 of the K shares' partials added in share order; one wave per
// (token block, channel block).
__global__ __launch_bounds__(64) void gemm_small_sum(const float* __restrict__ part, uint16_t* __restrict__ y,
                                                        int M, int N, int ldy, int MB, int splits) {
  const int lane = threadIdx.x, h = lane >> 5, lr = lane & 31;
  const int NB = N / 32, b = blockIdx.x / NB, nb = blockIdx.x - b * NB;
  f32x16 v = f32x16{};
  for (int sp = 0; sp < splits; ++sp) {
    const f32x4* src = reinterpret_cast<const f32x4*>(part) + ((((size_t)sp * MB + b) * NB + nb) * 64 + lane) * 4;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 w = src[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * c + e] = sp == 0 ? w[e] : v[4 * c + e] + w[e];
    }
  }
  sm_store_block(v, y, M, ldy, nb * 32, b * 32 + lr, h);
}

bool gemm_small_fits(const GemmArgs& a, int num_cus) {
  if (a.M <= kFewTokens) return true;
  if (a.fmt != SVDQ_FMT_INT4_G64 || a.M <= 768 || a.M > 1024) return false;
  // 769 to 1024 INT4 tokens run one eight-wave workgroup per CU at a time:
  // a little over one round of channel blocks would leave most CUs idle in
  // the second round, and the tiled kernel does better there
  const int cus = num_cus > 0 ? num_cus : 256, NB = a.N / 32;
  return !(NB > cus && 4 * NB <= 5 * cus);
}

// Shape of the launch for MB token blocks: token parts TT, ring depth PD.
// With one or two token blocks the waves split K; from four blocks on they
// split the tokens, each wave then holding two blocks' sums. The INT4 kernel
// is bound by the dequant's vector instructions rather than by the weight
// stream, so the launch aims at busy SIMDs: eight waves per workgroup when
// the channel blocks cannot fill half the CUs, and K shares (with an fp32
// partial pass) only while CUs would otherwise idle and each wave keeps 512
// channels or more.
template <int FMT, int MB, int TT, int PD, int NW, bool DBG>
static hipError_t launch_nw(const GemmArgs& a, int num_cus, hipStream_t st) {
  constexpr int KK = NW / TT, FPU = FMT == SVDQ_FMT_MXFP4_G32 ? 2 : 1;
  const int KU = a.K / 64 / FPU, NB = a.N / 32;
  const int cus = num_cus > 0 ? num_cus : 256;
  int splits = 1;
  while ((splits + 1) * NB <= cus && KU / (KK * (splits + 1)) >= 8 / FPU) ++splits;
  const int mb = (a.M + 31) / 32;
  const size_t per_split = (size_t)mb * 32 * a.N * 4;   // fp32 partial bytes of one share
  while (splits > 1 && (size_t)splits * per_split > kPartAreaBytes) --splits;
  if (a.part == nullptr) splits = 1;   // no partial area: whole K per workgroup
  hipLaunchKernelGGL((gemm_small_kernel<FMT, MB, TT, PD, NW, DBG>), dim3(NB * splits), dim3(64 * NW), 0, st, a,
                     splits, a.part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1 || DBG) return e;
  hipLaunchKernelGGL(gemm_small_sum, dim3(mb * NB), dim3(64), 0, st, a.part, a.y, a.M, a.N, a.ldy, mb, splits);
  return hipGetLastError();
}

template <int FMT, int MB, int TT, bool DBG>
static hipError_t launch_shape(const GemmArgs& a, int num_cus, hipStream_t st) {
  const int cus = num_cus > 0 ? num_cus : 256;
  return 2 * (a.N / 32) <= cus ? launch_nw<FMT, MB, TT, 2, 8, DBG>(a, num_cus, st)
                               : launch_nw<FMT, MB, TT, 2, 4, DBG>(a, num_cus, st);
}

template <int FMT, bool DBG>
static hipError_t launch_fmt(const GemmArgs& a, int num_cus, hipStream_t st) {
  switch ((a.M + 31) / 32) {   // exact token blocks: no read past the round32(M) rows
    case 1: return launch_shape<FMT, 1, 1, DBG>(a, num_cus, st);
    case 2: return launch_shape<FMT, 2, 1, DBG>(a, num_cus, st);
    case 3: return launch_shape<FMT, 3, 1, DBG>(a, num_cus, st);
    case 4: return launch_shape<FMT, 4, 2, DBG>(a, num_cus, st);
    case 5: return launch_shape<FMT, 5, 4, DBG>(a, num_cus, st);
    case 6: return launch_shape<FMT, 6, 4, DBG>(a, num_cus, st);
    case 7: return launch_shape<FMT, 7, 4, DBG>(a, num_cus, st);
    default: return launch_shape<FMT, 8, 4, DBG>(a, num_cus, st);
  }
}

template <bool DBG>
static hipError_t launch_int4(const GemmArgs& a, int num_cus, hipStream_t st) {
  // 769 to 1024 INT4 tokens: eight token parts of four blocks each (the last
  // parts' surplus blocks repeat the last block and are dropped)
  if (a.M > 256) return launch_nw<SVDQ_FMT_INT4_G64, 32, 8, 2, 8, DBG>(a, num_cus, st);
  return launch_fmt<SVDQ_FMT_INT4_G64, DBG>(a, num_cus, st);
}

hipError_t launch_gemm_small(const GemmArgs& a, int num_cus, hipStream_t st) {
  if (a.fmt == SVDQ_FMT_MXFP4_G32) return launch_fmt<SVDQ_FMT_MXFP4_G32, false>(a, num_cus, st);
  // the group-sum hook runs the forward's own launch shape with DEBUG_P
  return a.p != nullptr ? launch_int4<true>(a, num_cus, st) : launch_int4<false>(a, num_cus, st);
}

}  // namespace svdq
