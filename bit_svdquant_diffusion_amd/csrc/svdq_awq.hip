// The AWQ-style W4A16 linear on the GPU: 4-bit weights with a scale and a
// zero point per 128 input channels, 16-bit activations (aiflownews.com, "How
// Nunchaku four bit quantization actually works": the adaptive-normalization
// and modulation layers). Its inputs are a few conditioning rows, so the
// layer is a GEMV over 4-bit weights and its time is the weight stream.
//
// y[m,n] = b[n] + sum_g scale[n,g] sum_{k in g} x_hat[m,k] (q[n,k] - zero[n,g]),
// x_hat = fl32(x inv_s) rounded to bf16 for the matrix unit. Per group the
// inner sum runs on v_mfma_f32_16x16x32_bf16 as
//   P = sum_k x_hat[m,k] (128 + q[n,k])   (128 + q is exact in bf16, and its
//       bits come from the nibble with one and-or: 0x4300 | q)
// and the zero point is taken out once per output and group:
//   y += scale (P - (128 + zero) S),  S = sum_k x_hat[m,k] (per token and group).
// So a weight costs under one vector instruction to unpack (seven per eight
// nibbles) and the matrix unit does the multiply-adds.
//
// A workgroup of eight waves covers NB n-blocks of 16 output channels; the
// waves of one n-block split its groups (K parts) and add their sums in
// K-part order through LDS. Tokens go in chunks of up to 16 (the MFMA's
// rows): the chunk's live rows of x_hat (bf16, rows padded by 8 channels
// against LDS bank conflicts) and their S sit in LDS, so with a couple of
// rows the LDS is small and several workgroups share a CU; MFMA rows past
// the chunk repeat a staged row, and their outputs are never stored. Each
// wave keeps six groups of weights in
// flight (16-byte loads, 1 KiB per n-block and group), the first ones issued
// before the staging.
#include "svdq_device.h"
#include "svdq_internal.h"

#include <algorithm>

namespace svdq {

namespace {
constexpr int kAwqWaves = 8;
constexpr int kAwqRing = 6;     // groups of weights in flight per wave
constexpr int kAwqPadK = 8;     // bf16 padding of an x_hat row in LDS
}  // namespace

// rows: x_hat rows staged at once (min(16, M))
size_t awq_lds_bytes(int K, int rows) {
  return (size_t)rows * (K + kAwqPadK) * 2 + (size_t)(K / 128) * 16 * 4 + (size_t)kAwqWaves * 4 * 64 * 4;
}

// NB >= 4 runs when the staged rows hold one workgroup per CU: two waves per
// SIMD, so it takes their registers and stages six items per thread at a
// time; the others keep four waves per SIMD and stage one at a time.
template <int NB>
__global__ __launch_bounds__(64 * kAwqWaves) __attribute__((amdgpu_waves_per_eu(NB >= 4 ? 2 : 4))) void awq_kernel(AwqArgs a) {
  constexpr int KP = kAwqWaves / NB;   // waves (K parts) per n-block
  static_assert(KP == 1 || KP == 2 || KP == 4 || KP == 8, "eight parts split evenly over the K parts");
  constexpr int kAwqStage = NB >= 4 ? 6 : 1;   // staging items per thread with their loads in flight together
  extern __shared__ __align__(16) uint8_t smem[];
  const int K = a.K, G = K / 128, ldx = K + kAwqPadK;
  const int rows = min(16, a.M);   // rows of x_hat staged at once
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                              // [rows][ldx] bf16
  float* sxg = reinterpret_cast<float*>(smem + (size_t)rows * ldx * 2);          // [G][16]
  float* red = sxg + G * 16;                                                     // [waves][4][64]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nbl = wave % NB, kp = wave / NB;
  const int nb = blockIdx.x * NB + nbl;   // this wave's n-block
  const bool live = nb * 16 < a.N;
  const int g0 = G * kp / KP, g1 = G * (kp + 1) / KP;
  const int r = lane & 15, c = lane >> 4;
  const i32x4* wsrc = reinterpret_cast<const i32x4*>(a.qw) + ((size_t)min(nb, a.N / 16 - 1) * G) * 64 + lane;
  const float* ssrc = a.scales + (size_t)min(nb, a.N / 16 - 1) * G * 16 + r;
  const uint8_t* zsrc = a.zeros + (size_t)min(nb, a.N / 16 - 1) * G * 16 + r;

  // a ring of kAwqRing groups of weights (and their scales and zero points),
  // each slot refilled with the group kAwqRing later as soon as it is used
  i32x4 wq[kAwqRing];
  float sc[kAwqRing];
  uint32_t zp[kAwqRing];
  auto load = [&](int u, int g) {
    g = min(g, g1 - 1);   // past the part's end: repeat its last group (not used)
    wq[u] = wsrc[(size_t)g * 64];
    sc[u] = ssrc[g * 16];
    zp[u] = zsrc[g * 16];
  };
  for (int t0 = 0; t0 < a.M; t0 += 16) {
    const int rc = min(16, a.M - t0);   // live rows of this chunk
    if (t0 > 0) __syncthreads();         // the last chunk's LDS reads are done
    // the first weights do not depend on x_hat: in flight during the staging
    if (g0 < g1) {
#pragma unroll
      for (int u = 0; u < kAwqRing; ++u) load(u, g0 + u);
    }
    // x_hat of the live rows, eight channels a thread; the sixteen threads of
    // a 128-channel group (consecutive lanes) then add their partial sums of
    // the bf16 values in a fixed butterfly order into S. With many rows
    // (NB >= 4) a thread's items go in batches of kAwqStage whose loads are
    // all issued before any is used, so a batch costs one memory round trip.
    const int items = rc * (K / 8);
    auto stage_item = [&](int i, bool in, const u32x4& xv, const f32x4& s0, const f32x4& s1) {
      const int t = in ? i / (K / 8) : 0, k = in ? (i - t * (K / 8)) * 8 : 0;
      float part = 0.f;
      if (in) {
        u32x4 o;
        o[0] = cvt_bf16x2(bf16lo(xv[0]) * s0[0], bf16hi(xv[0]) * s0[1]);
        o[1] = cvt_bf16x2(bf16lo(xv[1]) * s0[2], bf16hi(xv[1]) * s0[3]);
        o[2] = cvt_bf16x2(bf16lo(xv[2]) * s1[0], bf16hi(xv[2]) * s1[1]);
        o[3] = cvt_bf16x2(bf16lo(xv[3]) * s1[2], bf16hi(xv[3]) * s1[3]);
        *reinterpret_cast<u32x4*>(xs + (size_t)t * ldx + k) = o;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          part += bf16lo(o[d]);
          part += bf16hi(o[d]);
        }
      }
      // i and the group's first thread are multiples of 16 apart: a group's
      // sixteen threads are lanes 16 j .. 16 j + 15 of one wave
      part += __shfl_xor(part, 8, 16);
      part += __shfl_xor(part, 4, 16);
      part += __shfl_xor(part, 2, 16);
      part += __shfl_xor(part, 1, 16);
      if (in && (i & 15) == 0) sxg[(k / 128) * 16 + t] = part;
    };
    auto item_src = [&](int i, int& t, int& k) {
      t = i < items ? i / (K / 8) : 0;
      k = i < items ? (i - t * (K / 8)) * 8 : 0;
    };
    if constexpr (kAwqStage == 1) {
      for (int i0 = 0; i0 < items; i0 += 64 * kAwqWaves) {
        const int i = i0 + tid;
        const bool in = i < items;
        const int t = in ? i / (K / 8) : 0, k = in ? (i - t * (K / 8)) * 8 : 0;
        float part = 0.f;
        if (in) {
          const u32x4 xv = *reinterpret_cast<const u32x4*>(a.x + (size_t)(t0 + t) * K + k);
          const f32x4 s0 = *reinterpret_cast<const f32x4*>(a.inv_s + k);
          const f32x4 s1 = *reinterpret_cast<const f32x4*>(a.inv_s + k + 4);
          u32x4 o;
          o[0] = cvt_bf16x2(bf16lo(xv[0]) * s0[0], bf16hi(xv[0]) * s0[1]);
          o[1] = cvt_bf16x2(bf16lo(xv[1]) * s0[2], bf16hi(xv[1]) * s0[3]);
          o[2] = cvt_bf16x2(bf16lo(xv[2]) * s1[0], bf16hi(xv[2]) * s1[1]);
          o[3] = cvt_bf16x2(bf16lo(xv[3]) * s1[2], bf16hi(xv[3]) * s1[3]);
          *reinterpret_cast<u32x4*>(xs + (size_t)t * ldx + k) = o;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            part += bf16lo(o[d]);
            part += bf16hi(o[d]);
          }
        }
        part += __shfl_xor(part, 8, 16);
        part += __shfl_xor(part, 4, 16);
        part += __shfl_xor(part, 2, 16);
        part += __shfl_xor(part, 1, 16);
        if (in && (i & 15) == 0) sxg[(k / 128) * 16 + t] = part;
      }
    } else {
      for (int i0 = 0; i0 < items; i0 += 64 * kAwqWaves * kAwqStage) {
        u32x4 xv[kAwqStage];
        f32x4 s0[kAwqStage], s1[kAwqStage];
#pragma unroll
        for (int b = 0; b < kAwqStage; ++b) {   // out-of-range items load row 0 (in bounds, unused)
          int t, k;
          item_src(i0 + b * 64 * kAwqWaves + tid, t, k);
          xv[b] = *reinterpret_cast<const u32x4*>(a.x + (size_t)(t0 + t) * K + k);
          s0[b] = *reinterpret_cast<const f32x4*>(a.inv_s + k);
          s1[b] = *reinterpret_cast<const f32x4*>(a.inv_s + k + 4);
        }
#pragma unroll
        for (int b = 0; b < kAwqStage; ++b) {
          const int i = i0 + b * 64 * kAwqWaves + tid;
          stage_item(i, i < items, xv[b], s0[b], s1[b]);
        }
      }
    }
    __syncthreads();

    // The groups fall into eight fixed parts (part q: groups [G q / 8,
    // G (q + 1) / 8)), each summed from zero, and the parts are added as a
    // balanced binary tree: a wave owns 8 / KP whole parts and builds their
    // subtree, the K-part reduction below adds the waves' subtrees as the
    // upper levels. So the sums associate the same way for any KP, and a
    // row's output does not depend on how many rows the launch had. The
    // pending left siblings sit in s0, s1, s2 (four or eight parts, the
    // instances with 256 registers), or, with two parts, the first one in
    // the wave's own slot of the reduction area (registers are short there).
    constexpr int kParts = 8 / KP;   // parts of this wave
    const f32x4 z4 = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 acc = z4, s0 = z4, s1 = z4, s2 = z4;
    float* myred = red + wave * 4 * 64 + lane;   // [e * 64]
    int q = 0;   // parts of this wave finished
    auto part_end = [&](int qq) { return G * (kParts * kp + qq + 1) / 8; };
    const int pe0 = part_end(0);
    auto finish_parts = [&](int gn) {   // close every part that ends at or before group gn
      if constexpr (kParts == 1) {
        return;   // one part: acc is the wave's sum
      } else if constexpr (kParts == 2) {
        if (gn == pe0) {   // the first part ends here: called at g0, then after each group (gn > g0), so once
#pragma unroll
          for (int e = 0; e < 4; ++e) myred[e * 64] = acc[e];
          acc = z4;
        }
        return;
      }
      while (q < kParts && part_end(q) <= gn) {
        switch (q) {
          case 0: s0 = acc; break;
          case 1: s1 = s0 + acc; break;
          case 2: s0 = acc; break;
          case 3: s1 = s1 + (s0 + acc); break;
          case 4: s0 = acc; break;
          case 5: s2 = s0 + acc; break;
          case 6: s0 = acc; break;
          default: s1 = s1 + (s2 + (s0 + acc)); break;
        }
        acc = z4;
        ++q;
      }
    };
    finish_parts(g0);
    // the group after which the next part closes: the per-group test is one
    // comparison, and the part bookkeeping runs only where a part ends
    int next_end = kParts > 1 && q < kParts ? part_end(q) : 0x7fffffff;
    // A row r of the MFMA feeds only output row r (token r of the chunk):
    // lanes of rows past the chunk read a staged row (the last one, so the
    // read stays inside the staging area) and their outputs are not stored.
    // An unconditional read lets the group's four reads issue together.
    const int arow_off = min(r, rows - 1) * ldx;
    for (int gb = g0; gb < g1; gb += kAwqRing) {
#pragma unroll
      for (int u = 0; u < kAwqRing; ++u) {
        const int g = gb + u;
        if (g < g1) {
          f32x4 p = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            // A: token r, channels 128 g + 32 t + 8 c + (0..7); B: the same
            // channels of output 16 nb + r as bf16 128 + q
            const u32x4 av = *reinterpret_cast<const u32x4*>(xs + arow_off + g * 128 + 32 * t + 8 * c);
            const uint32_t w = (uint32_t)wq[u][t];
            const u32x4 bv = u32x4{(w & 0x000F000Fu) | 0x43004300u, ((w >> 4) & 0x000F000Fu) | 0x43004300u,
                                   ((w >> 8) & 0x000F000Fu) | 0x43004300u, ((w >> 12) & 0x000F000Fu) | 0x43004300u};
            p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv),
                                                        p, 0, 0, 0);
          }
          // lane l holds tokens 4 c + (0..3) of output 16 nb + r (S of rows
          // past the chunk is never written: their sums are not stored)
          const f32x4 s4 = *reinterpret_cast<const f32x4*>(sxg + g * 16 + 4 * c);
          const float zf = 128.f + (float)zp[u], scu = sc[u];
          if (g + kAwqRing < g1) load(u, g + kAwqRing);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(scu, __builtin_fmaf(-zf, s4[e], p[e]), acc[e]);
          if (g + 1 >= next_end) {
            finish_parts(g + 1);
            next_end = q < kParts ? part_end(q) : 0x7fffffff;
          }
        }
      }
    }
    if constexpr (kParts == 2) {
      // the second part ends at g1: its sum is acc
#pragma unroll
      for (int e = 0; e < 4; ++e) s1[e] = myred[e * 64] + acc[e];
    } else {
      finish_parts(g1);   // the last parts, empty ones included
    }
    const f32x4 mine = kParts == 1 ? acc : s1;   // this wave's subtree
    // the waves' subtrees as the tree's upper levels, + bias, bf16 out
#pragma unroll
    for (int e = 0; e < 4; ++e) red[(wave * 4 + e) * 64 + lane] = mine[e];
    __syncthreads();
    if (kp == 0 && live) {
      const int n = nb * 16 + r;
      const float bv = __uint_as_float((uint32_t)a.bias[n] << 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        auto rk = [&](int k2) { return red[((nbl + NB * k2) * 4 + e) * 64 + lane]; };
        float s;
        if constexpr (KP == 1) s = rk(0);
        else if constexpr (KP == 2) s = rk(0) + rk(1);
        else if constexpr (KP == 4) s = (rk(0) + rk(1)) + (rk(2) + rk(3));
        else s = ((rk(0) + rk(1)) + (rk(2) + rk(3))) + ((rk(4) + rk(5)) + (rk(6) + rk(7)));
        const int m = t0 + 4 * c + e;
        if (m < a.M) a.y[(size_t)m * a.N + n] = (uint16_t)f2bf(s + bv);
      }
    }
  }
}

hipError_t prepare_awq() {
  const int most = (int)awq_lds_bytes(4096, 16);
  hipError_t e = hipFuncSetAttribute((const void*)awq_kernel<8>, hipFuncAttributeMaxDynamicSharedMemorySize, most);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)awq_kernel<4>, hipFuncAttributeMaxDynamicSharedMemorySize, most);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)awq_kernel<2>, hipFuncAttributeMaxDynamicSharedMemorySize, most);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void*)awq_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, most);
}

// n-blocks per workgroup. While two workgroups fit a CU (a few rows keep the
// LDS small; two is the register file's limit at four waves per SIMD): one
// n-block up to two per CU, two above. Measured on the FLUX shapes (graph
// replays): 576 n-blocks 9.7 us with one, 8.9 with two; 1152 n-blocks 15.7,
// 13.8 and 15.2 with one, two and four; 384 n-blocks the same with any.
// When the LDS holds one workgroup per CU (16-row chunks), four n-blocks, or
// eight where four would leave workgroups for a second round on the CUs.
hipError_t launch_awq(const AwqArgs& a, int num_cus, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  const int cus = num_cus > 0 ? num_cus : 256, nblk = a.N / 16;
  const size_t lds = awq_lds_bytes(a.K, a.M < 16 ? a.M : 16);
  const bool two_per_cu = 2 * lds <= 160 * 1024;
  if (two_per_cu && nblk <= 2 * cus) {
    hipLaunchKernelGGL(awq_kernel<1>, dim3(nblk), dim3(64 * kAwqWaves), lds, st, a);
  } else if (two_per_cu) {
    hipLaunchKernelGGL(awq_kernel<2>, dim3((nblk + 1) / 2), dim3(64 * kAwqWaves), lds, st, a);
  } else if (nblk <= 4 * cus) {
    hipLaunchKernelGGL(awq_kernel<4>, dim3((nblk + 3) / 4), dim3(64 * kAwqWaves), lds, st, a);
  } else {
    hipLaunchKernelGGL(awq_kernel<8>, dim3((nblk + 7) / 8), dim3(64 * kAwqWaves), lds, st, a);
  }
  return hipGetLastError();
}

}  // namespace svdq
