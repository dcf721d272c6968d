// Internal launch interface between the C-ABI glue and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svdq.h"

namespace svdq {

struct Stage1Args {
  int fmt, M, K, r32;   // K: padded to whole 256-channel steps
  int xk;               // the layer's K: X's row stride, and its channels (the rest read as zero)
  const uint16_t* x;    // bf16 [M][xk]
  const float* mu;      // [K]
  const uint16_t* l1s;  // L1 in stage-1 MFMA order
  // activation codes, scales and Z = X_hat L1 over round32(M) rows: codes
  // and Z in fragment order (the layouts of the weight's qw and l2); scales
  // fp32 [K/64][round16(M)] (INT4) or E8M0 bytes in fragment order (MXFP4)
  uint8_t* qx;
  void* sx;
  uint16_t* z;
  uint32_t* flags;   // INT4 GEMM split ticket counters to clear (nflags of them), or null
  int nflags;
  float* zp;         // partial Z per token group and K piece (see ws_layout)
};
// stage 1; with few token groups its K pieces are dealt over the CUs and a
// second kernel adds the partial Z (num_cus sizes that grid)
hipError_t launch_stage1(const Stage1Args& a, int num_cus, hipStream_t st);
hipError_t prepare_stage1();   // one-time per device: kernels' dynamic LDS attribute

struct GemmArgs {
  int fmt, M, N, K, r32;   // N, K: padded (whole 32-row blocks, whole 256-channel steps)
  int ldy;                 // the layer's N: Y's row stride and width (stores past it are dropped)
  int ldk;                 // the layer's K (the group-sum hook's groups)
  // operands in the layouts of Stage1Args and the packed layer (z and l2t
  // unused when r32 == 0)
  const uint8_t* qx;
  const void* sx;
  const uint16_t* z;
  const uint8_t* qw;
  const void* sw;
  const uint16_t* l2t;
  const uint16_t* bias;  // bf16 [N]
  uint16_t* y;           // bf16 [M][ldy]
  // tiled INT4 GEMM: the workspace areas that receive the FP6 copies of qx
  // and qw (the launch fills them before the GEMM; layout in ws_layout)
  uint8_t* qx6;
  uint8_t* qw6;
  // INT4 split of the last tiles: per-tile ticket counters (cleared by
  // stage 1) and fp32 partial tiles, in the workspace
  uint32_t* flags;
  float* part;
  // group-sum test hook (INT4): window and output [mc][nc][K/64], p ==
  // nullptr for the normal epilogue
  int32_t* p;
  int m0, mc, n0, nc;
  // fused next layer (tiled kernels only; nxt_qx == nullptr otherwise):
  // instead of Y, the epilogue writes the next layer's codes and scales (its
  // format, the same as this layer's) of GELU(bf16(Y)) smoothed by nxt_mu
  // (its stage-1 layout, K = this N) and the fp32 partial X_hat L1 of each
  // tile column (256 channels INT4, 384 MXFP4), [N/tile width][M][nxt_r32]
  uint8_t* nxt_qx;
  void* nxt_sx;
  const float* nxt_mu;
  const uint16_t* nxt_l1s;   // next layer's L1 in its stage-1 layout
  float* nxt_zpart;
  int nxt_r32;
};
hipError_t launch_gemm_int4(const GemmArgs& a, int num_cus, hipStream_t st);
// after a fused MLP-up GEMM: Z of the next layer = bf16 of the tile partials
// added in tile order, in fragment order; also clears that layer's split
// counters (its stage 1 does not run)
hipError_t launch_fused_zsum(const float* zpart, int tiles_n, int M, int r32, uint16_t* z, uint32_t* flags,
                             int nflags, hipStream_t st);
// y = GELU(y) in place over n bf16 values (n % 8 == 0): the activation between
// the MLP layers when they are not fused
hipError_t launch_gelu_bf16(uint16_t* y, size_t n, hipStream_t st);
// few tokens (INT4: at most 256, or 769 to 1024; MXFP4: at most 256; no
// group-sum hook): the weight-streaming kernel of either format
bool gemm_small_fits(const GemmArgs& a, int num_cus);
hipError_t launch_gemm_small(const GemmArgs& a, int num_cus, hipStream_t st);
hipError_t launch_gemm_mxfp4(const GemmArgs& a, int num_cus, hipStream_t st);
// one-time per device: the kernels' dynamic LDS attribute
hipError_t prepare_gemm_int4();
hipError_t prepare_gemm_mxfp4();

// The AWQ-style W4A16 linear (layouts in svdq.h): y [M][N] bf16.
struct AwqArgs {
  int M, K, N;
  const uint16_t* x;       // bf16 [M][K]
  const float* inv_s;      // [K]
  const uint8_t* qw;       // [N/16][K/128][64][16]
  const float* scales;     // [N/16][K/128][16]
  const uint8_t* zeros;    // [N/16][K/128][16]
  const uint16_t* bias;    // bf16 [N]
  uint16_t* y;
};
hipError_t launch_awq(const AwqArgs& a, int num_cus, hipStream_t st);
hipError_t prepare_awq();

// measured ceilings of the part (not part of the layer): an MFMA-only loop
// (kind 0 scaled FP4, 1 i8, 2 bf16; *flops = its flop count) and a device copy
hipError_t launch_mfma_peak(int kind, int constant, int iters, int grid, float* sink, hipStream_t st, double* flops);
hipError_t launch_copy(const void* src, void* dst, size_t bytes, int num_cus, hipStream_t st);

inline hipError_t launch_gemm(const GemmArgs& a, int num_cus, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  if (gemm_small_fits(a, num_cus)) return launch_gemm_small(a, num_cus, st);
  return a.fmt == SVDQ_FMT_MXFP4_G32 ? launch_gemm_mxfp4(a, num_cus, st) : launch_gemm_int4(a, num_cus, st);
}

}  // namespace svdq
