// Internal launch interface between the C-ABI glue and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svdq.h"

namespace svdq {

struct Stage1Args {
  int fmt, M, K, r32;
  const uint16_t* x;    // bf16 [M][K]
  const float* mu;      // [K]
  const uint16_t* l1s;  // L1 in stage-1 MFMA order
  // activation codes, scales and Z = X_hat L1 over round32(M) rows: codes
  // and Z in fragment order (the layouts of the weight's qw and l2); scales
  // fp32 [K/64][round16(M)] (INT4) or E8M0 bytes in fragment order (MXFP4)
  uint8_t* qx;
  void* sx;
  uint16_t* z;
  uint32_t* flags;   // INT4 GEMM split flags to clear (nflags of them), or null
  int nflags;
  float* zp;         // partial Z per token group and K piece (see ws_layout)
};
// stage 1; with few token groups its K pieces are dealt over the CUs and a
// second kernel adds the partial Z (num_cus sizes that grid)
hipError_t launch_stage1(const Stage1Args& a, int num_cus, hipStream_t st);
hipError_t prepare_stage1();   // one-time per device: kernels' dynamic LDS attribute

struct GemmArgs {
  int fmt, M, N, K, r32;
  // operands in the layouts of Stage1Args and the packed layer (z and l2t
  // unused when r32 == 0)
  const uint8_t* qx;
  const void* sx;
  const uint16_t* z;
  const uint8_t* qw;
  const void* sw;
  const uint16_t* l2t;
  const uint16_t* bias;  // bf16 [N]
  uint16_t* y;           // bf16 [M][N]
  // INT4 split of the last tiles: per-workgroup flags (cleared by stage 1)
  // and fp32 partial tiles, in the workspace
  uint32_t* flags;
  float* part;
  // group-sum test hook (INT4): window and output [mc][nc][K/64], p ==
  // nullptr for the normal epilogue
  int32_t* p;
  int m0, mc, n0, nc;
};
hipError_t launch_gemm_int4(const GemmArgs& a, int num_cus, hipStream_t st);
// few tokens (INT4: at most 256, or 769 to 1024; MXFP4: at most 256; no
// group-sum hook): the weight-streaming kernel of either format
bool gemm_small_fits(const GemmArgs& a, int num_cus);
hipError_t launch_gemm_small(const GemmArgs& a, int num_cus, hipStream_t st);
hipError_t launch_gemm_mxfp4(const GemmArgs& a, int num_cus, hipStream_t st);
// one-time per device: the kernels' dynamic LDS attribute
hipError_t prepare_gemm_int4();
hipError_t prepare_gemm_mxfp4();

inline hipError_t launch_gemm(const GemmArgs& a, int num_cus, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  if (gemm_small_fits(a, num_cus)) return launch_gemm_small(a, num_cus, st);
  return a.fmt == SVDQ_FMT_MXFP4_G32 ? launch_gemm_mxfp4(a, num_cus, st) : launch_gemm_int4(a, num_cus, st);
}

}  // namespace svdq
