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
  uint8_t* qx;          // [M][K/2]
  void* sx;             // INT4 fp32 [K/64][M]; MXFP4 u8 [M][K/256][2][4]
  uint16_t* z;          // bf16 [M][r32]
};
hipError_t launch_stage1(const Stage1Args& a, hipStream_t st);

struct GemmArgs {
  int fmt, M, N, K, r32;
  const uint8_t* qx;
  const void* sx;
  const uint16_t* z;     // bf16 [M][r32] (unused when r32 == 0)
  const uint8_t* qw;     // [N][K/2]
  const void* sw;        // INT4 fp32 [K/64][N]; MXFP4 u8 [N][K/256][2][4]
  const uint16_t* l2t;   // bf16 [N][r32]
  const uint16_t* bias;  // bf16 [N]
  uint16_t* y;           // bf16 [M][N]
  // group-sum test hook (INT4): window and output, p == nullptr for the normal epilogue
  int32_t* p;
  int m0, mc, n0, nc;
};
hipError_t launch_gemm_int4(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_mxfp4(const GemmArgs& a, hipStream_t st);
hipError_t prepare_gemm_mxfp4();   // one-time per device: kernel LDS attribute

inline hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  return a.fmt == SVDQ_FMT_MXFP4_G32 ? launch_gemm_mxfp4(a, st) : launch_gemm_int4(a, st);
}

}  // namespace svdq
