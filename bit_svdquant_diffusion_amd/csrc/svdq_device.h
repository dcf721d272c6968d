// Device-side helpers for the gfx950 kernels of libsvdq: operand vector types,
// bf16 conversion, the exact INT4 and E2M1 quantizers, MFMA wrappers.
// gfx950 wave64; MFMA operand/result lane layouts used by the kernels:
//   32x32 result (16 regs): lane l, reg i -> row 8(i/4) + 4(l/32) + i%4, col l%32
//   16x16 result (4 regs):  lane l, reg i -> row 4(l/16) + i,           col l%16
//   A operand: lane l holds row l%32 (32x32) or l%16 (16x16) and a contiguous
//   run of K; B operand symmetric with columns. Only the pairing of A and B
//   runs matters for the product, and both sides are always packed the same.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) int i32x16;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(32))) float f32x32;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f2bf(lo) | (f2bf(hi) << 16);
}

// Exact INT4 code of x_hat for a group with scale s = fl32(amax/7) > 0: round
// half to even of the exact quotient x_hat/s, clamped to [-7, 7]. The code is
// counted from the signs of |x_hat| - (k + 1/2) s, each an exactly-signed
// fused multiply-add (the product (k + 1/2) s is exact inside it). Used when a
// rounded quotient lies too close to a half-integer to be trusted.
__device__ __forceinline__ int q_int4_slow(float xh, float s) {
  float a = fabsf(xh);
  int q = 0;
#pragma unroll 1
  for (int k = 0; k < 7; ++k) {
    float d = __builtin_fmaf(-((float)k + 0.5f), s, a);
    if (d > 0.f) {
      q = k + 1;
    } else {
      if (d == 0.f) q = (k & 1) ? k + 1 : k;   // tie: the even neighbour
      break;
    }
  }
  return xh < 0.f ? -q : q;
}

// E2M1 code (sign | e1 e0 | m) of an already scaled value v, round to nearest
// with ties to the even mantissa bit, saturating at 6. The grid spacing is
// 1/2 below 2, 1 in [2, 4) and 2 from 4 on: with r = [|v| >= 2] + [|v| >= 4],
// q = rint(|v| 2^(1-r)) (an exact product, then round half to even) counts
// grid steps inside range r, and the code is q + 2r, saturated at 7.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = __builtin_fabsf(v);
  const int r = (int)(a >= 2.0f) + (int)(a >= 4.0f);
  const float step_inv = __uint_as_float((uint32_t)(128 - r) << 23);   // 2^(1-r)
  const uint32_t c = (uint32_t)__builtin_rintf(a * step_inv) + 2u * (uint32_t)r;
  return (c < 7u ? c : 7u) | ((__float_as_uint(v) >> 28) & 8u);
}

// OCP MX shared exponent for E2M1: floor(log2 amax) - 2 clamped to [-127, 127]
// (amax == 0 or subnormal -> -127). Returns e; the scale byte is e + 127.
__device__ __forceinline__ int mx_exponent(float amax) {
  uint32_t eb = (__float_as_uint(amax) >> 23) & 0xffu;
  int e = (int)eb - 127 - 2;
  if (eb == 0) e = -127;
  return e < -127 ? -127 : e;
}
// 2^-e as a float for e in [-127, 125].
__device__ __forceinline__ float exp2_neg(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

}  // namespace svdq
