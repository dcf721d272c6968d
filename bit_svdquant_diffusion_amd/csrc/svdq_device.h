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

// two floats -> packed bf16 (lo in bits 0..15), round to nearest even: one
// v_cvt_pk_bf16_f32
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

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
// counted from the signs of |x_hat| - (k + 1/2) s, each a fused multiply-add
// (the product (k + 1/2) s is exact inside it) whose sign is exact as long as
// a nonzero difference cannot round to zero: the caller brings tiny operands
// into the normal range first.
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

// E2M1 codes of 8 values scaled by 2^-e, value k in nibble k (low nibble
// first): v_cvt_scalef32_pk_fp4_f32 for a normal scale (it divides by 2^e
// exactly, rounds to nearest even and saturates), else the exact
// software encoder. Shared by stage 1 and the GEMM epilogue that quantizes
// the next layer's activations, so both give the same bits.
// Every lane runs the converter (with the smallest normal scale where its
// own would be denormal); only lanes with e = -127 then redo their values in
// software, so the common case has no branch around the converter.
__device__ __forceinline__ uint32_t e2m1x8_codes(const float* v, int e) {
  const float sc = __uint_as_float((uint32_t)((e >= -126 ? e : -126) + 127) << 23);
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], sc, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], sc, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], sc, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], sc, 3);
  if (e < -126) {
    const float sinv = exp2_neg(e);
    w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= e2m1_code(v[i] * sinv) << (4 * i);
  }
  return w;
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// GELU(v) = v Phi(v), Phi the standard normal distribution function, with
// Phi(-|v|) = erfc(|v| / sqrt 2) / 2 from the Chebyshev fit of Numerical
// Recipes (Press et al., function erfcc: erfc(z) ~ t exp(-z^2 + P(t)),
// t = 1 / (1 + z / 2), fractional error below 1.2e-7 for all z >= 0) and
// Phi(|v|) = 1 - Phi(-|v|). Written in base 2 with the constants folded:
// t = 1 / (1 + |v| / (2 sqrt 2)) and Phi(-|v|) = t 2^(P(t) log2(e) - 1 -
// v^2 log2(e) / 2), the coefficients below being those of P times log2(e)
// (the constant one also minus 1). Branch-free: one reciprocal, one exp2 and
// sixteen other operations; every step is written out (no contraction left
// to the compiler), so the fused epilogue and the standalone kernel agree bit
// for bit. The fractional error stays near 1e-7, far below the half ulp of
// the bf16 it is rounded to.
__device__ __forceinline__ float gelu_f32(float v) {
  const float a = __builtin_fabsf(v);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(a, 0.3535533845424652f, 1.0f));
  float p = 0.24651730060577393f;
  p = __builtin_fmaf(p, t, -1.1861149072647095f);
  p = __builtin_fmaf(p, t, 2.147474527359009f);
  p = __builtin_fmaf(p, t, -1.6377531290054321f);
  p = __builtin_fmaf(p, t, 0.40232157707214355f);
  p = __builtin_fmaf(p, t, -0.2687568664550781f);
  p = __builtin_fmaf(p, t, 0.1396300494670868f);
  p = __builtin_fmaf(p, t, 0.5397006273269653f);
  p = __builtin_fmaf(p, t, 1.4427292346954346f);
  p = __builtin_fmaf(p, t, -2.8257482051849365f);
  const float lo = __fmul_rn(t, __builtin_amdgcn_exp2f(__builtin_fmaf(__fmul_rn(a, -0.7213475108146667f), a, p)));
  return __fmul_rn(v, v >= 0.f ? __fsub_rn(1.0f, lo) : lo);
}

// The 16 INT4 codes of one lane's values xh (8 to c0, 8 to c1, low nibble
// first) for a group scale sc = fl32(amax / 7): the round-half-to-even of
// the exact quotient xh / sc, clamped to [-7, 7]; sc == 0 gives zeros. The
// fast path and its exact redo are explained inline. Shared by stage 1 and
// the GEMM epilogue that quantizes the next layer's activations, so both give
// the same bits.
__device__ __forceinline__ void int4_codes16(const float (&xh)[16], float sc, uint32_t& c0, uint32_t& c1) {
  // t = x_hat * rcp(s) is within 2e-6 of the exact quotient (|q| <= 7,
  // rcp within 1 ulp), so rint(t) is the answer unless t lies within
  // 1e-5 of a half-integer. Adding 1.5 * 2^23 rounds t to an integer
  // (nearest, ties to even) held in the low mantissa bits, whose low
  // nibble is the two's complement code.
  constexpr float kRound = 12582912.0f;
  const float inv = __builtin_amdgcn_rcpf(sc);
  float dmax = 0.f;   // largest |t - rint(t)| of the lane
  c0 = 0;
  c1 = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float t0 = xh[e] * inv, t1 = xh[8 + e] * inv;
    const float u0 = t0 + kRound, u1 = t1 + kRound;
    dmax = __builtin_fmaxf(dmax, __builtin_fabsf(t0 - (u0 - kRound)));
    dmax = __builtin_fmaxf(dmax, __builtin_fabsf(t1 - (u1 - kRound)));
    c0 |= (__float_as_uint(u0) & 15u) << (4 * e);
    c1 |= (__float_as_uint(u1) & 15u) << (4 * e);
  }
  if (!(sc >= 0x1p-100f)) {
    // zero and tiny scales (rcp out of range): one comparison per level, on
    // the values and the scale times 2^100 (exact: |x_hat| < 7.5 s). Below
    // about 2^-125 the unscaled |x_hat| - (k + 1/2) s can be 2^-150, which
    // rounds to zero and would read as a tie; scaled, every nonzero
    // difference stays far above the smallest float.
    c0 = 0;
    c1 = 0;
    if (sc > 0.f) {
      const float su = sc * 0x1p100f;
#pragma unroll 1
      for (int e = 0; e < 8; ++e) {
        c0 |= ((uint32_t)q_int4_slow(xh[e] * 0x1p100f, su) & 15u) << (4 * e);
        c1 |= ((uint32_t)q_int4_slow(xh[8 + e] * 0x1p100f, su) & 15u) << (4 * e);
      }
    }
  } else if (dmax > 0.49999f) {
    // a value near a half-integer: redo the lane's values exactly.
    // With k = floor(|t|) the answer is k or k + 1, and the sign of
    // the fused |x_hat| - (k + 1/2) s, the sign of the exact
    // difference, decides: above goes up, below stays, zero is an
    // exact tie and goes to the even one. Where |t| and the exact
    // quotient lie on two sides of an integer n the pair tested is
    // (n - 1, n) or (n, n + 1), whose midpoint is still on the right
    // side of the quotient. k + 1 never passes 7: |x_hat| <= amax <
    // 7.5 s.
    c0 = 0;
    c1 = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float ax = __builtin_fabsf(xh[e]);
      const float k = __builtin_floorf(ax * inv);
      const float d = __builtin_fmaf(-(k + 0.5f), sc, ax);
      const bool up = d > 0.f || (d == 0.f && (__float_as_uint(k + kRound) & 1u));
      const float q = up ? k + 1.f : k;
      const uint32_t code = __float_as_uint(__builtin_copysignf(q, xh[e]) + kRound) & 15u;
      if (e < 8)
        c0 |= code << (4 * e);
      else
        c1 |= code << (4 * (e - 8));
    }
  }
}


}  // namespace svdq
