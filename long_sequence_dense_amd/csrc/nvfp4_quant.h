// NVFP4 block quantization shared by the Q/K prep, the NVFP4 linear
// quantizer and the attention kernel that quantizes Q in its prologue: one
// E4M3 scale per 16 values (nearest to max|y| / 6, ties to even, saturating at
// 448) and E2M1 codes of y / scale (nearest, ties to even, saturating at 6).
//
// Method: "Pika H3 Flex in FastVideo: 7x Faster, and Near Real Time in 4-bit",
// sections "FP4 attention" (E2M1 values, one E4M3 scale per 16 channels, unit
// global scale) and "NVFP4 QAD" (one 8-bit scale per 16 values).
//
// Every float operation here is one IEEE operation with round-to-nearest-even
// in the order written (contraction into fma is switched off in each
// function), so the codes are an exact function of y, whichever translation
// unit includes this file.
#pragma once
#include "device_common.h"

namespace lsd {

constexpr float kHadamardScale = 0x1.6a09e6p-4f;   // RN32(1/sqrt(128)), bits 0x3DB504F3

__device__ __forceinline__ float e4m3_pos(uint32_t j) {            // value of code j, 0 <= j <= 126
#pragma clang fp contract(off)
  const uint32_t e = j >> 3, m = j & 7;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * (1.0f / 512.0f);
}

// Nearest E4M3 code to amax/6 (ties to the even code, saturating at 448).
// Candidate: round r = RN(amax * RN(1/6)) (within a few units in the last
// place of amax/6) to 3 mantissa bits; then settle it exactly against the
// values of max|y| where the nearest scale changes, 6 * (v_{c-1} + v_c) / 2 and
// 6 * (v_c + v_{c+1}) / 2 (at most 7 significant bits: exact in fp32), which
// moves it by at most one.
__device__ __forceinline__ uint32_t e4m3_scale_code(float amax) {
#pragma clang fp contract(off)
  const float r = amax * 0x1.555556p-3f;
  uint32_t c;
  if (!(r < 448.0f)) {
    c = 0x7Eu;
  } else if (r >= 0x1p-6f) {
    const uint32_t u = __float_as_uint(r);
    c = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - (120u << 3);
    c = c > 0x7Eu ? 0x7Eu : c;
  } else {
    c = (uint32_t)__builtin_rintf(r * 512.0f);
  }
  const float v = e4m3_pos(c);
  const float hi = c < 0x7Eu ? 3.0f * (v + e4m3_pos(c + 1)) : __builtin_inff();
  const float lo = c > 0u ? 3.0f * (e4m3_pos(c - 1) + v) : -1.0f;
  if (amax > hi || (amax == hi && (c & 1u))) return c + 1;          // a tie goes to the even neighbour
  if (amax < lo || (amax == lo && (c & 1u))) return c - 1;
  return c;
}

// t = RN32(y / s) for a block scale value s (E4M3, at most 4 significant
// bits) and its reciprocal rinv = RN32(1 / s): Markstein's correction of
// q0 = RN(y * rinv).  The remainder fma(q0, s, -y) is exact, and the corrected
// value before its one rounding lies within 2^-23 ulp of y / s, while y / s
// (24-bit over 4-bit) is never an fp32 midpoint and never within 2^-6 ulp of
// one, so the result is the correctly rounded quotient.  t keeps the sign of a
// signed-zero y, and t = +-0 when s = 0 (rinv = 0).
__device__ __forceinline__ float div_scale(float y, float s, float rinv) {
#pragma clang fp contract(off)
  const float q0 = y * rinv;
  const float rr = __builtin_fmaf(q0, s, -y);
  return __builtin_fmaf(-rr, rinv, q0);
}

__device__ __forceinline__ float scale_reciprocal(uint32_t sc, float s) {
#pragma clang fp contract(off)
  return sc ? (float)(1.0 / (double)s) : 0.0f;                    // RN32(1/s)
}

// Eight values of a block (t = y / s already formed) to eight E2M1 codes in
// one dword, value j in nibble j (round to nearest even, saturating at 6).
__device__ __forceinline__ uint32_t e2m1_pack8(const float* t) {
  uint32_t acc = 0u;
  acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, t[0], t[1], 1.0f, 0);
  acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, t[2], t[3], 1.0f, 1);
  acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, t[4], t[5], 1.0f, 2);
  acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, t[6], t[7], 1.0f, 3);
  return acc;
}

// One 16-value block: its E4M3 scale code (nearest to max|y| / 6) and the
// packed E2M1 codes of y / scale (value j in nibble j, low nibble first).
__device__ __forceinline__ u32x2 quant_block16(float* y, uint32_t& scode) {
#pragma clang fp contract(off)
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i += 2)
    amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(y[i]), __builtin_fabsf(y[i + 1])));
  const uint32_t sc = e4m3_scale_code(amax);
  scode = sc;
  const float s = e4m3_pos(sc);
  const float rinv = scale_reciprocal(sc, s);
  float t[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = div_scale(y[i], s, rinv);
  u32x2 w;
  w[0] = e2m1_pack8(t);
  w[1] = e2m1_pack8(t + 8);
  return w;
}


}  // namespace lsd
