// Small device-side helpers shared by the gfx950 kernels of this library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// OCP FP8 E4M3 (bias 7, 3 mantissa bits, exponent 0 subnormal) to float.
// Codes 0x00..0x7E and their negatives; never called with the NaN codes.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  const uint32_t e = (code >> 3) & 0xF;
  const uint32_t m = code & 0x7;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * (1.0f / 512.0f);
  return (code & 0x80) ? -mag : mag;
}

// FP4 E2M1 code (bit 3 sign, 2-bit exponent bias 1, 1 mantissa bit) to the
// float32 bit pattern of its value.
__device__ __forceinline__ uint32_t e2m1_to_f32_bits(uint32_t code) {
  const uint32_t e = code & 7;
  uint32_t mag = (e >= 2) ? ((((e >> 1) + 126u) << 23) | ((e & 1u) << 22)) : (e ? 0x3F000000u : 0u);
  return mag | ((code & 8u) << 28);
}

// Two FP4 codes (byte J of w) decoded exactly by the hardware (unit scale),
// times the block scale s.
template <int J>
__device__ __forceinline__ void fp4_pair(uint32_t w, float s, float* f) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, J);
  f[2 * J] = a[0] * s;
  f[2 * J + 1] = a[1] * s;
}

typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));

// E4M3 code to FP16, exactly: the bits (code & 0x7F) << 7 read as FP16 carry
// the exponent and mantissa fields (biases 15 vs 7; a zero exponent lands on
// an FP16 subnormal of the same form), times 2^8; bit 7 is the sign.
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t code) {
  const _Float16 mag = __builtin_bit_cast(_Float16, (uint16_t)((code & 0x7Fu) << 7)) * (_Float16)256.0f;
  return (code & 0x80u) ? -mag : mag;
}

// Two FP4 codes (byte J of w) decoded exactly by the hardware to FP16 (unit
// scale), times the FP16 block scale: one packed multiply, exact.
template <int J>
__device__ __forceinline__ uint32_t fp4_pair_h(uint32_t w, h16x2 s2) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, J) * s2);
}

// 8 codes (one dword, low nibble first) times the FP16 scale s -> 8 FP16 bit
// patterns.  E2M1 x E4M3 products have at most 6 significant bits and lie in
// [2^-10, 2688] when nonzero: exact FP16 normals.
__device__ __forceinline__ u16x8 dequant8_h(uint32_t w, _Float16 s) {
  const h16x2 s2 = {s, s};
  u32x4 r;
  r[0] = fp4_pair_h<0>(w, s2);
  r[1] = fp4_pair_h<1>(w, s2);
  r[2] = fp4_pair_h<2>(w, s2);
  r[3] = fp4_pair_h<3>(w, s2);
  return __builtin_bit_cast(u16x8, r);
}

// 8 codes (one dword, low nibble first) times scale s -> 8 BF16 bit patterns.
// Every product E2M1 x E4M3 has at most 6 significant bits and lies in
// [2^-10, 2688], so the float32 product is exact and truncating it to BF16 is
// exact.
__device__ __forceinline__ u16x8 dequant8(uint32_t w, float s) {
  float f[8];
  fp4_pair<0>(w, s, f);
  fp4_pair<1>(w, s, f);
  fp4_pair<2>(w, s, f);
  fp4_pair<3>(w, s, f);
  u16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (uint16_t)(__float_as_uint(f[j]) >> 16);
  return r;
}

}  // namespace lsd
