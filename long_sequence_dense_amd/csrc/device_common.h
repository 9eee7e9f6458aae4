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

}  // namespace lsd
