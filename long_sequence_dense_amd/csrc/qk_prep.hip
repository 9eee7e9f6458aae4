// Q/K preparation for FP4-QK attention on gfx950: exact mean key, Hadamard
// rotation, NVFP4 block quantization.
//
// Method: "Pika H3 Flex in FastVideo: 7x Faster, and Near Real Time in 4-bit",
// section "FP4 attention": subtract each head's mean key, multiply Q and K by
// the same orthonormal Hadamard matrix, quantize both to E2M1 with one E4M3
// scale per 16 channels and unit global scale, all in a fused pass.
//
// This translation unit is built with -ffp-contract=off: every float operation
// below is one IEEE operation with round-to-nearest-even, in the order
// written, so the codes are an exact function of the inputs.
//
// Kernels (in launch order):
//   zero_ws      clear the integer workspace (a fill kernel, graph-safe).
//   kmean_bins   exact column sums of K: each BF16 value is +-M * 2^(E-134)
//                with an 8-bit integer M, so per (channel, exponent E) an
//                integer sum of +-M is exact; LDS int32 bins per workgroup,
//                flushed into int64 bins [H][128][256] with integer atomics
//                (order-independent, hence deterministic).
//   kmean_final  one thread per (head, channel): combine the 256 bins into a
//                320-bit two's-complement integer, round it once to fp64
//                (nearest, ties to even), divide by L in fp64 and round to
//                fp32.
//   nvfp4_quant  four lanes per 128-channel row, 32 consecutive channels per
//                lane: (K only) subtract the mean; butterfly stages 0-4 in
//                registers, stages 5-6 across the lane quad (DPP); multiply by
//                RN32(1/sqrt(128)); per 16-channel block the E4M3 scale; codes
//                via a correctly rounded quotient y/s and the hardware
//                E2M1 conversion with a unit (power-of-two) scale.
#include "lsd_internal.h"
#include "device_common.h"

namespace lsd {
namespace {

constexpr int BIN_STRIDE = kExpBins + 1;        // padded LDS row of bins (bank spread)
constexpr int MEAN_THREADS = 256;
constexpr int QUANT_THREADS = 256;              // 64 rows per workgroup
constexpr float kHadamardScale = 0x1.6a09e6p-4f;   // RN32(1/sqrt(128)), bits 0x3DB504F3

__global__ __launch_bounds__(256) void zero_ws_kernel(unsigned long long* __restrict__ ws, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    ws[i] = 0ull;
}

__global__ __launch_bounds__(MEAN_THREADS) void kmean_bins_kernel(const uint16_t* __restrict__ k,
                                                                  unsigned long long* __restrict__ bins,
                                                                  int L, int rows_per_block) {
  __shared__ int sb[kHeadDim * BIN_STRIDE];
  const int h = blockIdx.y;
  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(L, r0 + rows_per_block);
  for (int i = threadIdx.x; i < kHeadDim * BIN_STRIDE; i += MEAN_THREADS) sb[i] = 0;
  __syncthreads();
  const uint16_t* base = k + (size_t)h * (size_t)L * kHeadDim;
  const int nchunks = (r1 - r0) * (kHeadDim / 8);
  for (int id = threadIdx.x; id < nchunks; id += MEAN_THREADS) {
    const int row = r0 + (id >> 4);
    const int c0 = (id & 15) * 8;
    const u16x8 v = *(const u16x8*)(base + (size_t)row * kHeadDim + c0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t b = v[j];
      uint32_t e = (b >> 7) & 0xFF;
      uint32_t m = b & 0x7F;
      if (e) m |= 0x80; else e = 1;             // subnormal: M * 2^(1-134)
      if (m) atomicAdd(&sb[(c0 + j) * BIN_STRIDE + e], (b & 0x8000) ? -(int)m : (int)m);
    }
  }
  __syncthreads();
  unsigned long long* gb = bins + (size_t)h * kHeadDim * kExpBins;
  for (int i = threadIdx.x; i < kHeadDim * kExpBins; i += MEAN_THREADS) {
    const int v = sb[(i >> 8) * BIN_STRIDE + (i & 255)];
    if (v) atomicAdd(&gb[i], (unsigned long long)(long long)v);
  }
}

// value = sum_e bins[e] * 2^(e - 134) exactly, as a multiple of 2^-133 held in
// 5 little-endian 64-bit limbs (two's complement); then one rounding to fp64.
__global__ __launch_bounds__(256) void kmean_final_kernel(const unsigned long long* __restrict__ bins,
                                                          float* __restrict__ kmean, int n, int L) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const long long* b = (const long long*)(bins + (size_t)i * kExpBins);
  uint64_t limb[5] = {0, 0, 0, 0, 0};
  for (int e = 1; e < 255; ++e) {
    const long long B = b[e];
    if (B == 0) continue;
    const int sh = e - 1;
    const int w = sh >> 6, r = sh & 63;
    const uint64_t ext = B < 0 ? ~0ull : 0ull;
    const uint64_t lo = (uint64_t)B << r;
    const uint64_t hi = r ? (uint64_t)(B >> (64 - r)) : ext;
    uint64_t carry = 0;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const uint64_t add = j < w ? 0ull : (j == w ? lo : (j == w + 1 ? hi : ext));
      const uint64_t s1 = limb[j] + add;
      const uint64_t c1 = s1 < add;
      const uint64_t s2 = s1 + carry;
      const uint64_t c2 = s2 < s1;
      limb[j] = s2;
      carry = c1 | c2;
    }
  }
  const bool neg = (long long)limb[4] < 0;
  if (neg) {
    uint64_t carry = 1;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const uint64_t x = ~limb[j] + carry;
      carry = (carry && x == 0) ? 1ull : 0ull;
      limb[j] = x;
    }
  }
  int top = -1;
#pragma unroll
  for (int j = 4; j >= 0; --j) {
    if (top < 0 && limb[j] != 0) top = 64 * j + 63 - __clzll(limb[j]);
  }
  double value = 0.0;
  if (top >= 0) {
    // bits [pos, pos+64) of the magnitude
    auto window = [&](int pos) -> uint64_t {
      const int w = pos >> 6, r = pos & 63;
      uint64_t x = w < 5 ? (limb[w] >> r) : 0ull;
      if (r && w + 1 < 5) x |= limb[w + 1] << (64 - r);
      return x;
    };
    if (top <= 52) {
      value = __builtin_ldexp((double)limb[0], -133);           // exact
    } else {
      int shift = top - 52;
      uint64_t m = window(shift) & ((1ull << 53) - 1);
      const bool guard = (window(shift - 1) & 1ull) != 0;
      bool sticky = false;
      for (int j = 0; j < 5 && !sticky; ++j) {
        const int lo_bit = 64 * j;
        if (lo_bit >= shift - 1) break;
        const int nb = (shift - 1) - lo_bit;                     // bits of this limb below the guard
        const uint64_t mask = nb >= 64 ? ~0ull : ((1ull << nb) - 1);
        sticky = (limb[j] & mask) != 0;
      }
      if (guard && (sticky || (m & 1ull))) ++m;
      if (m >> 53) { m >>= 1; ++shift; }
      value = __builtin_ldexp((double)m, shift - 133);
    }
    if (neg) value = -value;
  }
  kmean[i] = (float)(value / (double)L);
}

// Nearest E4M3 code to amax / 6 (amax >= 0), ties to even, saturating at 448.
// r = RN32(amax / 6) (one fp64 division, then one rounding to fp32) is never
// pushed onto an E4M3 rounding boundary unless amax / 6 is exactly on it, so
// rounding r to 3 mantissa bits equals rounding amax / 6 itself.
__device__ __forceinline__ uint32_t e4m3_scale_code(float amax) {
  const float r = (float)((double)amax / 6.0);
  if (!(r < 448.0f)) return 0x7Eu;
  if (r >= 0x1p-6f) {
    const uint32_t u = __float_as_uint(r);
    const uint32_t rounded = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;   // exponent|3-bit mantissa, RNE
    return rounded - (120u << 3);
  }
  return (uint32_t)__builtin_rintf(r * 512.0f);                        // subnormal m * 2^-9, m in 0..8
}

__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}

__global__ __launch_bounds__(QUANT_THREADS) void nvfp4_quant_kernel(const uint16_t* __restrict__ src,
                                                                    const float* __restrict__ kmean,
                                                                    uint8_t* __restrict__ codes,
                                                                    uint8_t* __restrict__ scales,
                                                                    long long nrows, int L) {
  const int tid = threadIdx.x;
  const int part = tid & 3;                      // channels 32*part .. 32*part+31
  const long long row = (long long)blockIdx.x * (QUANT_THREADS / 4) + (tid >> 2);
  if (row >= nrows) return;                      // whole lane quads leave together

  const uint16_t* rp = src + row * kHeadDim + part * 32;
  float x[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u16x8 raw = *(const u16x8*)(rp + 8 * i);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[8 * i + j] = bf16_bits_to_f32(raw[j]);
  }
  if (kmean != nullptr) {
    const float* km = kmean + (row / L) * kHeadDim + part * 32;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4 m4 = *(const f32x4*)(km + 4 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[4 * i + j] = x[4 * i + j] - m4[j];
    }
  }
  // butterfly stages 0..4: channel bits 0..4 are the register index
#pragma unroll
  for (int s = 0; s < 5; ++s) {
    const int hs = 1 << s;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & hs) == 0) {
        const float a = x[i], b = x[i + hs];
        x[i] = a + b;
        x[i + hs] = a - b;
      }
    }
  }
  // stages 5 and 6: channel bits 5 and 6 are bits 0 and 1 of the lane in its quad.
  // The lane with the bit clear holds x_i and forms x_i + x_j; its partner holds
  // x_j and forms x_i - x_j; fma(own, +-1, partner) is that one rounded operation.
  const float sg5 = (part & 1) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = __builtin_fmaf(x[i], sg5, dpp_xor1(x[i]));
  const float sg6 = (part & 2) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = __builtin_fmaf(x[i], sg6, dpp_xor2(x[i]));

#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = x[i] * kHadamardScale;

  uint32_t scode[2];
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, __builtin_fabsf(x[16 * blk + i]));
    const uint32_t sc = e4m3_scale_code(amax);
    scode[blk] = sc;
    const float s = e4m3_to_f32(sc);
    const float rinv = sc ? (float)(1.0 / (double)s) : 0.0f;    // RN32(1/s)
    // t = RN32(y / s): Markstein's correction from q0 = RN(y * RN(1/s)); the
    // remainder fma(q0, s, -y) is exact.  Written so that t keeps the sign of
    // y also when y is a signed zero, and t = +-0 when s = 0.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float y = x[16 * blk + i];
      const float q0 = y * rinv;
      const float rr = __builtin_fmaf(q0, s, -y);
      x[16 * blk + i] = __builtin_fmaf(-rr, rinv, q0);
    }
  }
  // E2M1 with round-to-nearest-even and saturation (unit scale): channel 2j in
  // the low nibble of byte j, 2j+1 in the high nibble.
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t acc = 0u;
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, x[8 * d + 0], x[8 * d + 1], 1.0f, 0);
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, x[8 * d + 2], x[8 * d + 3], 1.0f, 1);
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, x[8 * d + 4], x[8 * d + 5], 1.0f, 2);
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, x[8 * d + 6], x[8 * d + 7], 1.0f, 3);
    w[d] = acc;
  }
  u32x4 wv = {w[0], w[1], w[2], w[3]};
  *(u32x4*)(codes + row * (kHeadDim / 2) + part * 16) = wv;
  *(uint16_t*)(scales + row * (kHeadDim / kBlock) + part * 2) = (uint16_t)(scode[0] | (scode[1] << 8));
}

}  // namespace

size_t prep_workspace_bytes(int H) { return (size_t)H * kHeadDim * kExpBins * sizeof(unsigned long long); }

hipError_t launch_qk_prep(const uint16_t* q, const uint16_t* k, uint8_t* qc, uint8_t* qs, uint8_t* kc,
                          uint8_t* ks, float* kmean, void* ws, int H, int L, hipStream_t stream) {
  unsigned long long* bins = (unsigned long long*)ws;
  const size_t nbins = (size_t)H * kHeadDim * kExpBins;
  hipLaunchKernelGGL(zero_ws_kernel, dim3(512), dim3(256), 0, stream, bins, nbins);
  // about two LDS-heavy workgroups per CU in total
  const int blocks_per_head = max(1, min((L + 255) / 256, (512 + H - 1) / H));
  const int rows_per_block = (L + blocks_per_head - 1) / blocks_per_head;
  const int nbx = (L + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(kmean_bins_kernel, dim3(nbx, H), dim3(MEAN_THREADS), 0, stream, k, bins, L,
                     rows_per_block);
  const int n = H * kHeadDim;
  hipLaunchKernelGGL(kmean_final_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, bins, kmean, n, L);
  const long long nrows = (long long)H * L;
  const unsigned qblocks = (unsigned)((nrows + (QUANT_THREADS / 4) - 1) / (QUANT_THREADS / 4));
  hipLaunchKernelGGL(nvfp4_quant_kernel, dim3(qblocks), dim3(QUANT_THREADS), 0, stream, q,
                     (const float*)nullptr, qc, qs, nrows, L);
  hipLaunchKernelGGL(nvfp4_quant_kernel, dim3(qblocks), dim3(QUANT_THREADS), 0, stream, k,
                     (const float*)kmean, kc, ks, nrows, L);
  return hipGetLastError();
}

}  // namespace lsd
