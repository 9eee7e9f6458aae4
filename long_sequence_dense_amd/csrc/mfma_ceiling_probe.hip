// Dense BF16 matrix-core rate this GPU sustains when nothing but MFMAs run:
// the attainable ceiling against which the attention kernels' rate is read
// (the published peak assumes 2.4 GHz; under a sustained MFMA load the clock
// drops with the power the matrix cores draw, which depends on how many
// operand bits toggle).
//
// 1024 workgroups of eight waves (two per SIMD), each wave 8 independent
// 32x32x16 accumulators fed from registers (no memory traffic and no other
// instructions in the loop), for random BF16 operands (random sign and
// mantissa, exponents 2^-1 .. 2^1) and for all-zero operands.  Prints one
// JSON line: TFLOP/s per operand kind, best of the timed launches.
// Standalone measurement tool built in-tree beside the library; it shares no
// code with it.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstdio>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

namespace {

constexpr int kBlocks = 1024;
constexpr int kThreads = 512;
constexpr int kIters = 2560;            // 16 MFMAs per iteration per wave

__global__ __launch_bounds__(kThreads, 1) void mfma_loop(const u16x8* __restrict__ src, float* __restrict__ out) {
  const int t = threadIdx.x;
  bf16x8 a[4], b[4];
  for (int i = 0; i < 4; ++i) {
    a[i] = __builtin_bit_cast(bf16x8, src[(blockIdx.x * 8 + i) * kThreads + t]);
    b[i] = __builtin_bit_cast(bf16x8, src[(blockIdx.x * 8 + 4 + i) * kThreads + t]);
  }
  f32x16 c[8];
  for (int j = 0; j < 8; ++j) c[j] = (f32x16)0.0f;
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + i) & 3], b[(j >> 1) & 3], c[j], 0, 0, 0);
  }
  float s = 0.0f;
  for (int i = 0; i < 16; ++i)
    for (int j = 0; j < 8; ++j) s += c[j][i];
  out[blockIdx.x * kThreads + t] = s;
}

// xorshift32, seeded: operand bits only
uint32_t next(uint32_t& x) {
  x ^= x << 13;
  x ^= x >> 17;
  x ^= x << 5;
  return x;
}

}  // namespace

int main() {
  const size_t nvec = (size_t)kBlocks * 8 * kThreads;
  std::vector<u16x8> h(nvec);
  uint32_t x = 12345u;
  for (size_t i = 0; i < nvec; ++i)
    for (int j = 0; j < 8; ++j) {
      const uint32_t r = next(x);
      h[i][j] = (uint16_t)(((r & 1u) << 15) | ((126u + (r >> 1) % 3u) << 7) | ((r >> 8) & 0x7Fu));
    }
  u16x8 *dr = nullptr, *dz = nullptr;
  float* out = nullptr;
  if (hipMalloc(&dr, nvec * sizeof(u16x8)) != hipSuccess || hipMalloc(&dz, nvec * sizeof(u16x8)) != hipSuccess ||
      hipMalloc(&out, (size_t)kBlocks * kThreads * sizeof(float)) != hipSuccess ||
      hipMemcpy(dr, h.data(), nvec * sizeof(u16x8), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemset(dz, 0, nvec * sizeof(u16x8)) != hipSuccess) {
    fprintf(stderr, "mfma_ceiling_probe: allocation or copy failed\n");
    return 1;
  }
  const double flop = (double)kBlocks * (kThreads / 64) * kIters * 16 * 32768.0;
  double best[2] = {0.0, 0.0};
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  for (int rep = 0; rep < 3; ++rep)
    for (int zero = 0; zero < 2; ++zero) {
      hipLaunchKernelGGL(mfma_loop, dim3(kBlocks), dim3(kThreads), 0, 0, zero ? dz : dr, out);   // warm-up
      if (hipEventRecord(e0) != hipSuccess) return 1;
      hipLaunchKernelGGL(mfma_loop, dim3(kBlocks), dim3(kThreads), 0, 0, zero ? dz : dr, out);
      if (hipEventRecord(e1) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) return 1;
      float ms = 0.0f;
      if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return 1;
      const double tf = flop / (ms * 1e-3) / 1e12;
      if (tf > best[zero]) best[zero] = tf;
    }
  const hipError_t err = hipDeviceSynchronize();
  if (err != hipSuccess) {
    fprintf(stderr, "mfma_ceiling_probe: %s\n", hipGetErrorString(err));
    return 1;
  }
  printf("{\"mfma_ceiling_bf16_TFLOP/s\": {\"random_operands\": %.1f, \"zero_operands\": %.1f}, "
         "\"flop_per_launch\": %.4e}\n", best[0], best[1], flop);
  return 0;
}
