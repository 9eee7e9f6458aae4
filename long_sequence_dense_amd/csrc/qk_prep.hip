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
//   quant (Q)        four lanes per 128-channel row, 32 consecutive channels
//                    per lane: butterfly stages 0-4 in registers, stages 5-6
//                    across the lane quad (DPP); times RN32(1/sqrt(128)); per
//                    16-channel block the E4M3 scale (a candidate from
//                    max|y| * (1/6), settled exactly against the two
//                    neighbouring rounding boundaries); codes from the correctly rounded
//                    quotient y/s (Markstein's correction from y * RN(1/s))
//                    and the hardware E2M1 conversion with a unit
//                    (power-of-two) scale.
//   kmean_partial    exact partial column sums of K in fp64: a thread sums up
//                    to n = 256 BF16 values per channel; all of them are
//                    multiples of 2^(E_min-134) and below 2^(E_max-126), so
//                    the fp64 sum is exact when E_max - E_min <= 45 - log2(n)
//                    (tracked per thread with packed 16-bit min/max);
//                    otherwise the partial is flagged and recomputed exactly
//                    by kmean_final.
//   kmean_final      one wave per (head, channel): adds the partials in fp64
//                    with every addition checked by TwoSum; when one rounded
//                    (or a partial was flagged), adds the exact partials
//                    into 320-bit two's-complement integers (units of
//                    2^-133), combines them, rounds once to fp64 (nearest,
//                    ties to even).  Then divides by L in fp64 and rounds to
//                    fp32.
//   quant (K)        as for Q after x = RN32(k - mean).
// Ablation variants (same section: plain quantization against quantization
// after the two transforms): without smoothing the mean kernels are skipped
// and K is quantized as given; without the rotation the butterfly and the
// 1/sqrt(128) factor are skipped and each block is 16 consecutive channels.
#include <mutex>

#include "lsd_internal.h"
#include "device_common.h"
#include "nvfp4_quant.h"
#include "../../include/lsd_attn.h"

namespace lsd {
namespace {

constexpr int QUANT_THREADS = 256;              // 64 rows per iteration
constexpr int MEAN_THREADS = QUANT_THREADS;     // 16 row slots x 16 channel groups (shares a grid)
constexpr int MEAN_ROWS = 4096;                 // rows per column-sum workgroup
constexpr int MEAN_SLOTS = MEAN_THREADS / 16;   // partials per channel per workgroup
constexpr int MEAN_PER_THREAD = MEAN_ROWS / MEAN_SLOTS;   // values summed by one thread (a power of two)
// Largest exponent span for which the fp64 sum of MEAN_PER_THREAD values is
// certified exact: MEAN_PER_THREAD * 2^(span + 8) <= 2^53.
constexpr int kMeanSpan = 45 - __builtin_ctz(MEAN_PER_THREAD);
static_assert((MEAN_PER_THREAD & (MEAN_PER_THREAD - 1)) == 0, "rows per thread must be a power of two");

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

int mean_chunks(int L) { return (L + MEAN_ROWS - 1) / MEAN_ROWS; }

// ---------------------------------------------------------------- quantizer --

// Partner value across the lane quad: lane ^ 1 and lane ^ 2.
__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}

// Four lanes per 128-channel row, 32 consecutive channels per lane.  grid:
// (row blocks of one head, heads), one lane quad per row.  K (KMEAN):
// x = RN32(k - mean) first.  ROT: the rotation (otherwise y = x).
template <bool KMEAN, bool ROT>
__global__ __launch_bounds__(QUANT_THREADS) void quant_kernel(const uint16_t* __restrict__ src,
                                                              const float* __restrict__ kmean,
                                                              uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales, int L) {
  const int tid = threadIdx.x;
  const int part = tid & 3;                      // channels 32*part .. 32*part+31
  const int r = blockIdx.x * (QUANT_THREADS / 4) + (tid >> 2);
  const int h = blockIdx.y;
  const bool valid = r < L;
  if constexpr (!KMEAN) {
    if (!valid) return;                          // whole lane quads leave together
  }
  const long long row = (long long)h * L + r;
  const uint16_t* rp = src + row * kHeadDim + part * 32;
  u32x4 raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[i] = (!KMEAN || valid) ? *(const u32x4*)(rp + 8 * i) : (u32x4)0;
  // Every row of the workgroup is in head h: its mean is read once into LDS,
  // by the first 32 threads, before any thread leaves.
  __shared__ __attribute__((aligned(16))) float km[kHeadDim];
  if constexpr (KMEAN) {
    if (tid < kHeadDim / 4) *(f32x4*)(km + 4 * tid) = *(const f32x4*)(kmean + h * kHeadDim + 4 * tid);
    __syncthreads();
  }
  if constexpr (KMEAN) {
    if (!valid) return;
  }

  float x[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * i + 2 * j] = __uint_as_float(raw[i][j] << 16);
      x[8 * i + 2 * j + 1] = __uint_as_float(raw[i][j] & 0xFFFF0000u);
    }
  }
  if constexpr (KMEAN) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4 m4 = *(const f32x4*)(km + part * 32 + 4 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[4 * i + j] = x[4 * i + j] - m4[j];
    }
  }
  if constexpr (ROT) {
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
    // stages 5 and 6: channel bits 5 and 6 are bits 0 and 1 of the lane in its
    // quad.  The lane with the bit clear holds x_i and forms x_i + x_j; its
    // partner holds x_j and forms x_i - x_j; fma(own, +-1, partner) is that one
    // rounded operation, signed zeros included.
    const float k5 = (part & 1) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = __builtin_fmaf(x[i], k5, dpp_xor1(x[i]));
    const float k6 = (part & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = __builtin_fmaf(x[i], k6, dpp_xor2(x[i]));
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = x[i] * kHadamardScale;
  }

  u32x4 wv;
  uint32_t scode[2];
#pragma unroll
  for (int blk2 = 0; blk2 < 2; ++blk2) {
    const u32x2 c = quant_block16(x + 16 * blk2, scode[blk2]);
    wv[2 * blk2] = c[0];
    wv[2 * blk2 + 1] = c[1];
  }
  *(u32x4*)(codes + row * (kHeadDim / 2) + part * 16) = wv;
  *(uint16_t*)(scales + row * (kHeadDim / kBlock) + part * 2) = (uint16_t)(scode[0] | (scode[1] << 8));
}

// NVFP4 quantization of the rows of a linear layer's operand: y = RN32(x / g)
// for the tensor's global scale g, then each block of 16 consecutive values of
// a row is quantized as above (no rotation).
//
// The quotient is formed as y = RN32(RN64(x * r64)) with r64 = RN64(1 / g);
// for every BF16 x and float32 g > 0 whose quotient is not in float32's
// subnormal range, that is exactly RN32(x / g):
//   * x = X 2^a and g = G 2^b with odd integers X < 2^8 and G < 2^24.  A
//     rounding boundary of normal float32 values (a midpoint, or the overflow
//     threshold 2^128 - 2^103) is m = M 2^c with M odd, 2^24 < M < 2^25.
//     x / g = m would need X = G M > 2^8: impossible.  Otherwise
//     x / g - m = (X 2^a - G M 2^(b+c)) / (G 2^b), and a > b + c (the two
//     terms are within a factor of two and X < 2^8 < M), so the numerator is
//     a nonzero multiple of 2^(b+c): x / g is at least 2^c / G, i.e. more
//     than 2^-49 |m|, away from m.
//   * r64 and the product are one fp64 rounding each: the product lies within
//     (1 + 2^-53)^2 - 1 < 2^-52 of x / g relatively, on the same side of every
//     boundary, so rounding it to float32 gives the float32 nearest to x / g
//     (infinite past the overflow threshold).
// Subnormal quotients (|product| < 2^-126) can sit exactly on a boundary
// (x = 15 * 2^-133, g = 3 * 2^17 gives 5 * 2^-150); there the fp64 quotient
// x / g (IEEE division, exact whenever x / g fits in fp64) rounded to float32
// is used, which is RN32(x / g) by Figueroa's double-rounding theorem
// (53 >= 2 * 24 + 2).  An infinite y is replaced by +-FLT_MAX: it takes the
// same scale (448) and the same code (+-6) as +-inf.
struct GlobalScale {
  double r;   // RN64(1 / g)
  double g;
};

__device__ __forceinline__ float clamp_finite(float y) {
  return __builtin_fminf(__builtin_fmaxf(y, -3.40282347e38f), 3.40282347e38f);
}

// Sixteen quotients of one block.  The rare subnormal ones are redone with the
// division behind one branch for the whole block, so the common path stays a
// multiply and two conversions per value.
__device__ __forceinline__ void div_global16(const float* x, const GlobalScale& gs, float* y) {
  bool rare = false;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const double p = (double)x[i] * gs.r;
    rare = rare || (p != 0.0 && __builtin_fabs(p) < 0x1p-126);
    y[i] = (float)p;
  }
  if (__builtin_expect(rare, 0)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const double p = (double)x[i] * gs.r;
      if (p != 0.0 && __builtin_fabs(p) < 0x1p-126) y[i] = (float)((double)x[i] / gs.g);
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = clamp_finite(y[i]);
}

__device__ __forceinline__ u32x2 quant_linear_raw(u32x4 a, u32x4 b, const GlobalScale& gs, uint32_t& sc) {
  float x[16], y[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = __uint_as_float(a[j] << 16);
    x[2 * j + 1] = __uint_as_float(a[j] & 0xFFFF0000u);
    x[8 + 2 * j] = __uint_as_float(b[j] << 16);
    x[8 + 2 * j + 1] = __uint_as_float(b[j] & 0xFFFF0000u);
  }
  div_global16(x, gs, y);
  return quant_block16(y, sc);
}

__device__ __forceinline__ u32x2 quant_linear_block(const uint16_t* src, const GlobalScale& r, uint32_t& sc) {
  const u32x4* p = (const u32x4*)src;
  return quant_linear_raw(p[0], p[1], r, sc);
}

// Row-major output: thread i takes block i (values 16 i .. 16 i + 15; rows
// are whole blocks), codes at 8 i, scale at i.
__global__ __launch_bounds__(QUANT_THREADS) void nvfp4_quant_rows_kernel(const uint16_t* __restrict__ src,
                                                                        uint8_t* __restrict__ codes,
                                                                        uint8_t* __restrict__ scales,
                                                                        long long nblocks, GlobalScale r) {
  const long long i = (long long)blockIdx.x * QUANT_THREADS + threadIdx.x;
  if (i >= nblocks) return;
  uint32_t sc;
  *(u32x2*)(codes + 8 * i) = quant_linear_block(src + 16 * i, r, sc);
  scales[i] = (uint8_t)sc;
}

// Tiled output (the product's load order): rows in tiles of kLinTileRows, K in
// stages of kLinStage values; chunk (tile, stage) holds the tile's rows, each
// row's kLinStage / 16 blocks contiguous (8 bytes of codes, 1 byte of scale
// per block), chunks ordered tile-major.  Rows past the matrix and blocks past
// K are written as zeros.  Workgroup g * ceil(stages / 4) + h takes rows
// 32 g .. 32 g + 31 and stages 4 h .. 4 h + 3; lane l of wave w takes row 32 g + 8 w + l / 8 and the
// two adjacent blocks 2 (l % 8) and 2 (l % 8) + 1 of the four stages: a wave
// reads 512 contiguous bytes of each of its 8 rows and writes, per stage and
// row, 32 contiguous bytes of codes with two 16-byte stores.
__global__ __launch_bounds__(QUANT_THREADS) void nvfp4_quant_tiled_kernel(const uint16_t* __restrict__ src,
                                                                         uint8_t* __restrict__ codes,
                                                                         uint8_t* __restrict__ scales,
                                                                         long long rows, int kb_real, int stages,
                                                                         GlobalScale r) {
  constexpr int kbs = kLinStage / kBlock;                 // blocks per row per stage
  static_assert(QUANT_THREADS == 32 * 8 && kbs == 4 && kLinTileRows % 32 == 0, "32 rows x 4 stages per workgroup");
  const int hgroups = (stages + 3) / 4;                   // consecutive workgroups sweep one row group's K
  const long long g = blockIdx.x / hgroups;
  const int h = (int)(blockIdx.x - g * hgroups);
  const long long row = g * 32 + (threadIdx.x >> 3);
  const int pair = threadIdx.x & 7;                       // blocks 2 pair, 2 pair + 1 of the four stages
  const int stage = h * 4 + (pair >> 1);
  if (stage >= stages) return;
  const int kg = stage * kbs + 2 * (pair & 1);            // first of the two blocks
  u32x4 c = {0u, 0u, 0u, 0u};
  uint32_t s2 = 0u;
  if (row < rows && kg + 1 < kb_real) {                   // both blocks: all four loads issued first
    const u32x4* p = (const u32x4*)(src + (row * kb_real + kg) * kBlock);
    const u32x4 a0 = p[0], b0 = p[1], a1 = p[2], b1 = p[3];
    uint32_t s0, s1;
    const u32x2 c0 = quant_linear_raw(a0, b0, r, s0);
    const u32x2 c1 = quant_linear_raw(a1, b1, r, s1);
    c = u32x4{c0[0], c0[1], c1[0], c1[1]};
    s2 = (s0 & 0xFFu) | ((s1 & 0xFFu) << 8);
  } else if (row < rows && kg < kb_real) {                // the row's last block, K / 16 odd
    uint32_t s0;
    const u32x2 c0 = quant_linear_block(src + (row * kb_real + kg) * kBlock, r, s0);
    c[0] = c0[0];
    c[1] = c0[1];
    s2 = s0 & 0xFFu;
  }
  const long long chunk = (row / kLinTileRows) * stages + stage;
  const int within = (int)(row % kLinTileRows) * kbs + 2 * (pair & 1);
  *(u32x4*)(codes + chunk * (kLinTileRows * kLinStage / 2) + 8 * within) = c;
  *(uint16_t*)(scales + chunk * (kLinTileRows * kbs) + within) = (uint16_t)s2;
}

// ---------------------------------------------------------------- mean -------

// 16 bytes of K read by the column sums: a non-temporal load, so the lines of
// this one-pass stream are not kept in the caches.  A wave's load covers 1 KB
// of consecutive rows; read this way the column sums take about 200 us
// instead of 250 us at 40 x 109,000 (a plain streaming read reaches about
// 7.0 TB/s with such loads against 5.6-6.4 TB/s with ordinary ones).  The
// quantizers keep ordinary loads: each of their load instructions covers a
// quarter of every 64-byte piece of a wave's 4 KB, and the other three
// quarters come from the cache.
__device__ __forceinline__ u32x4 stream_load16(const uint16_t* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

// Exact partial column sums of rows chunk*MEAN_ROWS .. +MEAN_ROWS-1 of head h.
// Thread t: channels 8*(t%16) .. +7, rows r0 + t/16 + 16*i.
__device__ __forceinline__ void mean_block(const uint16_t* __restrict__ k, double* __restrict__ parts, int L,
                                           int nparts, int h, int chunk) {
  const int tid = threadIdx.x;
  const int g = tid & 15, slot = tid >> 4;
  const int r0 = chunk * MEAN_ROWS;
  const int r1 = min(L, r0 + MEAN_ROWS);
  const uint16_t* base = k + (size_t)h * (size_t)L * kHeadDim + 8 * g;
  double acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0;
  u16x2 emax = {0, 0};                          // max magnitude bits (sign cleared)
  u16x2 emin = {0xFFFF, 0xFFFF};                // min of (magnitude bits - 1): zero never wins
  constexpr int U = 4;                           // rows in flight per thread
  for (int r = r0 + slot; r < r1; r += U * MEAN_SLOTS) {
    u32x4 w[U];                                  // rows past the end add zero
#pragma unroll
    for (int u = 0; u < U; ++u)
      w[u] = r + u * MEAN_SLOTS < r1 ? stream_load16(base + (size_t)(r + u * MEAN_SLOTS) * kHeadDim) : (u32x4)0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += (double)__uint_as_float(w[u][j] << 16);
        acc[2 * j + 1] += (double)__uint_as_float(w[u][j] & 0xFFFF0000u);
        const u16x2 mag = __builtin_bit_cast(u16x2, w[u][j] & 0x7FFF7FFFu);
        emax = __builtin_elementwise_max(emax, mag);
        emin = __builtin_elementwise_min(emin, mag - (u16x2){1, 1});
      }
    }
  }
  const uint32_t mx = emax[0] > emax[1] ? emax[0] : emax[1];
  const uint32_t mn = emin[0] < emin[1] ? emin[0] : emin[1];
  bool exact = true;
  if (mn != 0xFFFFu) {                           // some nonzero value
    const int e_max = (int)(mx >> 7);
    int e_min = (int)((mn + 1) >> 7);
    e_min = e_min < 1 ? 1 : e_min;               // subnormals share exponent 1's quantum
    exact = e_max - e_min <= kMeanSpan;
  }
  double* out = parts + ((size_t)h * kHeadDim + 8 * g) * nparts + (size_t)chunk * MEAN_SLOTS + slot;
#pragma unroll
  for (int j = 0; j < 8; ++j) out[(size_t)j * nparts] = exact ? acc[j] : __builtin_nan("");
}

// 320-bit two's-complement accumulator in units of 2^-133.
struct BigSum {
  uint64_t limb[5];
  __device__ void clear() {
#pragma unroll
    for (int j = 0; j < 5; ++j) limb[j] = 0;
  }
  // += B * 2^sh for a signed 64-bit B and 0 <= sh < 256.
  __device__ void add_shifted(long long B, int sh) {
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
  // += one BF16 value, exactly: +-M * 2^(E-134), subnormals as E = 1.
  __device__ void add_bf16(uint32_t b) {
    uint32_t e = (b >> 7) & 0xFF;
    uint32_t m = b & 0x7F;
    if (e) m |= 0x80; else e = 1;
    if (m) add_shifted((b & 0x8000) ? -(long long)m : (long long)m, (int)e - 1);
  }
  // += an fp64 value that is an exact multiple of 2^-133.
  __device__ void add_f64(double d) {
    const uint64_t bits = __double_as_longlong(d);
    const int e = (int)((bits >> 52) & 0x7FF);
    if (e == 0) return;                          // zero (no nonzero multiple of 2^-133 is this small)
    const long long m = (long long)((bits & ((1ull << 52) - 1)) | (1ull << 52));
    const long long sm = (bits >> 63) ? -m : m;
    const int sh = e - 1075 + 133;               // value = m * 2^(e-1075)
    if (sh >= 0) add_shifted(sm, sh);
    else add_shifted(sm >> (-sh), 0);            // the dropped bits are zero
  }
  // RN64 of the sum.
  __device__ double round_f64() {
    const bool neg = (long long)limb[4] < 0;
    uint64_t mag[5];
    uint64_t carry = neg ? 1ull : 0ull;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const uint64_t x = neg ? ~limb[j] + carry : limb[j];
      carry = (neg && carry && x == 0) ? 1ull : 0ull;
      mag[j] = x;
    }
    int top = -1;
#pragma unroll
    for (int j = 4; j >= 0; --j)
      if (top < 0 && mag[j] != 0) top = 64 * j + 63 - __clzll(mag[j]);
    if (top < 0) return 0.0;
    auto window = [&](int pos) -> uint64_t {                     // bits [pos, pos + 64)
      const int w = pos >> 6, r = pos & 63;
      uint64_t x = w < 5 ? (mag[w] >> r) : 0ull;
      if (r && w + 1 < 5) x |= mag[w + 1] << (64 - r);
      return x;
    };
    double v;
    if (top <= 52) {
      v = __builtin_ldexp((double)mag[0], -133);                 // exact
    } else {
      int shift = top - 52;
      uint64_t m = window(shift) & ((1ull << 53) - 1);
      const bool guard = (window(shift - 1) & 1ull) != 0;
      bool sticky = false;
      for (int j = 0; j < 5 && !sticky; ++j) {
        const int lo_bit = 64 * j;
        if (lo_bit >= shift - 1) break;
        const int nb = (shift - 1) - lo_bit;                     // bits of this limb below the guard bit
        const uint64_t mask = nb >= 64 ? ~0ull : ((1ull << nb) - 1);
        sticky = (mag[j] & mask) != 0;
      }
      if (guard && (sticky || (m & 1ull))) ++m;
      if (m >> 53) { m >>= 1; ++shift; }
      v = __builtin_ldexp((double)m, shift - 133);
    }
    return neg ? -v : v;
  }
};

// s + e = a + b exactly (Knuth's TwoSum, round to nearest, no overflow): the
// fp64 addition a + b was exact iff e == 0.
__device__ __forceinline__ double two_sum(double a, double b, double& e) {
  const double s = a + b;
  const double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
  return s;
}

// One wave per (head, channel).  Fast path: the partials are added in fp64
// (each lane its share, then a butterfly across the wave), every addition
// checked with TwoSum; if none rounded and no partial was flagged, the fp64
// result is the exact column sum.  Otherwise: each lane adds its share into
// its own 320-bit integer, then lane 0 adds the 64 integers (exact).  Both
// paths round the exact sum once to fp64.
constexpr int FINAL_THREADS = 64;

__global__ __launch_bounds__(FINAL_THREADS) void kmean_final_kernel(const uint16_t* __restrict__ k,
                                                                    const double* __restrict__ parts,
                                                                    float* __restrict__ kmean, int L, int nparts) {
  __shared__ uint64_t limbs[FINAL_THREADS][5];
  const int i = blockIdx.x;                                     // head * 128 + channel
  const int h = i / kHeadDim, c = i - h * kHeadDim;
  const int lane = threadIdx.x;
  const double* p = parts + (size_t)i * nparts;
  {
    double sum = 0.0;
    bool exact = true;
    for (int j = lane; j < nparts; j += FINAL_THREADS) {
      const double d = p[j];
      double e;
      sum = two_sum(sum, d, e);
      exact = exact && d == d && e == 0.0;
    }
#pragma unroll
    for (int off = FINAL_THREADS / 2; off > 0; off >>= 1) {
      double e;
      sum = two_sum(sum, __shfl_xor(sum, off, FINAL_THREADS), e);
      exact = exact && e == 0.0;
    }
    if (__all(exact)) {                          // uniform across the wave
      if (lane == 0) kmean[i] = (float)((sum == 0.0 ? 0.0 : sum) / (double)L);   // an exact zero sum is +0
      return;
    }
  }
  BigSum acc;
  acc.clear();
  for (int j = lane; j < nparts; j += FINAL_THREADS) {
    const double d = p[j];
    if (d == d) {
      acc.add_f64(d);
    } else {                                     // flagged: recompute this partial's values exactly
      const int chunk = j / MEAN_SLOTS, slot = j - chunk * MEAN_SLOTS;
      const int r1 = min(L, (chunk + 1) * MEAN_ROWS);
      const uint16_t* col = k + (size_t)h * (size_t)L * kHeadDim + c;
      for (int r = chunk * MEAN_ROWS + slot; r < r1; r += MEAN_SLOTS) acc.add_bf16(col[(size_t)r * kHeadDim]);
    }
  }
#pragma unroll
  for (int j = 0; j < 5; ++j) limbs[lane][j] = acc.limb[j];
  __syncthreads();
  if (lane == 0) {
    for (int t = 1; t < FINAL_THREADS; ++t) {
      uint64_t carry = 0;
#pragma unroll
      for (int j = 0; j < 5; ++j) {
        const uint64_t add = limbs[t][j];
        const uint64_t s1 = acc.limb[j] + add;
        const uint64_t c1 = s1 < add;
        const uint64_t s2 = s1 + carry;
        const uint64_t c2 = s2 < s1;
        acc.limb[j] = s2;
        carry = c1 | c2;
      }
    }
    kmean[i] = (float)(acc.round_f64() / (double)L);
  }
}

// The K column sums.  grid (chunks, H).
__global__ __launch_bounds__(MEAN_THREADS) void kmean_partial_kernel(const uint16_t* __restrict__ k,
                                                                     double* __restrict__ parts, int L,
                                                                     int nparts) {
  mean_block(k, parts, L, nparts, (int)blockIdx.y, (int)blockIdx.x);
}

__global__ void fill_zero_kernel(float* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

template <bool KMEAN, bool ROT>
void launch_quant(const uint16_t* src, const float* kmean, uint8_t* codes, uint8_t* scales, int H, int L,
                  hipStream_t stream) {
  const unsigned blocks = (unsigned)((L + (QUANT_THREADS / 4) - 1) / (QUANT_THREADS / 4));
  hipLaunchKernelGGL((quant_kernel<KMEAN, ROT>), dim3(blocks, H), dim3(QUANT_THREADS), 0, stream, src, kmean, codes,
                     scales, L);
}

}  // namespace

hipError_t launch_nvfp4_quantize(const uint16_t* x, uint8_t* codes, uint8_t* scales, long long rows, int cols,
                                 float global_scale, bool tiled, hipStream_t stream) {
  const GlobalScale r = {1.0 / (double)global_scale, (double)global_scale};
  if (tiled) {
    const int stages = (cols + kLinStage - 1) / kLinStage;
    const long long groups = (rows + kLinTileRows - 1) / kLinTileRows * (kLinTileRows / 32) * ((stages + 3) / 4);
    if (groups > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(nvfp4_quant_tiled_kernel, dim3((unsigned)groups),
                       dim3(QUANT_THREADS), 0, stream, x, codes, scales, rows, cols / kBlock, stages, r);
    return hipGetLastError();
  }
  const long long nblocks = rows * (cols / kBlock);
  const long long grid = (nblocks + QUANT_THREADS - 1) / QUANT_THREADS;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(nvfp4_quant_rows_kernel, dim3((unsigned)grid), dim3(QUANT_THREADS), 0, stream, x, codes, scales,
                     nblocks, r);
  return hipGetLastError();
}

// Static scratch of the no-allocation prep: the exact partial column sums of K
// for up to LSD_PREP_NOALLOC_MAX_HEAD_CHUNKS (head, 4096-token chunk) pairs.
// In host code `scratch` names a host-side stand-in; the device address of
// each GPU's copy comes from hipGetSymbolAddress on that device.
constexpr size_t kScratchBytes = (size_t)LSD_PREP_NOALLOC_MAX_HEAD_CHUNKS * kHeadDim * MEAN_SLOTS * sizeof(double);
static __device__ __align__(256) double scratch[kScratchBytes / sizeof(double)];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

size_t prep_scratch_bytes() { return kScratchBytes; }

// This device's address of `scratch`, looked up on the first call with the
// device current (the caller's current device), then kept.
hipError_t prep_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t prep_workspace_bytes(int H, int L) {
  return (size_t)H * kHeadDim * (size_t)mean_chunks(L) * MEAN_SLOTS * sizeof(double);
}

hipError_t launch_qk_prep(const uint16_t* q, const uint16_t* k, uint8_t* qc, uint8_t* qs, uint8_t* kc,
                          uint8_t* ks, float* kmean, void* ws, int H, int L, bool smooth, bool rotate,
                          bool with_q, hipStream_t stream) {
  if (with_q) {
    if (rotate) launch_quant<false, true>(q, nullptr, qc, qs, H, L, stream);
    else launch_quant<false, false>(q, nullptr, qc, qs, H, L, stream);
  }
  if (smooth) {
    double* parts = (double*)ws;
    const int nchunks = mean_chunks(L);
    const int nparts = nchunks * MEAN_SLOTS;
    hipLaunchKernelGGL(kmean_partial_kernel, dim3(nchunks, H), dim3(MEAN_THREADS), 0, stream, k, parts, L, nparts);
    hipLaunchKernelGGL(kmean_final_kernel, dim3(H * kHeadDim), dim3(FINAL_THREADS), 0, stream, k,
                       (const double*)parts, kmean, L, nparts);
    if (rotate) launch_quant<true, true>(k, kmean, kc, ks, H, L, stream);
    else launch_quant<true, false>(k, kmean, kc, ks, H, L, stream);
  } else {
    if (kmean) hipLaunchKernelGGL(fill_zero_kernel, dim3((H * kHeadDim + 255) / 256), dim3(256), 0, stream, kmean,
                                  H * kHeadDim);
    if (rotate) launch_quant<false, true>(k, nullptr, kc, ks, H, L, stream);
    else launch_quant<false, false>(k, nullptr, kc, ks, H, L, stream);
  }
  return hipGetLastError();
}

}  // namespace lsd
