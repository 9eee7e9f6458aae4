// NVFP4 W4A4 linear layer on gfx950 (MI355X): Y = (X^ g_x)(W^ g_w)^T.
//
// Method: "Pika H3 Flex in FastVideo: 7x Faster, and Near Real Time in 4-bit",
// section "NVFP4 QAD": every attention and feed-forward linear runs with 4-bit
// weights and activations, one 8-bit scale per 16 values (the block format of
// section "FP4 attention": E2M1 values, an E4M3 scale per 16 consecutive
// values along K), plus one fp32 global scale per tensor.
//
// gfx950's scaled MFMA takes power-of-two (E8M0) scales per 32 values, and
// its scaled FP4 conversions apply only the power of two of their scale; an
// E4M3 scale per 16 values cannot be folded into either.  E2M1 x E4M3
// products have at most 6 significant bits and lie in [2^-10, 2688], so they
// are exact in FP16 (and BF16): both operands are dequantized exactly while
// they are staged into LDS (FP4 -> packed FP16 conversion, packed FP16
// multiply by the block scale) and multiplied on the 32x32x16 FP16 MFMA with
// fp32 accumulation; the product of the two global scales is applied to the
// fp32 result, which is rounded to BF16.
//
// Tiling: a workgroup computes a 256 (tokens m) x 256 (features n) tile of Y
// as Y^T blocks (W rows are the A operand, X rows the B operand, so that a
// lane's accumulator holds four consecutive features of one token); eight
// waves (two per SIMD) of 128 (n) x 64 (m), i.e. 4 x 2 blocks of 32 x 32.  K
// advances 64 at a time through double-buffered LDS tiles (row stride 144 B:
// the operand reads are free of bank conflicts); the codes of stage s + 1,
// loaded into registers one step earlier, are dequantized into the other
// buffer between the MFMAs of stage s.  With tiled codes a stage of a tile
// is one contiguous chunk, and each thread loads two adjacent blocks per
// operand with one 16-byte load (row-major codes: one load per block).  Workgroups are numbered so that each
// XCD (own L2) takes a contiguous range, walked in bands of 4 token tiles.
// Rows past M or N and blocks past K load as zeros; rows past M or N are not
// stored.
#include "lsd_internal.h"
#include "device_common.h"

namespace lsd {
namespace {

constexpr int GM = 256;                 // tokens (rows of Y) per workgroup
constexpr int GN = 256;                 // features (columns of Y) per workgroup
constexpr int GK = 64;                  // K per LDS stage
constexpr int GT = 512;                 // threads per workgroup
constexpr int GS = GK + 8;              // LDS row stride (fp16 values)
constexpr int NB = GK / kBlock;         // 16-value blocks per row per stage
constexpr int SB = (GN * NB) / GT;      // blocks of one operand staged per thread per stage
constexpr int kOutside = 0x7FFFFFF0;    // a byte offset past every buffer range (loads return 0)
constexpr int kGroup = 4;               // token tiles per band of the workgroup order
static_assert(GM == GN && SB == 2, "staging assumes square tiles and two blocks per thread");
static_assert(GM == kLinTileRows && GK == kLinStage, "the tiled code layout is this kernel's staging order");

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

struct GemmParams {
  const uint8_t* xc;
  const uint8_t* xs;
  const uint8_t* wc;
  const uint8_t* ws;
  uint16_t* y;
  int M, N, K;
  int tiles_n, tiles;
  float gscale;                         // RN32(g_x * g_w)
};

// Two LDS buffers per operand, as separate objects so that the compiler
// knows the stores into one never alias the operand reads from the other.
__shared__ __attribute__((aligned(16))) uint16_t lw0[GN * GS];
__shared__ __attribute__((aligned(16))) uint16_t lw1[GN * GS];
__shared__ __attribute__((aligned(16))) uint16_t lx0[GM * GS];
__shared__ __attribute__((aligned(16))) uint16_t lx1[GM * GS];

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, long long bytes) {
  const int n = bytes > 0x7FFFFFFFLL ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// Exact dequantization of one 16-value block (codes w0, w1; E4M3 scale code
// c, sign clear) into row `row`, block `kb` of an LDS tile: an E2M1 value
// times an E4M3 scale has at most 6 significant bits and lies in [2^-10,
// 2688] when nonzero, so it is exact in FP16 (normal range) as well as BF16.
// The packed FP16 multiply takes two values per instruction.
__device__ __forceinline__ void put_values(uint16_t* tile, int row, int kb, uint32_t w0, uint32_t w1, uint32_t c) {
  // E4M3 scale code to FP16: the bits c << 7 read as FP16 carry the exponent
  // and mantissa fields (biases 15 vs 7, codes with a zero exponent land on
  // FP16 subnormals of the same form), times 2^8 exact.
  const _Float16 sh = __builtin_bit_cast(_Float16, (uint16_t)((c & 0x7Fu) << 7)) * (_Float16)256.0f;
  const f16x2 s2 = {sh, sh};
  u32x4 lo, hi;
  lo[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 0) * s2);
  lo[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 1) * s2);
  lo[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 2) * s2);
  lo[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 3) * s2);
  hi[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 0) * s2);
  hi[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 1) * s2);
  hi[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 2) * s2);
  hi[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 3) * s2);
  *(u32x4*)(tile + row * GS + kBlock * kb) = lo;
  *(u32x4*)(tile + row * GS + kBlock * kb + 8) = hi;
}

// Staging of one operand's stage, row-major codes: thread t stages blocks
// b = t + GT * i (i < SB), row b / NB, values 16 (b % NB) .. +15 of the stage,
// each from its own 8-byte code load and 1-byte scale load.  Blocks past K (a
// ragged last stage, or a stage past the end) read beyond the buffer range:
// zeros.
struct RowsStaging {
  struct Stage {
    u32x2 c[SB];
    uint32_t s[SB];
  };
  __device__ static __forceinline__ void load(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, int K, int k0,
                                              int tid, Stage& st) {
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const int b = tid + GT * i;
      const int row = b / NB, kb = b % NB;
      const bool in = k0 + kBlock * kb < K;
      const int oc = in ? row * (K / 2) + k0 / 2 + 8 * kb : kOutside;
      const int os = in ? row * (K / kBlock) + k0 / kBlock + kb : kOutside;
      st.c[i] = __builtin_amdgcn_raw_buffer_load_b64(rc, oc, 0, 0);
      st.s[i] = __builtin_amdgcn_raw_buffer_load_b8(rs, os, 0, 0);
    }
  }
  __device__ static __forceinline__ void put(uint16_t* tile, int tid, int i, const Stage& st) {
    const int b = tid + GT * i;
    put_values(tile, b / NB, b % NB, st.c[i][0], st.c[i][1], st.s[i] & 0xFFu);
  }
};

// Staging of one operand's stage, tiled codes: the stage is one contiguous
// chunk (blocks in row order, 8 code bytes and 1 scale byte each), and thread
// t stages the adjacent blocks 2t and 2t + 1 (row t / 2, blocks 2 (t % 2) and
// 2 (t % 2) + 1) with one 16-byte code load and one 2-byte scale load.  Stages
// past the end of K lie beyond the buffer range: zeros.
struct TiledStaging {
  struct Stage {
    u32x4 c;
    uint32_t s;
  };
  __device__ static __forceinline__ void load(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, int, int k0,
                                              int tid, Stage& st) {
    const int stage = k0 / GK;
    st.c = __builtin_amdgcn_raw_buffer_load_b128(rc, stage * (GM * GK / 2) + 16 * tid, 0, 0);
    st.s = __builtin_amdgcn_raw_buffer_load_b16(rs, stage * (GM * NB) + 2 * tid, 0, 0);
  }
  __device__ static __forceinline__ void put(uint16_t* tile, int tid, int i, const Stage& st) {
    put_values(tile, tid >> 1, 2 * (tid & 1) + i, st.c[2 * i], st.c[2 * i + 1], (st.s >> (8 * i)) & 0xFFu);
  }
};
static_assert(GT * 2 == GM * NB, "tiled staging gives every thread two blocks of each operand's stage");

__device__ __forceinline__ f16x8 operand(const uint16_t* tile, int lane_off, int row0, int ks) {
  return __builtin_bit_cast(f16x8, *(const u16x8*)(tile + row0 * GS + lane_off + 16 * ks));
}

// One K stage: multiply the tiles in (wt, xt) while the codes in (dw, dx),
// the next stage, are dequantized into (wd, xd), one block per 16-wide step.
template <class SP>
__device__ __forceinline__ void stage_step(const uint16_t* wt, const uint16_t* xt, uint16_t* wd, uint16_t* xd,
                                           const typename SP::Stage& dw, const typename SP::Stage& dx,
                                           f32x16 (&acc)[4][2], int lane_off,
                                           int wn, int wm, int tid) {
#pragma unroll
  for (int ks = 0; ks < GK / 16; ++ks) {
    f16x8 a[4], b[2];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) a[nb] = operand(wt, lane_off, 128 * wn + 32 * nb, ks);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) b[mb] = operand(xt, lane_off, 64 * wm + 32 * mb, ks);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[nb], b[mb], acc[nb][mb], 0, 0, 0);
    if (ks < 2) SP::put(wd, tid, ks, dw);
    else SP::put(xd, tid, ks - 2, dx);
  }
}

template <class SP, bool kTiled>
__global__ __launch_bounds__(GT, 1) void nvfp4_gemm_kernel(GemmParams p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave >> 2, wm = wave & 3;          // wave tile: features 128 wn.., tokens 64 wm..
  const int l32 = lane & 31, hf = lane >> 5;
  const int lane_off = l32 * GS + 8 * hf;

  // XCD-aware numbering (hardware id % 8 = XCD: each XCD, with its own L2,
  // takes a contiguous range), then bands of kGroup token tiles: consecutive
  // workgroups walk the band's token tiles first, then its feature tiles, so
  // the ~32 workgroups an XCD runs at once share 4 X tiles (kept in L2) and
  // 8 W tiles.  A ragged last band is shorter.
  const int nblk = gridDim.x, bid = blockIdx.x;
  const int per = nblk >> 3, rem = nblk & 7, xcd = bid & 7;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + (bid >> 3);
  const int tiles_m = (p.M + GM - 1) / GM;
  const int band = logical / (kGroup * p.tiles_n);
  const int gh = tiles_m - band * kGroup < kGroup ? tiles_m - band * kGroup : kGroup;
  const int in_band = logical - band * kGroup * p.tiles_n;
  const int tm = band * kGroup + in_band % gh, tn = in_band / gh;
  const int m0 = tm * GM, n0 = tn * GN;
  const int K = p.K;

  const long long xrows = p.M - m0 < GM ? p.M - m0 : GM;
  const long long wrows = p.N - n0 < GN ? p.N - n0 : GN;
  const int nst = (K + GK - 1) / GK;
  // a tiled operand's tile is nst contiguous chunks (zero padded); a
  // row-major one is its rows
  const size_t tc = (size_t)nst * (GM * GK / 2), ts = (size_t)nst * (GM * NB);
  const __amdgpu_buffer_rsrc_t rxc = kTiled ? rsrc(p.xc + tm * tc, (long long)tc)
                                            : rsrc(p.xc + (size_t)m0 * (K / 2), xrows * (K / 2));
  const __amdgpu_buffer_rsrc_t rxs = kTiled ? rsrc(p.xs + tm * ts, (long long)ts)
                                            : rsrc(p.xs + (size_t)m0 * (K / kBlock), xrows * (K / kBlock));
  const __amdgpu_buffer_rsrc_t rwc = kTiled ? rsrc(p.wc + tn * tc, (long long)tc)
                                            : rsrc(p.wc + (size_t)n0 * (K / 2), wrows * (K / 2));
  const __amdgpu_buffer_rsrc_t rws = kTiled ? rsrc(p.ws + tn * ts, (long long)ts)
                                            : rsrc(p.ws + (size_t)n0 * (K / kBlock), wrows * (K / kBlock));

  f32x16 acc[4][2];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = (f32x16)0.0f;

  // Register stages: stage s lives in set s % 2 from the top of step s - 2
  // (when it is loaded) to step s - 1 (when it is dequantized into LDS
  // buffer s % 2, which step s multiplies).
  typename SP::Stage w0, x0, w1, x1;
  SP::load(rwc, rws, K, 0, tid, w0);
  SP::load(rxc, rxs, K, 0, tid, x0);
  SP::load(rwc, rws, K, GK, tid, w1);
  SP::load(rxc, rxs, K, GK, tid, x1);
#pragma unroll
  for (int i = 0; i < SB; ++i) {
    SP::put(lw0, tid, i, w0);
    SP::put(lx0, tid, i, x0);
  }
  __syncthreads();

  for (int s = 0; s < nst; s += 2) {
    SP::load(rwc, rws, K, (s + 2) * GK, tid, w0);
    SP::load(rxc, rxs, K, (s + 2) * GK, tid, x0);
    stage_step<SP>(lw0, lx0, lw1, lx1, w1, x1, acc, lane_off, wn, wm, tid);
    __syncthreads();
    if (s + 1 < nst) {
      SP::load(rwc, rws, K, (s + 3) * GK, tid, w1);
      SP::load(rxc, rxs, K, (s + 3) * GK, tid, x1);
      stage_step<SP>(lw1, lx1, lw0, lx0, w0, x0, acc, lane_off, wn, wm, tid);
      __syncthreads();
    }
  }

  // Y^T block (nb, mb): lane holds token m0 + 64 wm + 32 mb + l32 and, per
  // group g, features n0 + 128 wn + 32 nb + 8 g + 4 hf .. +3.
  const bool vec = (p.N & 3) == 0;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = m0 + 64 * wm + 32 * mb + l32;
    if (m >= p.M) continue;
    uint16_t* yrow = p.y + (size_t)m * p.N;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + 128 * wn + 32 * nb + 8 * g + 4 * hf;
        if (n >= p.N) continue;
        u16x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w[j] = __builtin_bit_cast(uint16_t, (__bf16)(acc[nb][mb][4 * g + j] * p.gscale));
        if (vec) {
          *(u16x4*)(yrow + n) = w;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (n + j < p.N) yrow[n + j] = w[j];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_nvfp4_linear(const uint8_t* xc, const uint8_t* xs, float gx, const uint8_t* wc, const uint8_t* ws,
                               float gw, uint16_t* y, int M, int N, int K, bool tiled, hipStream_t stream) {
  GemmParams p = {};
  p.xc = xc; p.xs = xs; p.wc = wc; p.ws = ws; p.y = y;
  p.M = M; p.N = N; p.K = K;
  p.tiles_n = (N + GN - 1) / GN;
  const long long tiles = (long long)((M + GM - 1) / GM) * p.tiles_n;
  if (tiles <= 0 || tiles > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  p.tiles = (int)tiles;
  p.gscale = gx * gw;
  if (tiled)
    hipLaunchKernelGGL((nvfp4_gemm_kernel<TiledStaging, true>), dim3((unsigned)tiles), dim3(GT), 0, stream, p);
  else
    hipLaunchKernelGGL((nvfp4_gemm_kernel<RowsStaging, false>), dim3((unsigned)tiles), dim3(GT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace lsd
