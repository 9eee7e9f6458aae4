// Flash-attention forward for gfx950 (MI355X): dense, non-causal, d = 128.
//
// Method: "Pika H3 Flex in FastVideo: 7x Faster, and Near Real Time in 4-bit",
// section "Faster at BF16" (dense attention over every token of the joint
// sequence; a tiled online-softmax forward in place of a library SDPA) and
// section "FP4 attention" (scores from NVFP4 Q and K, probabilities and V kept
// in BF16).
//
// Design (one workgroup = one head x BR query rows, four 64-wide waves, each
// wave owning 32 query rows):
//   * Scores are computed transposed, S^T = K Q^T, with the 32x32x16 BF16 MFMA:
//     K (LDS) is the A operand and the wave's Q rows (registers, loaded once)
//     the B operand.  In the accumulator layout every lane then owns one query
//     row (lane % 32), so the running max, running sum and output rescale are
//     per-lane values; only the tile max is exchanged between the two lane
//     halves that share a query.
//   * O^T = V^T P^T, again with the 32x32x16 BF16 MFMA: V^T (LDS, stored
//     transposed) is the A operand; P^T comes straight from the score
//     accumulators (rounded to BF16) as the B operand, because the accumulator
//     layout of S^T is the B-operand layout of P^T up to a fixed permutation
//     of the key index, which V^T is read with.
//   * Workgroups are renumbered so that each XCD (own L2) processes a
//     contiguous range of query tiles of the same head, which therefore stream
//     the same K/V tiles at about the same time.
//   * The FP4-QK variant dequantizes each K tile (E2M1 x E4M3, exact in BF16)
//     into the same LDS layout once per workgroup, and its Q rows once, then
//     runs the identical pipeline.
#include "lsd_internal.h"
#include "device_common.h"

namespace lsd {
namespace {

constexpr int BR = 128;                 // query rows per workgroup
constexpr int BC = 64;                  // keys per tile
constexpr int NTHREADS = 256;           // 4 waves
constexpr int KROW = kHeadDim + 8;      // LDS row of a K tile (bf16): 272 B, 16 B aligned
constexpr int VROW = BC + 4;            // LDS row of a V^T tile (bf16): 136 B, 8 B aligned

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint8_t* qc;
  const uint8_t* qs;
  const uint8_t* kc;
  const uint8_t* ks;
  uint16_t* o;
  float* lse;
  int L;
  int n_qtiles;
  float scale_log2;                     // softmax scale * log2(e)
};

// 16 NVFP4 values (8 code bytes + 1 scale byte) to 16 BF16 bit patterns.
// Every product E2M1 x E4M3 has at most 6 significant bits and lies in
// [2^-10, 2688], so truncating its float32 bits to BF16 is exact.
__device__ __forceinline__ void dequant16(uint64_t codes, uint32_t scale_byte, u16x8& lo, u16x8& hi) {
  const float s = e4m3_to_f32(scale_byte);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float a = __uint_as_float(e2m1_to_f32_bits((uint32_t)(codes >> (4 * j)) & 0xF)) * s;
    const float b = __uint_as_float(e2m1_to_f32_bits((uint32_t)(codes >> (4 * (j + 8))) & 0xF)) * s;
    lo[j] = (uint16_t)(__float_as_uint(a) >> 16);
    hi[j] = (uint16_t)(__float_as_uint(b) >> 16);
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

template <bool FP4>
__global__ __launch_bounds__(NTHREADS, 2) void attn_fwd_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BC * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kHeadDim * VROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;             // which half of the wave

  // XCD-aware renumbering: hardware block b runs on XCD b % 8; give XCD x a
  // contiguous range of logical tiles (head-major), bijectively.
  const int nblk = gridDim.x;
  const int bid = blockIdx.x;
  const int per = nblk >> 3, rem = nblk & 7;
  const int xcd = bid & 7;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + (bid >> 3);
  const int h = logical / p.n_qtiles;
  const int qt = logical - h * p.n_qtiles;
  const int L = p.L;
  const size_t head_row0 = (size_t)h * (size_t)L;

  // ---- this wave's 32 query rows -> B operands (8 chunks of 16 channels) ----
  const int qrow = qt * BR + wave * 32 + l32;
  const bool qvalid = qrow < L;
  bf16x8 qreg[8];
  if constexpr (!FP4) {
    const uint16_t* qp = p.q + (head_row0 + (size_t)(qvalid ? qrow : 0)) * kHeadDim + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u16x8 t = qvalid ? *(const u16x8*)(qp + 16 * kk) : (u16x8)0;
      qreg[kk] = __builtin_bit_cast(bf16x8, t);
    }
  } else {
    const size_t r = head_row0 + (size_t)(qvalid ? qrow : 0);
    const uint8_t* cp = p.qc + r * (kHeadDim / 2);
    const uint8_t* sp = p.qs + r * (kHeadDim / kBlock);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      // channels 16kk + 8hf .. +7 live in code bytes 8kk + 4hf .. +3
      const uint32_t c4 = qvalid ? *(const uint32_t*)(cp + 8 * kk + 4 * hf) : 0u;
      const float s = e4m3_to_f32(qvalid ? sp[kk] : 0u);
      u16x8 t;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float val = __uint_as_float(e2m1_to_f32_bits((c4 >> (4 * j)) & 0xF)) * s;
        t[j] = (uint16_t)(__float_as_uint(val) >> 16);
      }
      qreg[kk] = __builtin_bit_cast(bf16x8, t);
    }
  }

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = (f32x16)0.0f;
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  const int ntiles = (L + BC - 1) / BC;
  for (int t = 0; t < ntiles; ++t) {
    const int kv0 = t * BC;
    __syncthreads();                    // everyone is done reading the previous tile

    // ---- K tile -> LDS, row-major [key][channel] ----
    if constexpr (!FP4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int id = tid + NTHREADS * i;
        const int key = id >> 4;
        const int c8 = (id & 15) * 8;
        u16x8 val = (u16x8)0;
        if (kv0 + key < L) val = *(const u16x8*)(p.k + (head_row0 + kv0 + key) * kHeadDim + c8);
        *(u16x8*)(&Ks[key * KROW + c8]) = val;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int id = tid + NTHREADS * i;
        const int key = id >> 3;
        const int b = id & 7;
        uint64_t codes = 0;
        uint32_t sb = 0;
        if (kv0 + key < L) {
          const size_t r = head_row0 + kv0 + key;
          codes = *(const uint64_t*)(p.kc + r * (kHeadDim / 2) + 8 * b);
          sb = p.ks[r * (kHeadDim / kBlock) + b];
        }
        u16x8 lo, hi;
        dequant16(codes, sb, lo, hi);
        *(u16x8*)(&Ks[key * KROW + 16 * b]) = lo;
        *(u16x8*)(&Ks[key * KROW + 16 * b + 8]) = hi;
      }
    }
    // ---- V tile -> LDS transposed [channel][key], key pairs packed ----
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = tid + NTHREADS * i;
      const int kp = id >> 4;
      const int dc = (id & 15) * 8;
      const int key0 = kv0 + 2 * kp;
      u16x8 a = (u16x8)0, b = (u16x8)0;
      if (key0 < L) a = *(const u16x8*)(p.v + (head_row0 + key0) * kHeadDim + dc);
      if (key0 + 1 < L) b = *(const u16x8*)(p.v + (head_row0 + key0 + 1) * kHeadDim + dc);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *(uint32_t*)(&Vt[(dc + j) * VROW + 2 * kp]) = (uint32_t)a[j] | ((uint32_t)b[j] << 16);
    }
    __syncthreads();

    // ---- S^T = K Q^T for 64 keys x this wave's 32 queries ----
    f32x16 s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = (f32x16)0.0f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u16x8*)(&Ks[(32 * b + l32) * KROW + 16 * kk + 8 * hf]));
        s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], s[b], 0, 0, 0);
      }
    }

    // ---- online softmax (base 2); lane holds keys 32b + 8(i/4) + 4hf + i%4 ----
    float mx = -__builtin_inff();
    const bool ragged = kv0 + BC > L;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[b][i] * p.scale_log2;
        if (ragged) {
          const int key = kv0 + 32 * b + 8 * (i >> 2) + 4 * hf + (i & 3);
          if (key >= L) x = -__builtin_inff();
        }
        s[b][i] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float rs = 0.0f;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(s[b][i] - m_new);
        s[b][i] = e;
        rs += e;
      }
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] *= alpha;

    // ---- O^T += V^T P^T, 4 chunks of 16 keys x 4 blocks of 32 channels ----
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int b = c >> 1;
      const int base = 8 * (c & 1);
      f32x8 pf;
#pragma unroll
      for (int i = 0; i < 8; ++i) pf[i] = s[b][base + i];
      const bf16x8 pb = __builtin_convertvector(pf, bf16x8);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint16_t* vrow = &Vt[(32 * db + l32) * VROW + 16 * c + 4 * hf];
        const u16x4 v0 = *(const u16x4*)(vrow);
        const u16x4 v1 = *(const u16x4*)(vrow + 8);
        const u16x8 vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pb, oacc[db], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O = O / l, BF16 round to nearest even; LSE in natural log ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (qvalid) {
    uint16_t* orow = p.o + (head_row0 + qrow) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u16x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = f32_to_bf16_rne(oacc[db][4 * g + j] * inv);
        *(u16x4*)(orow + 32 * db + 8 * g + 4 * hf) = w;
      }
    }
    if (p.lse != nullptr && hf == 0)
      p.lse[head_row0 + qrow] = (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
  }
}

hipError_t launch(const AttnParams& prm, bool fp4, int H, hipStream_t stream) {
  const long long nblk = (long long)prm.n_qtiles * H;
  if (nblk <= 0 || nblk > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  if (fp4)
    hipLaunchKernelGGL(attn_fwd_kernel<true>, dim3((unsigned)nblk), dim3(NTHREADS), 0, stream, prm);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<false>, dim3((unsigned)nblk), dim3(NTHREADS), 0, stream, prm);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                            float* lse, int H, int L, float scale_log2, hipStream_t stream) {
  AttnParams prm = {};
  prm.q = q; prm.k = k; prm.v = v; prm.o = o; prm.lse = lse;
  prm.L = L; prm.n_qtiles = (L + BR - 1) / BR; prm.scale_log2 = scale_log2;
  return launch(prm, false, H, stream);
}

hipError_t launch_attn_fp4qk(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                             const uint16_t* v, uint16_t* o, float* lse, int H, int L, float scale_log2,
                             hipStream_t stream) {
  AttnParams prm = {};
  prm.qc = qc; prm.qs = qs; prm.kc = kc; prm.ks = ks; prm.v = v; prm.o = o; prm.lse = lse;
  prm.L = L; prm.n_qtiles = (L + BR - 1) / BR; prm.scale_log2 = scale_log2;
  return launch(prm, true, H, stream);
}

}  // namespace lsd
