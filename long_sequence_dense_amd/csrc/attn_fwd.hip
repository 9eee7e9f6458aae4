// Flash-attention forward for gfx950 (MI355X): dense, non-causal, d = 128.
//
// Method: "Pika H3 Flex in FastVideo: 7x Faster, and Near Real Time in 4-bit",
// section "Faster at BF16" (dense attention over every token of the joint
// sequence; a tiled online-softmax forward in place of a library SDPA) and
// section "FP4 attention" (scores from NVFP4 Q and K, probabilities and V kept
// in BF16).
//
// One workgroup = one head x 256 query rows = eight 64-wide waves of 32 rows
// (two waves per SIMD).  Keys are processed in tiles of 64.
//   * Scores are computed transposed, S^T = K Q^T, on the 32x32x16 BF16 MFMA:
//     K (LDS) is the A operand, the wave's Q rows (registers, loaded once) the
//     B operand.  In the accumulator layout each lane owns one query row
//     (lane % 32), so the running max, sum and output rescale are per-lane
//     values; only the tile max is exchanged between the two lane halves.
//   * O^T += V^T P^T on the same MFMA: P^T comes straight from the score
//     accumulators (rounded to BF16) as the B operand - the S^T accumulator
//     layout is the P^T operand layout up to a fixed permutation of the key
//     index - and V^T is read from the row-major V tile with the gfx950 LDS
//     transpose read (ds_read_b64_tr_b16), addressed to reproduce that
//     permutation.
//   * K and V tiles are double-buffered in LDS (XOR-swizzled rows, no bank
//     conflicts for the operand reads) and prefetched through registers one
//     iteration ahead; K runs one tile ahead of V so that the QK^T MFMAs of
//     tile t+1 are in flight while the softmax of tile t runs on the VALU.
//     One barrier per tile.
//   * Softmax in base 2 with the scale folded into one FMA per score; the
//     running max is updated lazily: a row is rescaled only when its tile max
//     exceeds the max in use by more than 2^8, which changes no result (the
//     same reference max is used for numerator and denominator) and skips the
//     O rescale on almost every tile.
//   * Workgroups are renumbered so that each XCD (own L2) processes a
//     contiguous range of query tiles of one head, which then stream the same
//     K/V tiles at about the same time.
//   * The FP4-QK variant dequantizes each K tile (E2M1 x E4M3, exact in BF16)
//     into the same LDS layout, and its Q rows once, then runs the same
//     pipeline on BF16 MFMA.
#include "lsd_internal.h"
#include "device_common.h"

namespace lsd {
namespace {

constexpr int BR = 256;                 // query rows per workgroup
constexpr int BC = 64;                  // keys per tile
constexpr int NTHREADS = 512;           // 8 waves
constexpr float kLazyRescale = 8.0f;    // log2 of the growth allowed before a rescale

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

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

struct Smem {
  uint16_t k[2][BC * kHeadDim];         // [key][channel], 16-byte chunks XOR-swizzled by key & 15
  uint16_t v[2][BC * kHeadDim];         // [key][channel], 16-byte chunks XOR-swizzled by 4*(key & 3)
};

__device__ __forceinline__ int k_elem(int key, int chunk) { return key * kHeadDim + ((chunk ^ (key & 15)) << 3); }
__device__ __forceinline__ int v_elem(int key, int chunk) { return key * kHeadDim + ((chunk ^ ((key & 3) << 2)) << 3); }

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

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// Registers holding one prefetched tile slice of this thread.
struct KPrefetch {
  u16x8 c[2];          // BF16: two 16-byte chunks
  uint64_t codes;      // FP4: one 16-channel block
  uint32_t scale;
};

template <bool FP4>
__device__ __forceinline__ void load_k(const AttnParams& p, size_t head_row0, int kv0, int tid, KPrefetch& r) {
  const int L = p.L;
  if constexpr (!FP4) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = tid + NTHREADS * i;
      const int key = id >> 4, chunk = id & 15;
      r.c[i] = (kv0 + key < L) ? *(const u16x8*)(p.k + (head_row0 + kv0 + key) * kHeadDim + chunk * 8) : (u16x8)0;
    }
  } else {
    const int key = tid >> 3, b = tid & 7;
    r.codes = 0;
    r.scale = 0;
    if (kv0 + key < L) {
      const size_t row = head_row0 + kv0 + key;
      r.codes = *(const uint64_t*)(p.kc + row * (kHeadDim / 2) + 8 * b);
      r.scale = p.ks[row * (kHeadDim / kBlock) + b];
    }
  }
}

template <bool FP4>
__device__ __forceinline__ void store_k(uint16_t* kb, int tid, const KPrefetch& r) {
  if constexpr (!FP4) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = tid + NTHREADS * i;
      *(u16x8*)(kb + k_elem(id >> 4, id & 15)) = r.c[i];
    }
  } else {
    const int key = tid >> 3, b = tid & 7;
    u16x8 lo, hi;
    dequant16(r.codes, r.scale, lo, hi);
    *(u16x8*)(kb + k_elem(key, 2 * b)) = lo;
    *(u16x8*)(kb + k_elem(key, 2 * b + 1)) = hi;
  }
}

__device__ __forceinline__ void load_v(const AttnParams& p, size_t head_row0, int kv0, int tid, u16x8 (&r)[2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int id = tid + NTHREADS * i;
    const int key = id >> 4, chunk = id & 15;
    r[i] = (kv0 + key < p.L) ? *(const u16x8*)(p.v + (head_row0 + kv0 + key) * kHeadDim + chunk * 8) : (u16x8)0;
  }
}

__device__ __forceinline__ void store_v(uint16_t* vb, int tid, const u16x8 (&r)[2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int id = tid + NTHREADS * i;
    *(u16x8*)(vb + v_elem(id >> 4, id & 15)) = r[i];
  }
}

// S^T (64 keys x 32 queries) for this wave from one K tile.
__device__ __forceinline__ void qk_tile(const uint16_t* kb, const bf16x8 (&qreg)[8], int l32, int hf, f32x16 (&s)[2]) {
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    s[b] = (f32x16)0.0f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u16x8*)(kb + k_elem(32 * b + l32, 2 * kk + hf)));
      s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], s[b], 0, 0, 0);
    }
  }
}

template <bool FP4>
__global__ __launch_bounds__(NTHREADS, 1) void attn_fwd_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;             // which half of the wave
  const int grp = lane >> 4;            // 16-lane group (transpose reads)
  const int r16 = lane & 15;

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

  const int ntiles = (L + BC - 1) / BC;

  // ---- prologue: K(0), V(0), K(1) into LDS; S(0) ----
  {
    KPrefetch kr;
    u16x8 vr[2];
    load_k<FP4>(p, head_row0, 0, tid, kr);
    load_v(p, head_row0, 0, tid, vr);
    store_k<FP4>(sm.k[0], tid, kr);
    store_v(sm.v[0], tid, vr);
    if (ntiles > 1) {
      load_k<FP4>(p, head_row0, BC, tid, kr);
      store_k<FP4>(sm.k[1], tid, kr);
    }
  }
  __syncthreads();

  f32x16 s_cur[2], s_nxt[2];
  qk_tile(sm.k[0], qreg, l32, hf, s_cur);
  __syncthreads();                      // K(0)'s buffer is overwritten with K(2) in the first iteration

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = (f32x16)0.0f;
  float m_used = -__builtin_inff();     // reference max (base-2 scaled units) of this lane's row
  float l_run = 0.0f;                   // this lane's partial row sum (its half of the keys)
  const float c = p.scale_log2;

  for (int t = 0; t < ntiles; ++t) {
    const bool has_next = t + 1 < ntiles;
    const bool has_next2 = t + 2 < ntiles;
    // prefetch V(t+1) and K(t+2) into registers
    KPrefetch kr;
    u16x8 vr[2];
    if (has_next) load_v(p, head_row0, (t + 1) * BC, tid, vr);
    if (has_next2) load_k<FP4>(p, head_row0, (t + 2) * BC, tid, kr);

    // S(t+1) on the matrix cores while the softmax of tile t runs
    if (has_next) qk_tile(sm.k[(t + 1) & 1], qreg, l32, hf, s_nxt);

    // ---- softmax of tile t; lane holds keys 32b + 8(i/4) + 4hf + i%4 ----
    const int kv0 = t * BC;
    if (kv0 + BC > L) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kv0 + 32 * b + 8 * (i >> 2) + 4 * hf + (i & 3) >= L) s_cur[b][i] = -__builtin_inff();
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = __builtin_fmaxf(mx, __builtin_fmaxf(s_cur[b][i], s_cur[b][i + 1]));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
    const float mz = mx * c;
    if (__builtin_amdgcn_ballot_w64(mz > m_used + kLazyRescale)) {
      const float m_new = __builtin_fmaxf(m_used, mz);
      const float alpha = __builtin_amdgcn_exp2f(m_used - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
      m_used = m_new;
    }
    const float negm = -m_used;
    bf16x8 pb[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      f32x8 pf;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[cc >> 1][8 * (cc & 1) + i], c, negm));
        pf[i] = e;
        l_run += e;
      }
      pb[cc] = __builtin_convertvector(pf, bf16x8);
    }

    // ---- O^T += V^T P^T: 4 chunks of 16 keys x 4 blocks of 32 channels ----
    const uint16_t* vb = sm.v[t & 1];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int key0 = 16 * cc + 4 * hf + (r16 >> 2);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int ch = 32 * db + 16 * (grp & 1) + 4 * (r16 & 3);
        const int e0 = v_elem(key0, ch >> 3) + (ch & 7);
        const int e1 = v_elem(key0 + 8, ch >> 3) + (ch & 7);
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)((lds_u16*)vb + e0));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)((lds_u16*)vb + e1));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[cc], oacc[db], 0, 0, 0);
      }
    }

    // ---- stage the prefetched tiles, then one barrier ----
    if (has_next) store_v(sm.v[(t + 1) & 1], tid, vr);
    if (has_next2) store_k<FP4>(sm.k[t & 1], tid, kr);
    __syncthreads();
    if (has_next) {
      s_cur[0] = s_nxt[0];
      s_cur[1] = s_nxt[1];
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
      p.lse[head_row0 + qrow] = (m_used + __log2f(l_tot)) * 0.69314718055994530942f;
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
