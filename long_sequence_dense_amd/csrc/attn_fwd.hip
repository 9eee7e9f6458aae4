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
//   * Software pipeline, per iteration t: the MFMAs of P(t-1) V(t-1) are
//     issued in fenced slots, each followed by two exponentials of tile t
//     and by the V reads of the MFMA four slots later, so the matrix core and
//     the vector ALU work at the same time inside each wave and no MFMA waits
//     on a fresh LDS read; then K(t+1) Q^T.  K runs two tiles ahead of the
//     P.V stage, V one tile.
//   * K and V tiles are double-buffered in LDS with padded rows (bank-conflict
//     free operand reads at immediate offsets) and prefetched through
//     registers one iteration ahead.  One barrier per tile.
//   * Softmax in base 2 with the scale folded into one FMA per score.  The
//     exponentials of a tile are taken against the reference max already in
//     use, without computing the tile max first; only when a lane's tile sum
//     exceeds 2^16 (or overflows, as on the first tile) does the wave compute
//     the true tile max, rescale its running sum and O, and redo the
//     exponentials.  Any reference max gives the same result (numerator and
//     denominator share it); the bound keeps P, the sums and O far from
//     overflow, and the rare path is taken on a few tiles per row.
//   * Workgroups are renumbered so that each XCD (own L2) processes a
//     contiguous range of query tiles of one head, which then stream the same
//     K/V tiles at about the same time.
//   * The FP4-QK variant dequantizes each K tile into the same LDS layout,
//     and its Q rows once, to FP16 (E2M1 x E4M3 products have at most 6
//     significant bits in [2^-10, 2688]: exact; the hardware FP4-to-FP16
//     pair conversion and one packed FP16 multiply per pair), then runs the
//     same pipeline with the score MFMAs in their FP16 form (same rate, same
//     exact products and fp32 sums as BF16 operands would give; P.V stays
//     BF16).  Its fused-Q form takes Q in BF16 and applies
//     the prep's rotation and quantizer to each wave's rows in the prologue
//     (the same fp32 operations in the same order, so the same codes), then
//     dequantizes them in registers: Q's codes never go through memory.
#include "lsd_internal.h"
#include "device_common.h"
#include "nvfp4_quant.h"

namespace lsd {
namespace {

#ifndef LSD_ATTN_WAVES
#define LSD_ATTN_WAVES 8
#endif
constexpr int NWAVES = LSD_ATTN_WAVES;  // waves per workgroup, 32 query rows each
constexpr int BR = 32 * NWAVES;         // query rows per workgroup
constexpr int BC = 64;                  // keys per tile
constexpr int NTHREADS = 64 * NWAVES;
constexpr int KCHUNKS = BC * kHeadDim * 2 / 16;   // 16-byte chunks per BF16 tile
constexpr int NLD = KCHUNKS / NTHREADS;            // chunks per thread per tile
constexpr int NLD4 = BC * (kHeadDim / kBlock) / NTHREADS;   // FP4 blocks per thread per tile
constexpr int KS = kHeadDim + 8;        // K row stride in LDS (bf16): 272 B
constexpr int VS = kHeadDim + 32;       // V row stride in LDS (bf16): 320 B
constexpr float kSumBound = 65536.0f;   // largest per-lane tile sum accepted without recomputing the max
#ifndef LSD_ATTN_KPRE
#define LSD_ATTN_KPRE 4
#endif
constexpr int KPRE = LSD_ATTN_KPRE;     // K operands of the next tile read during the P.V half

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
  float* o32;                           // training outputs (both or neither): O in fp32,
  float* ml;                            // and per row the reference max m and the sum l
  int L;
  int n_qtiles;
  float scale_log2;                     // softmax scale * log2(e)
};

struct Smem {
  uint16_t k[2][BC * KS];
  uint16_t v[2][BC * VS];
};

// 16 NVFP4 values (8 code bytes + 1 scale byte) to 16 FP16 bit patterns.
__device__ __forceinline__ void dequant16(uint64_t codes, uint32_t scale_byte, u16x8& lo, u16x8& hi) {
  const _Float16 s = e4m3_to_f16(scale_byte);
  lo = dequant8_h((uint32_t)codes, s);
  hi = dequant8_h((uint32_t)(codes >> 32), s);
}

// Score MFMA: BF16 operands, or (FP4-QK) the exactly dequantized FP16 ones.
template <bool F16>
__device__ __forceinline__ f32x16 score_mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h16x8, a), __builtin_bit_cast(h16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// Raw buffer resources over one head's rows: loads past the end of the head
// return zeros (hardware range check), so ragged last tiles need no branches.
struct HeadBufs {
  __amdgpu_buffer_rsrc_t k, v, kc, ks;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One thread's share of a prefetched K tile.
struct KPrefetch {
  u32x4 c[NLD];        // BF16: 16-byte chunks
  u32x2 codes[NLD4];   // FP4: 16-channel blocks
  uint32_t scale[NLD4];
};

template <bool FP4>
__device__ __forceinline__ void load_k(const HeadBufs& hb, int kv0, int tid, KPrefetch& r) {
  if constexpr (!FP4) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int id = tid + NTHREADS * i;          // key id >> 4, 16-byte chunk id & 15
      r.c[i] = __builtin_amdgcn_raw_buffer_load_b128(hb.k, id * 16, kv0 * (kHeadDim * 2), 0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NLD4; ++i) {
      // key id >> 3, block id & 7: 8 code bytes and 1 scale byte
      const int id = tid + NTHREADS * i;
      r.codes[i] = __builtin_amdgcn_raw_buffer_load_b64(hb.kc, id * 8, kv0 * (kHeadDim / 2), 0);
      r.scale[i] = __builtin_amdgcn_raw_buffer_load_b8(hb.ks, id, kv0 * (kHeadDim / kBlock), 0);
    }
  }
}

template <bool FP4>
__device__ __forceinline__ void store_k(uint16_t* kb, int tid, const KPrefetch& r) {
  if constexpr (!FP4) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int id = tid + NTHREADS * i;
      *(u32x4*)(kb + (id >> 4) * KS + (id & 15) * 8) = r.c[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < NLD4; ++i) {
      const int id = tid + NTHREADS * i;
      const int key = id >> 3, b = id & 7;
      u16x8 lo, hi;
      dequant16(((uint64_t)r.codes[i][1] << 32) | r.codes[i][0], r.scale[i] & 0xFF, lo, hi);
      *(u16x8*)(kb + key * KS + 16 * b) = lo;
      *(u16x8*)(kb + key * KS + 16 * b + 8) = hi;
    }
  }
}

__device__ __forceinline__ void load_v(const HeadBufs& hb, int kv0, int tid, u32x4 (&r)[NLD]) {
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int id = tid + NTHREADS * i;
    r[i] = __builtin_amdgcn_raw_buffer_load_b128(hb.v, id * 16, kv0 * (kHeadDim * 2), 0);
  }
}

__device__ __forceinline__ void store_v(uint16_t* vb, int tid, const u32x4 (&r)[NLD]) {
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int id = tid + NTHREADS * i;
    *(u32x4*)(vb + (id >> 4) * VS + (id & 15) * 8) = r[i];
  }
}

// S^T (64 keys x 32 queries) of this wave from one K tile.  kl points at
// this lane's row (lane % 32) and channel half (8 * (lane / 32)).
__device__ __forceinline__ bf16x8 k_operand(const uint16_t* kl, int i) {   // i = 8 * block + chunk
  return __builtin_bit_cast(bf16x8, *(const u16x8*)(kl + 32 * (i >> 3) * KS + 16 * (i & 7)));
}

// The first KPRE operands come from registers read earlier (kpre).
template <int NPRE, bool F16 = false>
__device__ __forceinline__ void qk_tile(const uint16_t* kl, const bf16x8 (&kpre)[KPRE], const bf16x8 (&qreg)[8],
                                        f32x16 (&s)[2]) {
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    s[b] = (f32x16)0.0f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int i = 8 * b + kk;
      const bf16x8 a = i < NPRE ? kpre[i < KPRE ? i : 0] : k_operand(kl, i);
      s[b] = score_mfma<F16>(a, qreg[kk], s[b]);
    }
  }
}

// O^T += V^T P^T for one tile.  vl points at this lane's transpose-read
// address for key chunk 0 and channel block 0: key 4*(lane/32) + (lane%16)/4,
// channel 16*((lane/16)%2) + 4*(lane%4).
__device__ __forceinline__ void pv_tile(const uint16_t* vl, const bf16x8 (&pb)[4], f32x16 (&oacc)[4]) {
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const uint16_t* a0 = vl + 16 * cc * VS + 32 * db;
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds_u16*)a0);
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds_u16*)(a0 + 8 * VS));
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[cc], oacc[db], 0, 0, 0);
    }
  }
}

// Per-wave running state of the pipeline.
struct WaveState {
  bf16x8 qreg[8];                       // Q rows as B operands (8 chunks of 16 channels)
  f32x16 s[2];                          // S^T of the tile being softmaxed (then of the next tile)
  f32x16 oacc[4];                       // O^T accumulators, 4 blocks of 32 channels
  bf16x8 p_prev[4];                     // P^T of the previous tile (B operands)
  float m_used;                         // reference max (base-2 scaled units) of this lane's row
  float l_run;                          // this lane's partial row sum (its half of the keys)
  float alpha;                          // pending O rescale factor (1 = none)
  bool rescale;                         // wave-uniform: an O rescale is pending
};

struct Ctx {
  HeadBufs hb;
  int tid, hf, k_lane, v_lane, L;
  float c;                              // softmax scale * log2(e)
};

// Masks for the scheduling groups: VALU 0x2, MFMA 0x8, VMEM read 0x20,
// DS read 0x100, DS write 0x200.  The score MFMAs start with KPRE operands
// in registers (read during the P.V half) and keep reading KPRE ahead.
__device__ __forceinline__ void schedule_qk_half() {
  if (KPRE < 4) __builtin_amdgcn_sched_group_barrier(0x100, 4 - KPRE, 0);
  constexpr int AHEAD = KPRE < 4 ? 4 : KPRE;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i + AHEAD < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
  }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Exponentials of the tile against the reference max in use, their BF16
// operands and the lane's partial sum.  The sum is taken over the BF16-rounded
// values that P.V multiplies (two per dot instruction, fp32 accumulation), so
// numerator and denominator carry the same weights: a row whose weight sits on
// one key returns that key's V row exactly, up to the output's rounding.
__device__ __forceinline__ float exp_tile(const f32x16 (&s)[2], float c, float negm, bf16x8 (&p)[4]) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float lsum = 0.0f;
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    f32x8 pf;
#pragma unroll
    for (int i = 0; i < 8; ++i) pf[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[cc >> 1][8 * (cc & 1) + i], c, negm));
    p[cc] = __builtin_convertvector(pf, bf16x8);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[cc][2 * j], p[cc][2 * j + 1]}, ones, lsum, false);
  }
  return lsum;
}

// The first half of a pipeline iteration as 16 fenced slots: slot i issues
// the V transpose reads of P.V MFMA i + 4, the MFMA i (channel block i % 4,
// key chunk i / 4), and two of the tile's exponentials; every fourth slot
// rounds the eight exponentials just taken to BF16 and adds them to the row
// sum.  The exponentials, their rounding and the order of the sum are those
// of exp_tile.  With the operands read four MFMAs ahead, no MFMA waits on a
// fresh LDS read, and the VALU work issues while the matrix core runs.  The
// last four slots also read the first KPRE K operands of the next tile.
template <bool KP>
__device__ __forceinline__ float pv_exp_tile(const uint16_t* vl, const bf16x8 (&pb)[4], f32x16 (&oacc)[4],
                                             const f32x16 (&s)[2], float c, float negm, bf16x8 (&p)[4],
                                             const uint16_t* kl, bf16x8 (&kpre)[KPRE]) {
  constexpr int AHEAD = 4;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  bf16x8 va[16];
  auto vread = [&](int i) {
    const uint16_t* a0 = vl + 16 * (i >> 2) * VS + 32 * (i & 3);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds_u16*)a0);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds_u16*)(a0 + 8 * VS));
    va[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) vread(i);
  __builtin_amdgcn_sched_barrier(0);
  float lsum = 0.0f;
  f32x8 pf;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i + AHEAD < 16) vread(i + AHEAD);
    if constexpr (KP) {
      if (i >= 16 - KPRE) kpre[i - (16 - KPRE)] = k_operand(kl, i - (16 - KPRE));
    }
    oacc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pb[i >> 2], oacc[i & 3], 0, 0, 0);
    const int g = i >> 2;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int k = 2 * (i & 3) + e;
      pf[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[g >> 1][8 * (g & 1) + k], c, negm));
    }
    if ((i & 3) == 3) {
      p[g] = __builtin_convertvector(pf, bf16x8);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[g][2 * j], p[g][2 * j + 1]}, ones, lsum, false);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  return lsum;
}

// The second half of a pipeline iteration as 16 fenced slots: slot j issues
// the K read of score MFMA j + KPRE and the score MFMA j (key block j / 8,
// channel chunk j % 8), the first KPRE operands coming from kpre; with STORE
// the slots also stage K(t+2) into LDS (its global loads were issued at the
// start of the iteration): the exact dequantization of this thread's FP4
// 16-value block, one pair of values per slot in slots 0-7, its two 16-byte
// stores in slots 8 and 9 (otherwise a VALU-only stretch after the score
// MFMAs).  The arithmetic and the store addresses are those of store_k.
template <bool FP4, bool STORE>
__device__ __forceinline__ void qk_stage_tile(const uint16_t* kl, const bf16x8 (&kpre)[KPRE], const bf16x8 (&qreg)[8],
                                              f32x16 (&s)[2], uint16_t* kb, int tid, const KPrefetch& kr) {
  static_assert(FP4 && NLD4 == 1, "FP4 staging: one 16-value block of K per thread and tile");
  bf16x8 ka[16];
#pragma unroll
  for (int i = 0; i < KPRE; ++i) ka[i] = kpre[i];
  s[0] = (f32x16)0.0f;
  s[1] = (f32x16)0.0f;
  u32x4 hw[2];
  h16x2 s2 = {(_Float16)0.0f, (_Float16)0.0f};
  if constexpr (FP4 && STORE) {
    const _Float16 sc = e4m3_to_f16(kr.scale[0] & 0xFF);
    s2 = h16x2{sc, sc};
  }
  const int key = tid >> 3, blk = tid & 7;       // FP4 staging: this thread's block
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j + KPRE < 16) ka[j + KPRE] = k_operand(kl, j + KPRE);
    s[j >> 3] = score_mfma<true>(ka[j], qreg[j & 7], s[j >> 3]);
    if constexpr (STORE) {
      if constexpr (FP4) {
        if (j < 8) {
          const uint32_t w = kr.codes[0][j >> 2];
          uint32_t v = 0;
          switch (j & 3) {                       // the byte select must be a constant
            case 0: v = fp4_pair_h<0>(w, s2); break;
            case 1: v = fp4_pair_h<1>(w, s2); break;
            case 2: v = fp4_pair_h<2>(w, s2); break;
            default: v = fp4_pair_h<3>(w, s2); break;
          }
          hw[j >> 2][j & 3] = v;
        } else if (j < 10) {
          const int h = j - 8;
          *(u32x4*)(kb + key * KS + 16 * blk + 8 * h) = hw[h];
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One pipeline iteration t.  First half: P(t-1) V(t-1) on the matrix cores
// while the VALU exponentiates tile t (pv_exp_tile).  Second half:
// S(t+1) = K(t+1) Q^T on the matrix cores, into the registers the
// exponentials just freed; then V(t) and K(t+2) are staged into LDS.
template <bool FP4, bool FIRST, bool NEXT, bool NEXT2, bool LAST>
__device__ __forceinline__ void step(Smem& sm, WaveState& st, const Ctx& cx, int t) {
  const int kv0 = t * BC;
  if (st.rescale) {                     // P(t-2) V(t-2) has accumulated; P(t-1) used the new max
#pragma unroll
    for (int db = 0; db < 4; ++db) st.oacc[db] *= st.alpha;
  }
  KPrefetch kr;
  u32x4 vr[NLD];
  load_v(cx.hb, kv0, cx.tid, vr);
  if constexpr (NEXT2) load_k<FP4>(cx.hb, kv0 + 2 * BC, cx.tid, kr);

  // ---- first half ----
  if constexpr (LAST) {
    if (kv0 + BC > cx.L) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kv0 + 32 * b + 8 * (i >> 2) + 4 * cx.hf + (i & 3) >= cx.L) st.s[b][i] = -__builtin_inff();
    }
  }
  // Exponentials against the reference max in use; a tile whose partial
  // sum could overflow (above 2^16, infinite on the first tile) is redone
  // below against its true max.
  bf16x8 p_cur[4];
  bf16x8 kpre[KPRE];
  float lsum;
  if constexpr (!FIRST) {
    lsum = pv_exp_tile<NEXT>(sm.v[(t - 1) & 1] + cx.v_lane, st.p_prev, st.oacc, st.s, cx.c, -st.m_used, p_cur,
                             sm.k[(t + 1) & 1] + cx.k_lane, kpre);
  } else {
    lsum = exp_tile(st.s, cx.c, -st.m_used, p_cur);
    if constexpr (NEXT) {
#pragma unroll
      for (int i = 0; i < KPRE; ++i) kpre[i] = k_operand(sm.k[(t + 1) & 1] + cx.k_lane, i);
    }
  }

  // ---- rare path: recompute the tile against its true max ----
  st.rescale = __builtin_amdgcn_ballot_w64(!(lsum <= kSumBound)) != 0;
  if (st.rescale) {
    float mx = -__builtin_inff();
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, st.s[b][i]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(mx), __float_as_int(mx), false, false);
    mx = __builtin_fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1]));
    const float m_new = __builtin_fmaxf(st.m_used, mx * cx.c);
    st.alpha = __builtin_amdgcn_exp2f(st.m_used - m_new);
    st.l_run *= st.alpha;
    st.m_used = m_new;
    lsum = exp_tile(st.s, cx.c, -m_new, p_cur);
  }
  st.l_run += lsum;

  // ---- second half ----
  // (K(t+2) goes to K(t)'s buffer: no wave reads K(t) after the last
  // barrier).  The FP4 path dequantizes it in the score slots; the BF16 path
  // stores it after them.
  if constexpr (NEXT && FP4) {
    qk_stage_tile<true, NEXT2>(sm.k[(t + 1) & 1] + cx.k_lane, kpre, st.qreg, st.s, sm.k[t & 1], cx.tid, kr);
  } else if constexpr (NEXT) {
    qk_tile<KPRE>(sm.k[(t + 1) & 1] + cx.k_lane, kpre, st.qreg, st.s);
    schedule_qk_half();
  }

  // ---- stage the prefetched tiles, then one barrier ----
  store_v(sm.v[t & 1], cx.tid, vr);
  if constexpr (NEXT2 && !FP4) store_k<false>(sm.k[t & 1], cx.tid, kr);
  __syncthreads();
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) st.p_prev[cc] = p_cur[cc];
}

// Q of this lane's query row through the prep's transform and quantizer,
// dequantized exactly: the Sylvester butterfly in fp32 (stage s pairs channel
// i with i + 2^s as (x_i + x_j, x_i - x_j), stages in order 0..6), times
// RN32(1/sqrt(128)), then per 16-channel block the E4M3 scale and E2M1 codes
// of the prep.  Lane (row, hf) holds channels 16 kk + 8 hf + j (kk, j = 0..7):
// channel bits 0-2 are j, bit 3 is hf (the partner lane, lane ^ 32), bits 4-6
// are kk.  Each block is split over the lane pair; its maximum is exchanged.
__device__ __forceinline__ void quant_dequant_q(const uint16_t* qp, bool valid, int hf, bf16x8 (&qreg)[8]) {
#pragma clang fp contract(off)
  float x[8][8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const u16x8 t = valid ? *(const u16x8*)(qp + 16 * kk) : (u16x8)0;
#pragma unroll
    for (int j = 0; j < 8; ++j) x[kk][j] = bf16_bits_to_f32(t[j]);
  }
#pragma unroll
  for (int st = 0; st < 3; ++st) {                 // stages 0-2: within j
    const int hs = 1 << st;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if ((j & hs) == 0) {
          const float a = x[kk][j], b = x[kk][j + hs];
          x[kk][j] = a + b;
          x[kk][j + hs] = a - b;
        }
  }
  // stage 3 across the lane pair: the lane with bit 3 clear forms x_i + x_j,
  // its partner x_i - x_j, each one rounded operation fma(own, +-1, partner)
  const float k3 = hf ? -1.0f : 1.0f;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
#pragma unroll
    for (int j = 0; j < 8; ++j) x[kk][j] = __builtin_fmaf(x[kk][j], k3, __shfl_xor(x[kk][j], 32));
#pragma unroll
  for (int st = 0; st < 3; ++st) {                 // stages 4-6: within kk
    const int hs = 1 << st;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      if ((kk & hs) == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float a = x[kk][j], b = x[kk + hs][j];
          x[kk][j] = a + b;
          x[kk + hs][j] = a - b;
        }
      }
  }
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[kk][j] = x[kk][j] * kHadamardScale;
      am = __builtin_fmaxf(am, __builtin_fabsf(x[kk][j]));
    }
    am = __builtin_fmaxf(am, __shfl_xor(am, 32));
    const uint32_t sc = e4m3_scale_code(am);
    const float s = e4m3_pos(sc);
    const float rinv = scale_reciprocal(sc, s);
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = div_scale(x[kk][j], s, rinv);
    qreg[kk] = __builtin_bit_cast(bf16x8, dequant8_h(e2m1_pack8(t), e4m3_to_f16(sc)));
  }
}

template <bool FP4, bool QUANT_Q>
__global__ __launch_bounds__(NTHREADS, 1) void attn_fwd_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;             // which half of the wave
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

  Ctx cx;
  if constexpr (!FP4) {
    cx.hb.k = head_rsrc(p.k + head_row0 * kHeadDim, (size_t)L * kHeadDim * 2);
  } else {
    cx.hb.kc = head_rsrc(p.kc + head_row0 * (kHeadDim / 2), (size_t)L * (kHeadDim / 2));
    cx.hb.ks = head_rsrc(p.ks + head_row0 * (kHeadDim / kBlock), (size_t)L * (kHeadDim / kBlock));
  }
  cx.hb.v = head_rsrc(p.v + head_row0 * kHeadDim, (size_t)L * kHeadDim * 2);
  cx.tid = tid;
  cx.hf = hf;
  cx.L = L;
  cx.k_lane = l32 * KS + 8 * hf;                                                     // qk_tile operand
  cx.v_lane = (4 * hf + (r16 >> 2)) * VS + 16 * ((lane >> 4) & 1) + 4 * (r16 & 3);   // pv_tile operand
  cx.c = p.scale_log2;

  WaveState st;
  // ---- this wave's 32 query rows -> B operands (8 chunks of 16 channels) ----
  const int qrow = qt * BR + wave * 32 + l32;
  const bool qvalid = qrow < L;
  if constexpr (!FP4) {
    const uint16_t* qp = p.q + (head_row0 + (size_t)(qvalid ? qrow : 0)) * kHeadDim + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u16x8 t = qvalid ? *(const u16x8*)(qp + 16 * kk) : (u16x8)0;
      st.qreg[kk] = __builtin_bit_cast(bf16x8, t);
    }
  } else if constexpr (QUANT_Q) {
    quant_dequant_q(p.q + (head_row0 + (size_t)(qvalid ? qrow : 0)) * kHeadDim + 8 * hf, qvalid, hf, st.qreg);
  } else {
    const size_t r = head_row0 + (size_t)(qvalid ? qrow : 0);
    const uint8_t* cp = p.qc + r * (kHeadDim / 2);
    const uint8_t* sp = p.qs + r * (kHeadDim / kBlock);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      // channels 16kk + 8hf .. +7 live in code bytes 8kk + 4hf .. +3
      const uint32_t c4 = qvalid ? *(const uint32_t*)(cp + 8 * kk + 4 * hf) : 0u;
      const _Float16 s = e4m3_to_f16(qvalid ? sp[kk] : 0u);
      st.qreg[kk] = __builtin_bit_cast(bf16x8, dequant8_h(c4, s));
    }
  }

  const int ntiles = (L + BC - 1) / BC;

  // ---- prologue: K(0), K(1) into LDS; S(0) ----
  {
    KPrefetch kr;
    load_k<FP4>(cx.hb, 0, tid, kr);
    store_k<FP4>(sm.k[0], tid, kr);
    load_k<FP4>(cx.hb, BC, tid, kr);    // zeros when there is no second tile
    store_k<FP4>(sm.k[1], tid, kr);
  }
  __syncthreads();
  {
    bf16x8 none[KPRE];
    qk_tile<0, FP4>(sm.k[0] + cx.k_lane, none, st.qreg, st.s);
  }
  __syncthreads();                      // K(0)'s buffer is refilled with K(2) in the first iteration

#pragma unroll
  for (int db = 0; db < 4; ++db) st.oacc[db] = (f32x16)0.0f;
  st.m_used = -3.402823466e38f;        // finite: the first tile overflows the sum bound and sets the max
  st.l_run = 0.0f;
  st.alpha = 1.0f;
  st.rescale = false;

  if (ntiles == 1) {
    step<FP4, true, false, false, true>(sm, st, cx, 0);
  } else if (ntiles == 2) {
    step<FP4, true, true, false, false>(sm, st, cx, 0);
    step<FP4, false, false, false, true>(sm, st, cx, 1);
  } else {
    step<FP4, true, true, true, false>(sm, st, cx, 0);
    for (int t = 1; t < ntiles - 2; ++t) step<FP4, false, true, true, false>(sm, st, cx, t);
    step<FP4, false, true, false, false>(sm, st, cx, ntiles - 2);
    step<FP4, false, false, false, true>(sm, st, cx, ntiles - 1);
  }
  if (st.rescale) {
#pragma unroll
    for (int db = 0; db < 4; ++db) st.oacc[db] *= st.alpha;
  }
  pv_tile(sm.v[(ntiles - 1) & 1] + cx.v_lane, st.p_prev, st.oacc);

  // ---- epilogue: O = O / l, BF16 round to nearest even; LSE in natural log ----
  float l_tot;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(st.l_run), __float_as_int(st.l_run), false, false);
    l_tot = __int_as_float(sw[0]) + __int_as_float(sw[1]);
  }
  const float inv = 1.0f / l_tot;
  if (qvalid) {
    uint16_t* orow = p.o + (head_row0 + qrow) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u16x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = f32_to_bf16_rne(st.oacc[db][4 * g + j] * inv);
        *(u16x4*)(orow + 32 * db + 8 * g + 4 * hf) = w;
      }
    }
    if (p.lse != nullptr && hf == 0)
      p.lse[head_row0 + qrow] = (st.m_used + __log2f(l_tot)) * 0.69314718055994530942f;
    if (p.o32 != nullptr) {
      // The fp32 quotients that were rounded to O above, and the row's
      // (m, l): P_ij = exp2(s_ij c - m) / l reproduces the weights without an
      // fp32 log-sum-exp (whose rounding near m ~ 1e5 would shift every P).
      float* orow32 = p.o32 + (head_row0 + qrow) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = st.oacc[db][4 * g + j] * inv;
          *(f32x4*)(orow32 + 32 * db + 8 * g + 4 * hf) = w;
        }
      if (hf == 0) *(float2*)(p.ml + 2 * (head_row0 + qrow)) = make_float2(st.m_used, l_tot);
    }
  }
}

hipError_t launch(const AttnParams& prm, bool fp4, bool quant_q, int H, hipStream_t stream) {
  const long long nblk = (long long)prm.n_qtiles * H;
  if (nblk <= 0 || nblk > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  if (quant_q)
    hipLaunchKernelGGL((attn_fwd_kernel<true, true>), dim3((unsigned)nblk), dim3(NTHREADS), 0, stream, prm);
  else if (fp4)
    hipLaunchKernelGGL((attn_fwd_kernel<true, false>), dim3((unsigned)nblk), dim3(NTHREADS), 0, stream, prm);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<false, false>), dim3((unsigned)nblk), dim3(NTHREADS), 0, stream, prm);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                            float* lse, float* o32, float* ml, int H, int L, float scale_log2, hipStream_t stream) {
  AttnParams prm = {};
  prm.q = q; prm.k = k; prm.v = v; prm.o = o; prm.lse = lse; prm.o32 = o32; prm.ml = ml;
  prm.L = L; prm.n_qtiles = (L + BR - 1) / BR; prm.scale_log2 = scale_log2;
  return launch(prm, false, false, H, stream);
}

hipError_t launch_attn_fp4qk(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                             const uint16_t* v, uint16_t* o, float* lse, float* o32, float* ml, int H, int L,
                             float scale_log2, hipStream_t stream) {
  AttnParams prm = {};
  prm.qc = qc; prm.qs = qs; prm.kc = kc; prm.ks = ks; prm.v = v; prm.o = o; prm.lse = lse; prm.o32 = o32; prm.ml = ml;
  prm.L = L; prm.n_qtiles = (L + BR - 1) / BR; prm.scale_log2 = scale_log2;
  return launch(prm, true, false, H, stream);
}

hipError_t launch_attn_fp4qk_fused_q(const uint16_t* q, const uint8_t* kc, const uint8_t* ks, const uint16_t* v,
                                     uint16_t* o, float* lse, int H, int L, float scale_log2, hipStream_t stream) {
  AttnParams prm = {};
  prm.q = q; prm.kc = kc; prm.ks = ks; prm.v = v; prm.o = o; prm.lse = lse;
  prm.L = L; prm.n_qtiles = (L + BR - 1) / BR; prm.scale_log2 = scale_log2;
  return launch(prm, true, true, H, stream);
}

}  // namespace lsd
