// Attention backward for gfx950 (MI355X): dense, non-causal, d = 128, BF16.
//
// Method: the gradients of softmax attention (calculus of the forward of
// "Pika H3 Flex in FastVideo: 7x Faster, and Near Real Time in 4-bit",
// section "Faster at BF16"), needed to train through attention as the
// distillation of section "NVFP4 QAD" does.  With S = sigma Q K^T,
// P = exp(S - LSE) (LSE saved by the forward), dO the gradient of O:
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,  dS = P * (dP - D),
//   dQ = sigma dS K,  dK = sigma dS^T Q.
//
// Three launches, deterministic (no atomics):
//   bwd_rowdot  D_i = dO_i . O_i in fp32 (BF16 products are exact in fp32)
//               and LSE_i * log2(e), into the workspace.
//   bwd_dkdv    one wave per 32 keys (eight waves, two per SIMD, per
//               workgroup of 256 keys): K of its keys stays in registers and
//               the workgroup's V rows in LDS, both read as MFMA B operands;
//               32-query tiles of Q, dO and their row statistics stream
//               through LDS (double-buffered, copied by LDS-DMA loads so that
//               no registers hold the next tile).  Per tile: S and dP on
//               the 32x32x16 BF16 MFMA with the query tile as the A operand
//               (rows = queries, columns = this wave's keys), P and dS on the
//               VALU, then dV^T += dO^T P and dK^T += Q^T dS with the
//               transposed query tiles read by ds_read_b64_tr_b16 as the A
//               operand and P, dS taken from the accumulators as the B operand
//               (the accumulator layout is the operand layout up to a fixed
//               permutation of the query index, which the transpose reads
//               reproduce).
//   bwd_dq      the forward's layout: one wave per 32 queries, eight waves
//               per workgroup; Q and dO of its rows in registers, 32-key
//               tiles of K and V through LDS.  S^T = K Q^T, dP^T = V dO^T,
//               dS^T on the VALU, dQ^T += K^T dS^T.
// P and dS are rounded to BF16 for their MFMAs; all sums are fp32.  Rows past
// L are zero-filled by the buffer loads: their keys add nothing, and their
// queries meet only zero operands (bwd_dq gives them an infinite LSE).
#include "lsd_internal.h"
#include "device_common.h"

namespace lsd {
namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

constexpr float kLog2eF = 1.44269504088896340736f;
constexpr int TS = kHeadDim + 32;       // LDS row stride (bf16) of the streamed tiles: 320 B
constexpr int TR = 32;                  // rows per streamed tile
constexpr int TILE = TR * TS;           // one tile in LDS (bf16 elements)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// Memory -> LDS without registers: buffer_load_dword with the LDS flag writes
// lane j's dword to M0 + 4 j (one 256-byte row per wave instruction).  Byte
// offsets go in the per-lane offset so the range check sees them: rows past
// the end are written as zeros.  Inline assembly so that the compiler does
// not wait for these loads before reading the other LDS buffer; the caller
// waits (vmcnt 0) before the barrier that publishes the data.  M0 is written
// by SALU and read by the load one instruction later (s_nop: the M0 read
// hazard of LDS DMA).
struct Rsrc {
  u32x4 w;
};
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  Rsrc r;
  r.w[0] = (uint32_t)a;
  r.w[1] = (uint32_t)(a >> 32) & 0xFFFFu;     // stride 0
  r.w[2] = bytes;
  r.w[3] = 0x00020000u;
  return r;
}
__device__ __forceinline__ void dma_dword(const Rsrc& r, const void* lds_dst, int voff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_dst);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(r.w)
               : "m0");
}
__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// A operand from rows of a row-major LDS tile: lane l reads row l % 32,
// channels 16 * kk + 8 * (l / 32) .. +7.  `lane_row` = (l % 32) * TS + 8 * (l / 32).
__device__ __forceinline__ bf16x8 row_operand(const uint16_t* tile, int lane_row, int kk) {
  return __builtin_bit_cast(bf16x8, *(const u16x8*)(tile + lane_row + 16 * kk));
}

// A operand X^T from a row-major LDS tile X[row][channel]: rows of the
// operand are channels 32 * db .. +31, its k index runs over tile rows
// 16 * cc .. +15 in the order of the accumulator-derived B operands.
// `lane_tr` = (4 * (l / 32) + (l % 16) / 4) * TS + 16 * ((l / 16) % 2) + 4 * (l % 4).
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* tile, int lane_tr, int cc, int db) {
  const uint16_t* a0 = tile + lane_tr + 16 * cc * TS + 32 * db;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds_u16*)a0);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds_u16*)(a0 + 8 * TS));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row data of 32 consecutive rows (TR) of one head, staged through registers:
// 32 rows x 256 B = 512 chunks of 16 B.
template <int NT>
struct RowStage {
  static constexpr int N = TR * kHeadDim * 2 / 16 / NT;
  u32x4 c[N];
};

template <int NT>
__device__ __forceinline__ void load_rows(__amdgpu_buffer_rsrc_t r, int row0, int tid, RowStage<NT>& s) {
#pragma unroll
  for (int i = 0; i < RowStage<NT>::N; ++i) {
    const int id = tid + NT * i;                  // row id >> 4, chunk id & 15
    s.c[i] = __builtin_amdgcn_raw_buffer_load_b128(r, row0 * (kHeadDim * 2) + id * 16, 0, 0);
  }
}

template <int NT>
__device__ __forceinline__ void store_rows(uint16_t* tile, int tid, const RowStage<NT>& s) {
#pragma unroll
  for (int i = 0; i < RowStage<NT>::N; ++i) {
    const int id = tid + NT * i;
    *(u32x4*)(tile + (id >> 4) * TS + (id & 15) * 8) = s.c[i];
  }
}

// Lane address parts shared by the two main kernels.
struct Lanes {
  int lane, l32, hf, lane_row, lane_tr;
};

__device__ __forceinline__ Lanes lanes(int tid) {
  Lanes x;
  x.lane = tid & 63;
  x.l32 = x.lane & 31;
  x.hf = x.lane >> 5;
  const int r16 = x.lane & 15;
  x.lane_row = x.l32 * TS + 8 * x.hf;
  x.lane_tr = (4 * x.hf + (r16 >> 2)) * TS + 16 * ((x.lane >> 4) & 1) + 4 * (r16 & 3);
  return x;
}

// Logical workgroup id with each XCD (hardware id % 8) given a contiguous
// range of logical ids, so that the workgroups of one head share an L2.
__device__ __forceinline__ int xcd_logical(int bid, int nblk) {
  const int per = nblk >> 3, rem = nblk & 7;
  const int xcd = bid & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + (bid >> 3);
}

// ----------------------------------------------------------------- rowdot --

constexpr int ROWDOT_THREADS = 256;            // 16 lanes per row, 16 rows per workgroup

__global__ __launch_bounds__(ROWDOT_THREADS) void bwd_rowdot_kernel(const uint16_t* __restrict__ o,
                                                                   const uint16_t* __restrict__ dout,
                                                                   const float* __restrict__ lse,
                                                                   float* __restrict__ dsum,
                                                                   float* __restrict__ lse2, long long nrows) {
  const int tid = threadIdx.x;
  const long long row = (long long)blockIdx.x * (ROWDOT_THREADS / 16) + (tid >> 4);
  const int part = tid & 15;                    // channels 8 * part .. +7
  float acc = 0.0f;
  if (row < nrows) {
    const u32x4 a = *(const u32x4*)(o + row * kHeadDim + 8 * part);
    const u32x4 b = *(const u32x4*)(dout + row * kHeadDim + 8 * part);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = __builtin_fmaf(__uint_as_float(a[j] << 16), __uint_as_float(b[j] << 16), acc);
      acc = __builtin_fmaf(__uint_as_float(a[j] & 0xFFFF0000u), __uint_as_float(b[j] & 0xFFFF0000u), acc);
    }
  }
  // sum over the 16 lanes of the row
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) acc += __shfl_xor(acc, m, 16);
  if (row < nrows && part == 0) {
    dsum[row] = acc;
    lse2[row] = lse[row] * kLog2eF;
  }
}

// ------------------------------------------------------------------- dK dV --

constexpr int DKDV_WAVES = 8;
constexpr int DKDV_THREADS = 64 * DKDV_WAVES;
constexpr int DKDV_KEYS = 32 * DKDV_WAVES;     // keys per workgroup

struct DkdvParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* dsum;
  const float* lse2;
  uint16_t* dk;
  uint16_t* dv;
  int L;
  int n_ktiles;
  float c;                                      // softmax scale * log2(e)
  float scale;                                  // softmax scale
};

constexpr int VKS = kHeadDim + 8;       // row stride (bf16) of the stationary V rows: 272 B
struct DkdvSmem {
  uint16_t q[2][TILE];
  uint16_t dout[2][TILE];
  float lse2[2][TR];
  float dsum[2][TR];
  uint16_t v[DKDV_KEYS * VKS];          // the workgroup's V rows, read as B operands
};

__global__ __launch_bounds__(DKDV_THREADS, 1) void bwd_dkdv_kernel(DkdvParams p) {
  __shared__ __attribute__((aligned(16))) DkdvSmem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const Lanes ln = lanes(tid);

  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int h = logical / p.n_ktiles;
  const int kt = logical - h * p.n_ktiles;
  const int L = p.L;
  const size_t head_row0 = (size_t)h * (size_t)L;
  const size_t head_bytes = (size_t)L * kHeadDim * 2;
  const Rsrc rq = make_rsrc(p.q + head_row0 * kHeadDim, (uint32_t)head_bytes);
  const Rsrc rdo = make_rsrc(p.dout + head_row0 * kHeadDim, (uint32_t)head_bytes);
  const Rsrc rl = make_rsrc(p.lse2 + head_row0, (uint32_t)L * 4);
  const Rsrc rd = make_rsrc(p.dsum + head_row0, (uint32_t)L * 4);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  // This wave's 32 keys: K and V rows as B operands (8 chunks of 16 channels).
  const int key = kt * DKDV_KEYS + wave * 32 + ln.l32;
  const bool kvalid = key < L;
  bf16x8 kreg[8];
  {
    const uint16_t* kp = p.k + (head_row0 + (size_t)(kvalid ? key : 0)) * kHeadDim + 8 * ln.hf;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      kreg[kk] = __builtin_bit_cast(bf16x8, kvalid ? *(const u16x8*)(kp + 16 * kk) : (u16x8)0);
    // V rows of the workgroup's keys into LDS (zeros past L): 256 rows of 16
    // chunks, 8 per thread.
    const __amdgpu_buffer_rsrc_t rv = rsrc(p.v + head_row0 * kHeadDim, head_bytes);
    const int key0 = kt * DKDV_KEYS;
#pragma unroll
    for (int i = 0; i < DKDV_KEYS * 16 / DKDV_THREADS; ++i) {
      const int id = tid + DKDV_THREADS * i;
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rv, key0 * (kHeadDim * 2) + id * 16, 0, 0);
      *(u32x4*)(sm.v + (id >> 4) * VKS + (id & 15) * 8) = x;
    }
  }
  const int v_lane = (wave * 32 + ln.l32) * VKS + 8 * ln.hf;      // this lane's V row, channel half
  f32x16 dvacc[4], dkacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    dvacc[db] = (f32x16)0.0f;
    dkacc[db] = (f32x16)0.0f;
  }

  // Query tile q0 into LDS buffer buf: each wave copies 4 rows of Q and of
  // dO (one row per instruction), waves 0 and 1 the 32 LSE2 and D values.
  // Rows past L arrive as zeros: their Q and dO rows are zero, so their
  // probabilities (exp2(0 - 0) = 1) meet only zero operands below and their
  // dS is zero.
  auto stage = [&](int q0, int buf) {
#pragma unroll
    for (int i = 0; i < TR / DKDV_WAVES; ++i) {
      const int r = wave_u * (TR / DKDV_WAVES) + i;
      const int voff = (q0 + r) * (kHeadDim * 2) + 4 * ln.lane;
      dma_dword(rq, sm.q[buf] + r * TS, voff);
      dma_dword(rdo, sm.dout[buf] + r * TS, voff);
    }
    if (wave_u == 0 && ln.lane < TR) dma_dword(rl, sm.lse2[buf], 4 * (q0 + ln.lane));
    if (wave_u == 1 && ln.lane < TR) dma_dword(rd, sm.dsum[buf], 4 * (q0 + ln.lane));
  };

  const int ntiles = (L + TR - 1) / TR;
  stage(0, 0);
  dma_wait();
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < ntiles;
    if (more) stage((t + 1) * TR, buf ^ 1);
    const uint16_t* qt = sm.q[buf];
    const uint16_t* dt = sm.dout[buf];
    // S = Q K^T and dP = dO V^T for this wave's keys: rows = queries.
    f32x16 s = (f32x16)0.0f, dp = (f32x16)0.0f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) s = mfma(row_operand(qt, ln.lane_row, kk), kreg[kk], s);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      dp = mfma(row_operand(dt, ln.lane_row, kk), __builtin_bit_cast(bf16x8, *(const u16x8*)(sm.v + v_lane + 16 * kk)),
                dp);
    // P = exp2(S c - LSE2) and dS = P (dP - D); accumulator element i is
    // query row 8 * (i / 4) + 4 * hf + i % 4 of the tile.
    f32x8 pf[2], df[2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 l4 = *(const f32x4*)(&sm.lse2[buf][8 * g + 4 * ln.hf]);
      const f32x4 d4 = *(const f32x4*)(&sm.dsum[buf][8 * g + 4 * ln.hf]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * g + j;
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], p.c, -l4[j]));
        pf[i >> 3][i & 7] = pv;
        df[i >> 3][i & 7] = pv * (dp[i] - d4[j]);
      }
    }
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      pb[cc] = __builtin_convertvector(pf[cc], bf16x8);
      dsb[cc] = __builtin_convertvector(df[cc], bf16x8);
    }
    // dV^T += dO^T P, dK^T += Q^T dS (channel blocks db, 16-query chunks cc).
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int db = 0; db < 4; ++db) dvacc[db] = mfma(tr_operand(dt, ln.lane_tr, cc, db), pb[cc], dvacc[db]);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int db = 0; db < 4; ++db) dkacc[db] = mfma(tr_operand(qt, ln.lane_tr, cc, db), dsb[cc], dkacc[db]);

    dma_wait();
    __syncthreads();
  }

  // dK = scale * (dK^T)^T, dV = (dV^T)^T: lane l holds key l % 32 and, per
  // channel block db and group g, channels 32 db + 8 g + 4 hf .. +3.
  if (kvalid) {
    uint16_t* dkrow = p.dk + (head_row0 + key) * kHeadDim;
    uint16_t* dvrow = p.dv + (head_row0 + key) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u16x4 wk, wv;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          wk[j] = f32_to_bf16_rne(dkacc[db][4 * g + j] * p.scale);
          wv[j] = f32_to_bf16_rne(dvacc[db][4 * g + j]);
        }
        *(u16x4*)(dkrow + 32 * db + 8 * g + 4 * ln.hf) = wk;
        *(u16x4*)(dvrow + 32 * db + 8 * g + 4 * ln.hf) = wv;
      }
    }
  }
}

// ----------------------------------------------------------------------- dQ --

constexpr int DQ_WAVES = 8;
constexpr int DQ_THREADS = 64 * DQ_WAVES;
constexpr int DQ_ROWS = 32 * DQ_WAVES;         // query rows per workgroup

struct DqParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* dsum;
  const float* lse2;
  uint16_t* dq;
  int L;
  int n_qtiles;
  float c;
  float scale;
};

struct DqSmem {
  uint16_t k[2][TILE];
  uint16_t v[2][TILE];
};

__global__ __launch_bounds__(DQ_THREADS, 1) void bwd_dq_kernel(DqParams p) {
  __shared__ __attribute__((aligned(16))) DqSmem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const Lanes ln = lanes(tid);

  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int h = logical / p.n_qtiles;
  const int qt = logical - h * p.n_qtiles;
  const int L = p.L;
  const size_t head_row0 = (size_t)h * (size_t)L;
  const size_t head_bytes = (size_t)L * kHeadDim * 2;
  const __amdgpu_buffer_rsrc_t rk = rsrc(p.k + head_row0 * kHeadDim, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = rsrc(p.v + head_row0 * kHeadDim, head_bytes);

  // This wave's 32 query rows: Q and dO as B operands, LSE2 and D per lane.
  const int qrow = qt * DQ_ROWS + wave * 32 + ln.l32;
  const bool qvalid = qrow < L;
  bf16x8 qreg[8], doreg[8];
  {
    const size_t r = head_row0 + (size_t)(qvalid ? qrow : 0);
    const uint16_t* qp = p.q + r * kHeadDim + 8 * ln.hf;
    const uint16_t* dp = p.dout + r * kHeadDim + 8 * ln.hf;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      qreg[kk] = __builtin_bit_cast(bf16x8, qvalid ? *(const u16x8*)(qp + 16 * kk) : (u16x8)0);
      doreg[kk] = __builtin_bit_cast(bf16x8, qvalid ? *(const u16x8*)(dp + 16 * kk) : (u16x8)0);
    }
  }
  const float lse2 = qvalid ? p.lse2[head_row0 + qrow] : __builtin_inff();
  const float dsum = qvalid ? p.dsum[head_row0 + qrow] : 0.0f;
  f32x16 dqacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) dqacc[db] = (f32x16)0.0f;

  const int ntiles = (L + TR - 1) / TR;
  {
    RowStage<DQ_THREADS> sk, sv;
    load_rows(rk, 0, tid, sk);
    load_rows(rv, 0, tid, sv);
    store_rows(sm.k[0], tid, sk);
    store_rows(sm.v[0], tid, sv);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    RowStage<DQ_THREADS> sk, sv;
    const bool more = t + 1 < ntiles;
    if (more) {
      load_rows(rk, (t + 1) * TR, tid, sk);
      load_rows(rv, (t + 1) * TR, tid, sv);
    }
    const uint16_t* kt = sm.k[buf];
    const uint16_t* vt = sm.v[buf];
    // S^T = K Q^T and dP^T = V dO^T: rows = keys of the tile, columns = this
    // wave's queries.  Keys past L are zero rows: they add nothing below.
    f32x16 s = (f32x16)0.0f, dp = (f32x16)0.0f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) s = mfma(row_operand(kt, ln.lane_row, kk), qreg[kk], s);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) dp = mfma(row_operand(vt, ln.lane_row, kk), doreg[kk], dp);
    f32x8 df[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], p.c, -lse2));
      df[i >> 3][i & 7] = pv * (dp[i] - dsum);
    }
    bf16x8 dsb[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) dsb[cc] = __builtin_convertvector(df[cc], bf16x8);
    // dQ^T += K^T dS^T
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int db = 0; db < 4; ++db) dqacc[db] = mfma(tr_operand(kt, ln.lane_tr, cc, db), dsb[cc], dqacc[db]);

    if (more) {
      store_rows(sm.k[buf ^ 1], tid, sk);
      store_rows(sm.v[buf ^ 1], tid, sv);
    }
    __syncthreads();
  }

  if (qvalid) {
    uint16_t* row = p.dq + (head_row0 + qrow) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u16x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = f32_to_bf16_rne(dqacc[db][4 * g + j] * p.scale);
        *(u16x4*)(row + 32 * db + 8 * g + 4 * ln.hf) = w;
      }
    }
  }
}

// ------------------------------------------------- training-time FP4 QK --
//
// Gradients of the FP4-QK forward with the quantizer passed straight through
// (the usual quantization-aware-training choice; the pages train with the
// deployed FP4 attention in the loop, "NVFP4 QAD" and "FP4 attention"): the
// BF16 backward above evaluated at the dequantized Q, K (exact in BF16), then
// dQ and dK rotated back by the same orthonormal Hadamard matrix (it is
// symmetric and its own inverse).  The mean subtraction's Jacobian
// (I - 11^T / L on dK) is left out: the key-side gradient of attention sums to
// zero over keys, so it would remove only rounding.

constexpr int DEQ_THREADS = 256;               // one 16-channel block per thread

__global__ __launch_bounds__(DEQ_THREADS) void fp4_dequant_kernel(const uint8_t* __restrict__ codes,
                                                                 const uint8_t* __restrict__ scales,
                                                                 uint16_t* __restrict__ out, long long nblocks) {
  const long long i = (long long)blockIdx.x * DEQ_THREADS + threadIdx.x;
  if (i >= nblocks) return;
  const u32x2 c = *(const u32x2*)(codes + 8 * i);
  const float sc = e4m3_to_f32(scales[i]);
  *(u16x8*)(out + 16 * i) = dequant8(c[0], sc);
  *(u16x8*)(out + 16 * i + 8) = dequant8(c[1], sc);
}

constexpr int ROT_THREADS = 256;               // four lanes per row, 64 rows per workgroup
constexpr float kInvSqrt128 = 0x1.6a09e6p-4f;  // RN32(1/sqrt(128))

__device__ __forceinline__ float quad_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}

// y = x H / sqrt(128) per 128-channel BF16 row, in fp32, rounded to BF16:
// lane p of a quad holds channels 32 p .. +31; butterfly stages 0-4 in
// registers, 5-6 across the quad.
__global__ __launch_bounds__(ROT_THREADS) void rotate_rows_kernel(const uint16_t* __restrict__ in,
                                                                 uint16_t* __restrict__ out, long long nrows) {
  const int tid = threadIdx.x;
  const int part = tid & 3;
  const long long row = (long long)blockIdx.x * (ROT_THREADS / 4) + (tid >> 2);
  if (row >= nrows) return;                    // whole quads leave together
  const uint16_t* rp = in + row * kHeadDim + 32 * part;
  float x[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 w = *(const u32x4*)(rp + 8 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
      x[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int st = 0; st < 5; ++st) {
    const int hs = 1 << st;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & hs) == 0) {
        const float a = x[i], b = x[i + hs];
        x[i] = a + b;
        x[i + hs] = a - b;
      }
    }
  }
  const float k5 = (part & 1) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = __builtin_fmaf(x[i], k5, quad_xor1(x[i]));
  const float k6 = (part & 2) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = __builtin_fmaf(x[i], k6, quad_xor2(x[i]));
  uint16_t* op = out + row * kHeadDim + 32 * part;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u16x8 w;
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = f32_to_bf16_rne(x[8 * i + j] * kInvSqrt128);
    *(u16x8*)(op + 8 * i) = w;
  }
}

}  // namespace

size_t attn_bwd_workspace_bytes(int H, int L) { return (size_t)2 * H * (size_t)L * sizeof(float); }

size_t attn_bwd_fp4qk_workspace_bytes(int H, int L) {
  return (size_t)4 * H * (size_t)L * kHeadDim * 2 + attn_bwd_workspace_bytes(H, L);
}

hipError_t launch_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                           const float* lse, const uint16_t* dout, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                           void* ws, int H, int L, float scale, hipStream_t stream) {
  const long long nrows = (long long)H * L;
  float* dsum = (float*)ws;
  float* lse2 = dsum + nrows;
  const unsigned rblocks = (unsigned)((nrows + (ROWDOT_THREADS / 16) - 1) / (ROWDOT_THREADS / 16));
  hipLaunchKernelGGL(bwd_rowdot_kernel, dim3(rblocks), dim3(ROWDOT_THREADS), 0, stream, o, dout, lse, dsum, lse2,
                     nrows);

  DkdvParams a = {};
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.dsum = dsum; a.lse2 = lse2; a.dk = dk; a.dv = dv;
  a.L = L; a.n_ktiles = (L + DKDV_KEYS - 1) / DKDV_KEYS; a.c = scale * kLog2eF; a.scale = scale;
  const long long nk = (long long)a.n_ktiles * H;
  if (nk > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)nk), dim3(DKDV_THREADS), 0, stream, a);

  DqParams b = {};
  b.q = q; b.k = k; b.v = v; b.dout = dout; b.dsum = dsum; b.lse2 = lse2; b.dq = dq;
  b.L = L; b.n_qtiles = (L + DQ_ROWS - 1) / DQ_ROWS; b.c = scale * kLog2eF; b.scale = scale;
  const long long nq = (long long)b.n_qtiles * H;
  if (nq > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)nq), dim3(DQ_THREADS), 0, stream, b);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_fp4qk(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                                 const uint16_t* v, const uint16_t* o, const float* lse, const uint16_t* dout,
                                 uint16_t* dq, uint16_t* dk, uint16_t* dv, void* ws, int H, int L, float scale,
                                 bool rotate, hipStream_t stream) {
  const long long nrows = (long long)H * L;
  const size_t elems = (size_t)nrows * kHeadDim;
  uint16_t* qh = (uint16_t*)ws;                // workspace: Qh, Kh, dQh, dKh (BF16), then the row statistics
  uint16_t* kh = qh + elems;
  uint16_t* dqh = kh + elems;
  uint16_t* dkh = dqh + elems;
  void* stats = dkh + elems;
  const long long nblocks = nrows * (kHeadDim / kBlock);
  const unsigned db = (unsigned)((nblocks + DEQ_THREADS - 1) / DEQ_THREADS);
  hipLaunchKernelGGL(fp4_dequant_kernel, dim3(db), dim3(DEQ_THREADS), 0, stream, qc, qs, qh, nblocks);
  hipLaunchKernelGGL(fp4_dequant_kernel, dim3(db), dim3(DEQ_THREADS), 0, stream, kc, ks, kh, nblocks);
  hipError_t e = launch_attn_bwd(qh, kh, v, o, lse, dout, rotate ? dqh : dq, rotate ? dkh : dk, dv, stats, H, L,
                                 scale, stream);
  if (e != hipSuccess) return e;
  if (rotate) {
    const unsigned rb = (unsigned)((nrows + (ROT_THREADS / 4) - 1) / (ROT_THREADS / 4));
    hipLaunchKernelGGL(rotate_rows_kernel, dim3(rb), dim3(ROT_THREADS), 0, stream, dqh, dq, nrows);
    hipLaunchKernelGGL(rotate_rows_kernel, dim3(rb), dim3(ROT_THREADS), 0, stream, dkh, dk, nrows);
  }
  return hipGetLastError();
}

}  // namespace lsd
