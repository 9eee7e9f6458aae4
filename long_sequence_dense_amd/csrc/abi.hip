// C ABI of liblsd_attn.so: host-side argument checks, then the launches.
// The declarations, argument meanings, layouts and error behaviour are in
// include/lsd_attn.h.
#include <cmath>
#include <climits>

#include "../../include/lsd_attn.h"
#include "lsd_internal.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(int H, int L, int d) {
  if (d != lsd::kHeadDim) return LSD_ERR_UNSUPPORTED_D;
  if (H < 1 || L < 1) return LSD_ERR_SHAPE;
  if ((long long)H * (long long)L > (long long)INT_MAX) return LSD_ERR_SHAPE;
  return LSD_OK;
}

int check_scale(float s) { return (std::isfinite(s) && s > 0.0f) ? LSD_OK : LSD_ERR_SCALE; }

int launch_status(hipError_t e) { return e == hipSuccess ? LSD_OK : LSD_ERR_LAUNCH; }

constexpr float kLog2e = 1.44269504088896340736f;

// The attention kernels address one head's rows through 32-bit buffer
// offsets: L * d * 2 bytes must stay below 2^31.
int check_attn_len(int L) { return L < (1 << 23) ? LSD_OK : LSD_ERR_SHAPE; }

size_t nvfp4_tiles(long long rows) { return (size_t)((rows + lsd::kLinTileRows - 1) / lsd::kLinTileRows); }
size_t nvfp4_stages(int cols) { return (size_t)((cols + lsd::kLinStage - 1) / lsd::kLinStage); }

}  // namespace

extern "C" {

int lsd_abi_version(void) { return LSD_ABI_VERSION; }

const char* lsd_status_str(int status) {
  switch (status) {
    case LSD_OK: return "ok";
    case LSD_ERR_NULL: return "null pointer argument";
    case LSD_ERR_SHAPE: return "bad shape (need H >= 1, L >= 1, H*L <= 2^31-1)";
    case LSD_ERR_UNSUPPORTED_D: return "unsupported head dimension (only d = 128)";
    case LSD_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case LSD_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case LSD_ERR_LAUNCH: return "kernel launch failed";
    case LSD_ERR_SCALE: return "scale must be finite and > 0";
    case LSD_ERR_FLAGS: return "unknown flag bits or layout";
    default: return "unknown status";
  }
}

int attn_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                  int H, int L, int d, float softmax_scale, void* stream) {
  int st = check_shape(H, L, d);
  if (st != LSD_OK) return st;
  if ((st = check_attn_len(L)) != LSD_OK) return st;
  if (!q || !k || !v || !o) return LSD_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return LSD_ERR_ALIGN;
  if (lse && ((uintptr_t)lse & 3u)) return LSD_ERR_ALIGN;
  if ((st = check_scale(softmax_scale)) != LSD_OK) return st;
  (void)hipGetLastError();
  return launch_status(lsd::launch_attn_bf16(q, k, v, o, lse, nullptr, nullptr, H, L, softmax_scale * kLog2e,
                                             (hipStream_t)stream));
}

int attn_fwd_bf16_train(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                        float* o_f32, float* row_ml, int H, int L, int d, float softmax_scale, void* stream) {
  int st = check_shape(H, L, d);
  if (st != LSD_OK) return st;
  if ((st = check_attn_len(L)) != LSD_OK) return st;
  if (!q || !k || !v || !o || !o_f32 || !row_ml) return LSD_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(o_f32) ||
      ((uintptr_t)row_ml & 7u))
    return LSD_ERR_ALIGN;
  if (lse && ((uintptr_t)lse & 3u)) return LSD_ERR_ALIGN;
  if ((st = check_scale(softmax_scale)) != LSD_OK) return st;
  (void)hipGetLastError();
  return launch_status(lsd::launch_attn_bf16(q, k, v, o, lse, o_f32, row_ml, H, L, softmax_scale * kLog2e,
                                             (hipStream_t)stream));
}

size_t qk_prep_fp4_workspace_bytes(int H, int L, int d) {
  if (check_shape(H, L, d) != LSD_OK) return 0;
  return lsd::prep_workspace_bytes(H, L);
}

int qk_prep_fp4_ex(const uint16_t* q, const uint16_t* k, uint8_t* q_codes, uint8_t* q_scales,
                   uint8_t* k_codes, uint8_t* k_scales, float* k_mean, void* workspace,
                   size_t workspace_bytes, int H, int L, int d, int flags, void* stream) {
  int st = check_shape(H, L, d);
  if (st != LSD_OK) return st;
  if (flags & ~(LSD_PREP_SMOOTH_K | LSD_PREP_ROTATE | LSD_PREP_K_ONLY)) return LSD_ERR_FLAGS;
  const bool smooth = (flags & LSD_PREP_SMOOTH_K) != 0;
  const bool with_q = (flags & LSD_PREP_K_ONLY) == 0;
  if (!k || !k_codes || !k_scales || (smooth && !k_mean)) return LSD_ERR_NULL;
  if (with_q && (!q || !q_codes || !q_scales)) return LSD_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_codes) || !aligned16(q_scales) ||
      !aligned16(k_codes) || !aligned16(k_scales) || !aligned16(k_mean))
    return LSD_ERR_ALIGN;
  if (smooth && (!workspace || ((uintptr_t)workspace & 255u) ||
                 workspace_bytes < lsd::prep_workspace_bytes(H, L)))
    return LSD_ERR_WORKSPACE;
  (void)hipGetLastError();
  return launch_status(lsd::launch_qk_prep(q, k, q_codes, q_scales, k_codes, k_scales, k_mean, workspace,
                                           H, L, smooth, (flags & LSD_PREP_ROTATE) != 0, with_q,
                                           (hipStream_t)stream));
}

int qk_prep_fp4(const uint16_t* q, const uint16_t* k, uint8_t* q_codes, uint8_t* q_scales,
                uint8_t* k_codes, uint8_t* k_scales, float* k_mean, void* workspace,
                size_t workspace_bytes, int H, int L, int d, void* stream) {
  return qk_prep_fp4_ex(q, k, q_codes, q_scales, k_codes, k_scales, k_mean, workspace, workspace_bytes, H, L, d,
                        LSD_PREP_SMOOTH_K | LSD_PREP_ROTATE, stream);
}

int qk_prep_fp4_noalloc(const uint16_t* q, const uint16_t* k, uint8_t* q_codes, uint8_t* q_scales,
                        uint8_t* k_codes, uint8_t* k_scales, float* k_mean, int H, int L, int d, void* stream) {
  int st = check_shape(H, L, d);
  if (st != LSD_OK) return st;
  if (!q || !k || !q_codes || !q_scales || !k_codes || !k_scales || !k_mean) return LSD_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_codes) || !aligned16(q_scales) ||
      !aligned16(k_codes) || !aligned16(k_scales) || !aligned16(k_mean))
    return LSD_ERR_ALIGN;
  if (lsd::prep_workspace_bytes(H, L) > lsd::prep_scratch_bytes()) return LSD_ERR_WORKSPACE;
  void* scratch = nullptr;
  if (lsd::prep_scratch(&scratch) != hipSuccess) return LSD_ERR_LAUNCH;
  (void)hipGetLastError();
  return launch_status(lsd::launch_qk_prep(q, k, q_codes, q_scales, k_codes, k_scales, k_mean, scratch, H, L,
                                           true, true, true, (hipStream_t)stream));
}

int attn_fwd_fp4qk(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                   const uint8_t* k_scales, const uint16_t* v, uint16_t* o, float* lse, int H, int L,
                   int d, float softmax_scale, void* stream) {
  int st = check_shape(H, L, d);
  if (st != LSD_OK) return st;
  if ((st = check_attn_len(L)) != LSD_OK) return st;
  if (!q_codes || !q_scales || !k_codes || !k_scales || !v || !o) return LSD_ERR_NULL;
  if (!aligned16(q_codes) || !aligned16(q_scales) || !aligned16(k_codes) || !aligned16(k_scales) ||
      !aligned16(v) || !aligned16(o))
    return LSD_ERR_ALIGN;
  if (lse && ((uintptr_t)lse & 3u)) return LSD_ERR_ALIGN;
  if ((st = check_scale(softmax_scale)) != LSD_OK) return st;
  (void)hipGetLastError();
  return launch_status(lsd::launch_attn_fp4qk(q_codes, q_scales, k_codes, k_scales, v, o, lse, nullptr, nullptr,
                                              H, L, softmax_scale * kLog2e, (hipStream_t)stream));
}

int attn_fwd_fp4qk_train(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                         const uint8_t* k_scales, const uint16_t* v, uint16_t* o, float* lse, float* o_f32,
                         float* row_ml, int H, int L, int d, float softmax_scale, void* stream) {
  int st = check_shape(H, L, d);
  if (st != LSD_OK) return st;
  if ((st = check_attn_len(L)) != LSD_OK) return st;
  if (!q_codes || !q_scales || !k_codes || !k_scales || !v || !o || !o_f32 || !row_ml) return LSD_ERR_NULL;
  if (!aligned16(q_codes) || !aligned16(q_scales) || !aligned16(k_codes) || !aligned16(k_scales) ||
      !aligned16(v) || !aligned16(o) || !aligned16(o_f32) || ((uintptr_t)row_ml & 7u))
    return LSD_ERR_ALIGN;
  if (lse && ((uintptr_t)lse & 3u)) return LSD_ERR_ALIGN;
  if ((st = check_scale(softmax_scale)) != LSD_OK) return st;
  (void)hipGetLastError();
  return launch_status(lsd::launch_attn_fp4qk(q_codes, q_scales, k_codes, k_scales, v, o, lse, o_f32, row_ml,
                                              H, L, softmax_scale * kLog2e, (hipStream_t)stream));
}

int attn_fwd_fp4qk_fused_q(const uint16_t* q, const uint8_t* k_codes, const uint8_t* k_scales, const uint16_t* v,
                           uint16_t* o, float* lse, int H, int L, int d, float softmax_scale, void* stream) {
  int st = check_shape(H, L, d);
  if (st != LSD_OK) return st;
  if ((st = check_attn_len(L)) != LSD_OK) return st;
  if (!q || !k_codes || !k_scales || !v || !o) return LSD_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(k_scales) || !aligned16(v) || !aligned16(o))
    return LSD_ERR_ALIGN;
  if (lse && ((uintptr_t)lse & 3u)) return LSD_ERR_ALIGN;
  if ((st = check_scale(softmax_scale)) != LSD_OK) return st;
  (void)hipGetLastError();
  return launch_status(lsd::launch_attn_fp4qk_fused_q(q, k_codes, k_scales, v, o, lse, H, L,
                                                      softmax_scale * kLog2e, (hipStream_t)stream));
}

size_t attn_bwd_bf16_workspace_bytes(int H, int L, int d) {
  if (check_shape(H, L, d) != LSD_OK) return 0;
  return lsd::attn_bwd_workspace_bytes(H, L);
}

int attn_bwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* o_f32,
                  const float* row_ml, const uint16_t* dout, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                  void* workspace, size_t workspace_bytes, int H, int L, int d, float softmax_scale, void* stream) {
  int st = check_shape(H, L, d);
  if (st != LSD_OK) return st;
  if ((st = check_attn_len(L)) != LSD_OK) return st;
  if (!q || !k || !v || !o_f32 || !row_ml || !dout || !dq || !dk || !dv) return LSD_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_f32) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || ((uintptr_t)row_ml & 7u))
    return LSD_ERR_ALIGN;
  if ((st = check_scale(softmax_scale)) != LSD_OK) return st;
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < lsd::attn_bwd_workspace_bytes(H, L))
    return LSD_ERR_WORKSPACE;
  (void)hipGetLastError();
  return launch_status(lsd::launch_attn_bwd(q, k, v, o_f32, row_ml, dout, dq, dk, dv, workspace, H, L,
                                            softmax_scale, (hipStream_t)stream));
}

size_t attn_bwd_fp4qk_workspace_bytes(int H, int L, int d) {
  if (check_shape(H, L, d) != LSD_OK) return 0;
  return lsd::attn_bwd_fp4qk_workspace_bytes(H, L);
}

int attn_bwd_fp4qk(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                   const uint8_t* k_scales, const uint16_t* v, const float* o_f32, const float* row_ml,
                   const uint16_t* dout, uint16_t* dq, uint16_t* dk, uint16_t* dv, void* workspace,
                   size_t workspace_bytes, int H, int L, int d, float softmax_scale, int flags, void* stream) {
  int st = check_shape(H, L, d);
  if (st != LSD_OK) return st;
  if ((st = check_attn_len(L)) != LSD_OK) return st;
  if (flags & ~(LSD_PREP_SMOOTH_K | LSD_PREP_ROTATE)) return LSD_ERR_FLAGS;
  if (!q_codes || !q_scales || !k_codes || !k_scales || !v || !o_f32 || !row_ml || !dout || !dq || !dk || !dv)
    return LSD_ERR_NULL;
  if (!aligned16(q_codes) || !aligned16(q_scales) || !aligned16(k_codes) || !aligned16(k_scales) ||
      !aligned16(v) || !aligned16(o_f32) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv) || ((uintptr_t)row_ml & 7u))
    return LSD_ERR_ALIGN;
  if ((st = check_scale(softmax_scale)) != LSD_OK) return st;
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < lsd::attn_bwd_fp4qk_workspace_bytes(H, L))
    return LSD_ERR_WORKSPACE;
  (void)hipGetLastError();
  return launch_status(lsd::launch_attn_bwd_fp4qk(q_codes, q_scales, k_codes, k_scales, v, o_f32, row_ml, dout,
                                                  dq, dk, dv, workspace, H, L, softmax_scale,
                                                  (flags & LSD_PREP_ROTATE) != 0, (hipStream_t)stream));
}

size_t nvfp4_codes_bytes(long long rows, int cols, int layout) {
  if (rows < 1 || cols < lsd::kBlock || cols % lsd::kBlock || rows > (1LL << 40)) return 0;
  if (layout == LSD_NVFP4_ROWS) return (size_t)rows * (size_t)(cols / 2);
  if (layout != LSD_NVFP4_TILED) return 0;
  return nvfp4_tiles(rows) * nvfp4_stages(cols) * (size_t)(lsd::kLinTileRows * lsd::kLinStage / 2);
}

size_t nvfp4_scales_bytes(long long rows, int cols, int layout) {
  if (rows < 1 || cols < lsd::kBlock || cols % lsd::kBlock || rows > (1LL << 40)) return 0;
  if (layout == LSD_NVFP4_ROWS) return (size_t)rows * (size_t)(cols / lsd::kBlock);
  if (layout != LSD_NVFP4_TILED) return 0;
  return nvfp4_tiles(rows) * nvfp4_stages(cols) * (size_t)(lsd::kLinTileRows * lsd::kLinStage / lsd::kBlock);
}

int nvfp4_quantize(const uint16_t* x, uint8_t* codes, uint8_t* scales, long long rows, int cols,
                   float global_scale, int layout, void* stream) {
  if (layout != LSD_NVFP4_ROWS && layout != LSD_NVFP4_TILED) return LSD_ERR_FLAGS;
  if (rows < 1 || cols < lsd::kBlock || cols % lsd::kBlock) return LSD_ERR_SHAPE;
  if (rows > (1LL << 40) || rows * (cols / lsd::kBlock) >= (1LL << 39)) return LSD_ERR_SHAPE;
  if (!x || !codes || !scales) return LSD_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return LSD_ERR_ALIGN;
  if (check_scale(global_scale) != LSD_OK) return LSD_ERR_SCALE;
  (void)hipGetLastError();
  return launch_status(lsd::launch_nvfp4_quantize(x, codes, scales, rows, cols, global_scale,
                                                  layout == LSD_NVFP4_TILED, (hipStream_t)stream));
}

int nvfp4_linear(const uint8_t* x_codes, const uint8_t* x_scales, float x_global_scale,
                 const uint8_t* w_codes, const uint8_t* w_scales, float w_global_scale,
                 uint16_t* y, int M, int N, int K, int layout, void* stream) {
  if (layout != LSD_NVFP4_ROWS && layout != LSD_NVFP4_TILED) return LSD_ERR_FLAGS;
  // tile counts are formed as (M + 255) / 256 in 32-bit arithmetic
  if (M < 1 || N < 1 || M > INT_MAX - 255 || N > INT_MAX - 255) return LSD_ERR_SHAPE;
  if (K < lsd::kBlock || K % lsd::kBlock || K > (1 << 20)) return LSD_ERR_SHAPE;
  if (!x_codes || !x_scales || !w_codes || !w_scales || !y) return LSD_ERR_NULL;
  if (!aligned16(x_codes) || !aligned16(x_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      ((uintptr_t)y & 7u))
    return LSD_ERR_ALIGN;
  if (check_scale(x_global_scale) != LSD_OK || check_scale(w_global_scale) != LSD_OK) return LSD_ERR_SCALE;
  (void)hipGetLastError();
  return launch_status(lsd::launch_nvfp4_linear(x_codes, x_scales, x_global_scale, w_codes, w_scales,
                                                w_global_scale, y, M, N, K, layout == LSD_NVFP4_TILED,
                                                (hipStream_t)stream));
}

}  // extern "C"
