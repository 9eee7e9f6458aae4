// Internal launch interface between the C ABI (abi.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace lsd {

constexpr int kHeadDim = 128;
constexpr int kBlock = 16;          // channels per NVFP4 scale

// attention (attn_fwd.hip); o32 and ml (the training outputs) are both null
// or both set
hipError_t launch_attn_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            uint16_t* o, float* lse, float* o32, float* ml, int H, int L,
                            float scale_log2, hipStream_t stream);
hipError_t launch_attn_fp4qk(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc,
                             const uint8_t* ks, const uint16_t* v, uint16_t* o, float* lse,
                             float* o32, float* ml, int H, int L, float scale_log2, hipStream_t stream);

hipError_t launch_attn_fp4qk_fused_q(const uint16_t* q, const uint8_t* kc, const uint8_t* ks, const uint16_t* v,
                                     uint16_t* o, float* lse, int H, int L, float scale_log2, hipStream_t stream);

// attention backward (attn_bwd.hip)
size_t attn_bwd_workspace_bytes(int H, int L);
hipError_t launch_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* o32,
                           const float* ml, const uint16_t* dout, uint16_t* dq, uint16_t* dk, uint16_t* dv, void* ws,
                           int H, int L, float scale, hipStream_t stream);

size_t attn_bwd_fp4qk_workspace_bytes(int H, int L);
hipError_t launch_attn_bwd_fp4qk(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                                 const uint16_t* v, const float* o32, const float* ml, const uint16_t* dout,
                                 uint16_t* dq, uint16_t* dk, uint16_t* dv, void* ws, int H, int L, float scale,
                                 bool rotate, hipStream_t stream);

// Q/K preparation (qk_prep.hip)
size_t prep_workspace_bytes(int H, int L);
// The prep's static scratch (no-allocation entry point): its capacity in bytes,
// and this device's address of it (looked up once per device).
size_t prep_scratch_bytes();
hipError_t prep_scratch(void** ptr);
hipError_t launch_qk_prep(const uint16_t* q, const uint16_t* k, uint8_t* qc, uint8_t* qs,
                          uint8_t* kc, uint8_t* ks, float* kmean, void* ws, int H, int L,
                          bool smooth, bool rotate, bool with_q, hipStream_t stream);

// NVFP4 W4A4 linear layer (qk_prep.hip: quantizer, nvfp4_gemm.hip: product).
// Tiled code layout: rows in tiles of kLinTileRows, K in stages of kLinStage
// values, one contiguous chunk of codes (and one of scales) per (tile, stage).
constexpr int kLinTileRows = 256;
constexpr int kLinStage = 64;
hipError_t launch_nvfp4_quantize(const uint16_t* x, uint8_t* codes, uint8_t* scales, long long rows, int cols,
                                 float global_scale, bool tiled, hipStream_t stream);
hipError_t launch_nvfp4_linear(const uint8_t* xc, const uint8_t* xs, float gx, const uint8_t* wc, const uint8_t* ws,
                               float gw, uint16_t* y, int M, int N, int K, bool tiled, hipStream_t stream);

}  // namespace lsd
