/*
 * lsd_attn.h - dense long-sequence attention on AMD MI355X (gfx950).
 *
 * C ABI of liblsd_attn.so.  Operations over per-head token tensors laid
 * out [H, L, d] (row-major: head, token, channel), d = 128:
 *
 *   attn_fwd_bf16   dense non-causal softmax attention, BF16 in and out.
 *   qk_prep_fp4     mean-key subtraction, shared 128-point Hadamard rotation
 *                   and NVFP4 block quantization of Q and K (qk_prep_fp4_ex:
 *                   the same with either transform switched off).
 *   attn_fwd_fp4qk  attention whose scores come from the NVFP4 Q and K;
 *                   probabilities and V stay BF16 (attn_fwd_fp4qk_fused_q:
 *                   the same with Q quantized inside the attention kernel).
 *   attn_fwd_bf16_train, attn_fwd_fp4qk_train  the two forwards with the
 *                   extra outputs their backward reads (fp32 O, row max and
 *                   row sum).
 *   attn_bwd_bf16   gradients of attn_fwd_bf16 with respect to Q, K and V.
 *   attn_bwd_fp4qk  training-time gradients of attn_fwd_fp4qk (straight-
 *                   through quantizer), with respect to the original Q, K, V.
 *   nvfp4_quantize  NVFP4 quantization (per-tensor global scale) of the rows
 *                   of a linear layer's activation or weight matrix, row-major
 *                   or in the product's tiled load order.
 *   nvfp4_linear    the W4A4 linear layer Y = X W^T from two such operands.
 *
 * The method is the one of "Pika H3 Flex in FastVideo: 7x Faster, and Near
 * Real Time in 4-bit" (haoailab blog): section "Faster at BF16" (dense
 * attention over the ~109k-token joint sequence of a 15-second clip) and
 * section "FP4 attention" (smooth K, rotate Q and K with one orthonormal
 * Hadamard matrix, E2M1 values with one E4M3 scale per 16 channels and unit
 * global scale, a fused kernel that applies the transforms while quantizing).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer to contiguous memory owned by
 *     the caller.  BF16 values are passed as their uint16 bit patterns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is enqueued asynchronously on it; nothing synchronizes.
 *   - Argument errors are detected on the host before anything is enqueued and
 *     returned as an lsd_status; a launch failure returns LSD_ERR_LAUNCH.  A
 *     device fault surfaces at the caller's next synchronization.  Nothing is
 *     printed and no exception crosses the ABI.
 *   - The library allocates no memory and keeps no state between calls;
 *     concurrent calls on different streams are safe as long as their output
 *     (and workspace) buffers do not overlap.
 *   - Limits: d must be 128; H >= 1; L >= 1; H * L <= 2^31 - 1; for the two
 *     attention calls also L < 2^23 (one head's rows are addressed with
 *     32-bit byte offsets).  Tensor pointers must be 16-byte aligned.
 *   - Inputs must be finite.  NaN or Inf in any input, or inputs so large that
 *     the rotation overflows float32 (|x| around 2^120), give unspecified
 *     output (no fault).
 */
#ifndef LSD_ATTN_H
#define LSD_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum lsd_status {
  LSD_OK = 0,
  LSD_ERR_NULL = 1,           /* a required pointer is NULL                   */
  LSD_ERR_SHAPE = 2,          /* H < 1, L < 1, H * L or (attention) L too large */
  LSD_ERR_UNSUPPORTED_D = 3,  /* d != 128                                     */
  LSD_ERR_ALIGN = 4,          /* a tensor pointer is not 16-byte aligned      */
  LSD_ERR_WORKSPACE = 5,      /* workspace missing, misaligned or too small   */
  LSD_ERR_LAUNCH = 6,         /* the HIP runtime rejected a kernel launch     */
  LSD_ERR_SCALE = 7,          /* a scale argument is not finite and positive  */
  LSD_ERR_FLAGS = 8           /* unknown bits in a flags or layout argument    */
};

/* Version of this ABI (the value of LSD_ABI_VERSION the library was built with). */
#define LSD_ABI_VERSION 5
int lsd_abi_version(void);

/* Static description of a status code ("ok", "null pointer", ...). */
const char* lsd_status_str(int status);

/*
 * attn_fwd_bf16 - O = softmax(softmax_scale * Q K^T) V for every head, no mask.
 *   q, k, v : [H, L, d] BF16 bits, read only.
 *   o       : [H, L, d] BF16 bits, written (round to nearest even of the fp32
 *             result).  Must not alias q, k or v.
 *   lse     : optional [H, L] float32 natural-log log-sum-exp of the scaled
 *             scores of each query row (NULL to skip).
 *   softmax_scale : sigma > 0 applied to the fp32 scores.
 * Scores and the P.V products accumulate in fp32 on the matrix cores; P is
 * rounded to BF16 before P.V.  Results are deterministic (no atomics).
 * Source: "Faster at BF16" (dense attention over all tokens of a clip).
 */
int attn_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  uint16_t* o, float* lse, int H, int L, int d,
                  float softmax_scale, void* stream);

/*
 * attn_fwd_bf16_train - attn_fwd_bf16 (the same o and optional lse, bit for
 * bit) that also writes what attn_bwd_bf16 reads:
 *   o_f32  : [H, L, d] float32, written: the fp32 values that o rounds (o is
 *            their round to nearest even), 16-byte aligned.
 *   row_ml : [H, L, 2] float32, written: per query row the pair (m, l) with
 *            the row's weights exp2(sigma log2(e) s_j - m) / l, m the
 *            reference max in log2 units and l the sum of the BF16-rounded
 *            weights that o is normalized by; 8-byte aligned.
 * The pair replaces one fp32 log-sum-exp, whose rounding (the scores reach
 * ~1e5 in log2 units on peaked workloads) would shift every recomputed
 * weight of a row.  Errors as attn_fwd_bf16; o_f32 and row_ml are required.
 * Source: "NVFP4 QAD" (training with the deployed attention in the loop).
 */
int attn_fwd_bf16_train(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        uint16_t* o, float* lse, float* o_f32, float* row_ml,
                        int H, int L, int d, float softmax_scale, void* stream);

/*
 * Bytes of device workspace qk_prep_fp4 needs for this shape (0 on a bad
 * shape): H * 128 * ceil(L / 4096) * 16 * 8.  It holds exact fp64 partial
 * column sums of K.
 */
size_t qk_prep_fp4_workspace_bytes(int H, int L, int d);

/*
 * qk_prep_fp4 - quantize Q and K for attn_fwd_fp4qk.
 *   q, k      : [H, L, d] BF16 bits, read only.
 *   q_codes, k_codes   : [H, L, d/2] uint8, written; byte j of a row holds the
 *                        E2M1 code of channel 2j in its low nibble and of
 *                        channel 2j+1 in its high nibble (bit 3 = sign).
 *   q_scales, k_scales : [H, L, d/16] uint8, written; OCP E4M3 bits of the
 *                        scale of channels 16b..16b+15 (never NaN, <= 448).
 *   k_mean    : [H, d] float32, written: per head and channel the mean of K
 *               over the L tokens, RN32(RN64(exact sum) / L).
 *   workspace : device buffer of at least qk_prep_fp4_workspace_bytes(H,L,d)
 *               bytes, 256-byte aligned; contents on entry are ignored and on
 *               return are unspecified.
 * Per row: K only: x = RN32(k - k_mean); then the in-order Sylvester butterfly
 * in fp32 (7 stages, stage s pairs channels i and i + 2^s), times
 * RN32(1/sqrt(128)); per 16-channel block the scale is the E4M3 value nearest
 * to max|y|/6 (ties to even, saturating at 448) and each code is the E2M1
 * value nearest to y/scale (ties to even, saturating at 6, sign kept, all
 * codes signed zero when the scale is 0).  Codes and scales are exact
 * functions of the inputs: bit-identical from run to run.
 * Source: "FP4 attention" (smooth K, rotate Q and K, E2M1 + E4M3 per 16).
 */
int qk_prep_fp4(const uint16_t* q, const uint16_t* k,
                uint8_t* q_codes, uint8_t* q_scales,
                uint8_t* k_codes, uint8_t* k_scales,
                float* k_mean, void* workspace, size_t workspace_bytes,
                int H, int L, int d, void* stream);

/* Bits of the `flags` argument of qk_prep_fp4_ex. */
enum lsd_prep_flags {
  LSD_PREP_SMOOTH_K = 1,      /* subtract the per-head mean key before quantizing K */
  LSD_PREP_ROTATE = 2,        /* shared 128-point Hadamard rotation of Q and K      */
  LSD_PREP_K_ONLY = 4         /* prepare K only (Q is quantized by attn_fwd_fp4qk_fused_q) */
};

/*
 * qk_prep_fp4_ex - qk_prep_fp4 with the two transforms switched separately,
 * for ablations of the quantization error.
 *   flags : LSD_PREP_SMOOTH_K | LSD_PREP_ROTATE gives exactly qk_prep_fp4;
 *           other bits -> LSD_ERR_FLAGS.
 *   Without LSD_PREP_SMOOTH_K: K is quantized as given (x = k); workspace may
 *           be NULL (it is not used); k_mean may be NULL, and if it is not it
 *           is written with zeros (the mean that was subtracted).
 *   Without LSD_PREP_ROTATE: no butterfly and no 1/sqrt(128) factor; the
 *           16-channel blocks are consecutive original channels.
 *   With LSD_PREP_K_ONLY: Q is neither read nor written (q, q_codes and
 *           q_scales may be NULL); K's outputs are those of the same call
 *           without it.
 * Everything else (layouts, rounding, codes, errors) is as in qk_prep_fp4.
 * Source: "FP4 attention" (quantizing naively costs accuracy; smoothing K and
 * the Hadamard rotation recover part of it; its per-layer error table).
 */
int qk_prep_fp4_ex(const uint16_t* q, const uint16_t* k,
                   uint8_t* q_codes, uint8_t* q_scales,
                   uint8_t* k_codes, uint8_t* k_scales,
                   float* k_mean, void* workspace, size_t workspace_bytes,
                   int H, int L, int d, int flags, void* stream);

/* Largest problem qk_prep_fp4_noalloc accepts: its static scratch holds the
 * prep's exact partial column sums, 16384 bytes per (head, 4096-token chunk
 * of L), i.e. H * ceil(L / 4096) <= 4096 (64 MiB per GPU). */
#define LSD_PREP_NOALLOC_MAX_HEAD_CHUNKS 4096

/*
 * qk_prep_fp4_noalloc - qk_prep_fp4 without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, outputs,
 * layouts, bit-exact results and errors as qk_prep_fp4, minus the workspace.
 * Its scratch is a static 64 MiB device array inside the library (one per
 * GPU, held until the process ends); the first call on a device looks up that
 * device's copy (no allocation).  H * ceil(L / 4096) above
 * LSD_PREP_NOALLOC_MAX_HEAD_CHUNKS -> LSD_ERR_WORKSPACE, before anything is
 * enqueued.  Every call on one GPU uses the same scratch: calls that overlap
 * in time on one GPU (different streams, different host threads) race and
 * must be ordered by the caller.  Nothing in the scratch needs clearing
 * between calls (each call writes every value it reads).
 */
int qk_prep_fp4_noalloc(const uint16_t* q, const uint16_t* k,
                        uint8_t* q_codes, uint8_t* q_scales,
                        uint8_t* k_codes, uint8_t* k_scales,
                        float* k_mean, int H, int L, int d, void* stream);

/*
 * attn_fwd_fp4qk - attention on quantized Q and K.
 *   q_codes, q_scales, k_codes, k_scales : as written by qk_prep_fp4 (or by
 *             qk_prep_fp4_ex: any variant, as long as Q and K come from the
 *             same call).
 *   v   : [H, L, d] BF16 bits.   o : [H, L, d] BF16 bits, written.
 *   lse : optional [H, L] float32 (NULL to skip).
 * Scores are softmax_scale * (Qhat . Khat) where Qhat, Khat are the exact
 * dequantized values (E2M1 times E4M3: at most 6 significant bits in
 * [2^-10, 2688], so exact in FP16, in which the score products run, and in
 * BF16); the rest is as in attn_fwd_bf16.  Because the smoothing and the
 * orthonormal rotation change no score before quantization, O approximates
 * attn_fwd_bf16 on the original Q, K.
 * Source: "FP4 attention" (queries and keys quantized, P and V in BF16).
 */
int attn_fwd_fp4qk(const uint8_t* q_codes, const uint8_t* q_scales,
                   const uint8_t* k_codes, const uint8_t* k_scales,
                   const uint16_t* v, uint16_t* o, float* lse,
                   int H, int L, int d, float softmax_scale, void* stream);

/*
 * attn_fwd_fp4qk_train - attn_fwd_fp4qk (the same o and optional lse, bit for
 * bit) that also writes o_f32 and row_ml exactly as attn_fwd_bf16_train does;
 * attn_bwd_fp4qk reads them.
 * Source: "NVFP4 QAD", "FP4 attention" (the training-time FP4 attention).
 */
int attn_fwd_fp4qk_train(const uint8_t* q_codes, const uint8_t* q_scales,
                         const uint8_t* k_codes, const uint8_t* k_scales,
                         const uint16_t* v, uint16_t* o, float* lse,
                         float* o_f32, float* row_ml,
                         int H, int L, int d, float softmax_scale, void* stream);

/*
 * attn_fwd_fp4qk_fused_q - attn_fwd_fp4qk with Q's preparation done inside
 * the attention kernel: each workgroup rotates and quantizes its own query
 * rows (the arithmetic of qk_prep_fp4, so the same codes) and dequantizes them
 * in registers; Q's codes never go through memory.
 *   q   : [H, L, d] BF16 bits (the unquantized queries).
 *   k_codes, k_scales : K prepared by qk_prep_fp4_ex with LSD_PREP_SMOOTH_K |
 *             LSD_PREP_ROTATE | LSD_PREP_K_ONLY (or by qk_prep_fp4).
 *   v, o, lse, softmax_scale, shape limits and errors : as attn_fwd_fp4qk.
 * Bit-identical to qk_prep_fp4 followed by attn_fwd_fp4qk on the same inputs.
 * Source: "FP4 attention" (a fused kernel applies the transforms while
 * quantizing Q and K) and "Faster at BF16" (the prologue work of attention
 * fused into the kernel).
 */
int attn_fwd_fp4qk_fused_q(const uint16_t* q, const uint8_t* k_codes,
                           const uint8_t* k_scales, const uint16_t* v,
                           uint16_t* o, float* lse, int H, int L, int d,
                           float softmax_scale, void* stream);

/*
 * Bytes of device workspace attn_bwd_bf16 needs (0 on a bad shape):
 * 3 * H * L * 4 (three fp32 statistics per query row).
 */
size_t attn_bwd_bf16_workspace_bytes(int H, int L, int d);

/*
 * attn_bwd_bf16 - gradients of attn_fwd_bf16 with respect to Q, K and V.
 *   q, k, v : [H, L, d] BF16 bits, the forward's inputs.
 *   o_f32, row_ml : as written by attn_fwd_bf16_train on the same inputs and
 *             softmax_scale (required).
 *   dout    : [H, L, d] BF16 bits, the gradient of the loss with respect to o.
 *   dq, dk, dv : [H, L, d] BF16 bits, written (round to nearest even of the
 *             fp32 results).  Must not alias any input.
 *   workspace : device buffer of at least attn_bwd_bf16_workspace_bytes
 *             bytes, 256-byte aligned; contents unspecified on return.
 *   softmax_scale : the sigma of the forward.
 * With P = softmax(sigma Q K^T) row-wise: dV = P^T dO, dP = dO V^T,
 * D = rowsum(P * dP), dS = P * (dP - D), dQ = sigma dS K, dK = sigma dS^T Q.
 * P is recomputed as exp2(sigma log2(e) s - m) / l from row_ml, and
 * D = rowsum(dO * O) from the fp32 O, which is the average of dP under the
 * forward's own weights: on rows that put nearly all their weight on one key
 * (dS nearly zero) dP - D then carries fp32 rounding only, where a BF16 O
 * would leave an error of 2^-9 |dP|.  P and dS are rounded to BF16 for the
 * matrix-core products; sums are fp32.  Seven of the 2 H L^2 d products per
 * call.  Deterministic (no atomics).  Same shape limits as attn_fwd_bf16.
 * Source: "NVFP4 QAD" and "FP4 attention" (the model is trained with the
 * deployed attention in the loop); the gradients are those of the forward.
 */
int attn_bwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  const float* o_f32, const float* row_ml, const uint16_t* dout,
                  uint16_t* dq, uint16_t* dk, uint16_t* dv,
                  void* workspace, size_t workspace_bytes,
                  int H, int L, int d, float softmax_scale, void* stream);

/*
 * Bytes of device workspace attn_bwd_fp4qk needs (0 on a bad shape):
 * 4 * H * L * d * 2 + 3 * H * L * 4 (dequantized Q, K and their gradients in
 * BF16, and the row statistics).
 */
size_t attn_bwd_fp4qk_workspace_bytes(int H, int L, int d);

/*
 * attn_bwd_fp4qk - training-time gradients of attn_fwd_fp4qk, with the NVFP4
 * quantizer passed straight through (its gradient taken as the identity).
 *   q_codes, q_scales, k_codes, k_scales : as written by qk_prep_fp4(_ex).
 *   v       : the forward's V (BF16).
 *   o_f32, row_ml : as written by attn_fwd_fp4qk_train on the same codes
 *             (required).
 *   dout      : [H, L, d] BF16, the gradient of the loss with respect to o.
 *   dq, dk    : [H, L, d] BF16, written: gradients with respect to the
 *             ORIGINAL Q and K (before smoothing and rotation).
 *   dv        : [H, L, d] BF16, written.
 *   flags     : the flags the codes were prepared with (LSD_PREP_ROTATE
 *             decides whether dQ, dK are rotated back; LSD_PREP_SMOOTH_K is
 *             accepted and changes nothing, see below); other bits ->
 *             LSD_ERR_FLAGS.
 *   workspace : at least attn_bwd_fp4qk_workspace_bytes bytes, 256-aligned.
 * Computes the attn_bwd_bf16 gradients at the exactly dequantized Q, K (in
 * the rotated basis) and then dQ = dQh R, dK = dKh R with R = H / sqrt(128)
 * (symmetric, orthonormal).  The Jacobian of the mean-key subtraction is
 * omitted: it would subtract the mean over keys of dK, which is zero because
 * softmax ignores a shift shared by every key (only rounding would change).
 * Source: "NVFP4 QAD" (distillation with the deployed numerics in the loop)
 * and "FP4 attention" (the training-time FP4 attention).
 */
int attn_bwd_fp4qk(const uint8_t* q_codes, const uint8_t* q_scales,
                   const uint8_t* k_codes, const uint8_t* k_scales,
                   const uint16_t* v, const float* o_f32, const float* row_ml,
                   const uint16_t* dout, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                   void* workspace, size_t workspace_bytes,
                   int H, int L, int d, float softmax_scale, int flags, void* stream);

/* Code layouts of nvfp4_quantize / nvfp4_linear operands. */
enum lsd_nvfp4_layout {
  LSD_NVFP4_ROWS = 0,   /* codes [rows, cols / 2], scales [rows, cols / 16], row-major     */
  LSD_NVFP4_TILED = 1   /* the product's load order: see nvfp4_codes_bytes                 */
};

/*
 * Bytes of the code and scale buffers of a [rows, cols] operand in a layout
 * (0 on bad arguments: rows < 1 or > 2^40, cols < 16 or not a multiple of 16,
 * unknown layout).
 *   LSD_NVFP4_ROWS : rows * cols / 2 and rows * cols / 16.
 *   LSD_NVFP4_TILED: rows are grouped in tiles of 256 and each row's values in
 *     stages of 64 (both zero-padded at the end); chunk (t, s), ordered
 *     t-major, holds rows 256 t .. 256 t + 255, values 64 s .. 64 s + 63 of
 *     each: 8192 code bytes (row r of the tile at 32 r, in the row-major byte
 *     order) and 1024 scale bytes (row r at 4 r).  ceil(rows / 256) *
 *     ceil(cols / 64) * 8192 and * 1024 bytes.  Padding holds zeros (code 0,
 *     scale 0: value 0).
 */
size_t nvfp4_codes_bytes(long long rows, int cols, int layout);
size_t nvfp4_scales_bytes(long long rows, int cols, int layout);

/*
 * nvfp4_quantize - NVFP4 codes of a row-major [rows, cols] BF16 matrix (an
 * activation X or a weight W of a linear layer).
 *   x       : [rows, cols] BF16 bits, read only, 16-byte aligned.
 *   codes   : nvfp4_codes_bytes(rows, cols, layout) bytes, written, 16-byte
 *             aligned.  Within a row, byte j holds value 2j in its low nibble
 *             and 2j+1 in its high nibble (E2M1: sign bit 3, magnitude index
 *             0..7 for 0, .5, 1, 1.5, 2, 3, 4, 6).
 *   scales  : nvfp4_scales_bytes(rows, cols, layout) bytes, written, 16-byte
 *             aligned: one E4M3 code per 16 consecutive values of a row.
 *   rows >= 1, cols >= 16 and a multiple of 16, rows * cols / 16 < 2^39
 *   (else LSD_ERR_SHAPE); layout an lsd_nvfp4_layout (else LSD_ERR_FLAGS).
 *   global_scale : g, float32, finite and > 0 (else LSD_ERR_SCALE).  The
 *             quantizer sees x' = RN32(x / g), the correctly rounded float32
 *             quotient (a quotient past the float32 range saturates like any
 *             value beyond 6 * 448), and quantizes each block of 16 as
 *             qk_prep_fp4 does (E4M3 scale
 *             of amax / 6 rounded to nearest even, then each value divided by
 *             it and rounded to nearest even E2M1, saturating at 6); a code e
 *             with block scale s stands for e * s * g, so g sets the clipping
 *             level 6 * 448 * g.  g is not stored: pass it to nvfp4_linear.
 * Source: "NVFP4 QAD" (4-bit weights and activations in every attention and
 * feed-forward linear, one 8-bit scale per 16 values; static activation
 * scales from calibration) with the block format of "FP4 attention".
 */
int nvfp4_quantize(const uint16_t* x, uint8_t* codes, uint8_t* scales, long long rows, int cols,
                   float global_scale, int layout, void* stream);

/*
 * nvfp4_linear - Y = (X^ g_x) (W^ g_w)^T, the W4A4 linear layer.
 *   x_codes, x_scales : the activation, [M, K] quantized by nvfp4_quantize
 *                       with global scale x_global_scale.
 *   w_codes, w_scales : the weight, [N, K] (one row per output feature),
 *                       quantized with global scale w_global_scale.
 *   layout  : the layout both operands were quantized in (else
 *             LSD_ERR_FLAGS); LSD_NVFP4_TILED is the faster one (every load
 *             of the product reads whole cache lines).
 *   y       : [M, N] BF16 bits, row-major, written (round to nearest even).
 *   1 <= M, N <= 2^31 - 256, K >= 16 and a multiple of 16, K <= 2^20 (else
 *   LSD_ERR_SHAPE); the scales must be finite and > 0 (else LSD_ERR_SCALE);
 *   code and scale pointers 16-byte aligned, y 8-byte aligned (else
 *   LSD_ERR_ALIGN).
 * Both operands are dequantized exactly on chip (an E2M1 value times an E4M3
 * scale fits FP16 and BF16), their products accumulate in fp32 on the matrix
 * cores, the fp32 sum is multiplied by RN32(g_x * g_w) and rounded to BF16.
 * No bias, no activation function.
 */
int nvfp4_linear(const uint8_t* x_codes, const uint8_t* x_scales, float x_global_scale,
                 const uint8_t* w_codes, const uint8_t* w_scales, float w_global_scale,
                 uint16_t* y, int M, int N, int K, int layout, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LSD_ATTN_H */
