/*
 * q8.h -- C ABI of libq4, per-output-channel INT8 weights (W8A16): symmetric
 * INT8 round-to-nearest with one float16 scale per row of W, and the fused
 * dequantize-and-multiply product with float16 activations, for AMD Instinct
 * MI355X (gfx950). Same library, status codes and conventions as q4.h
 * (device pointers owned by the caller, enqueue-only on `stream`, host-side
 * validation before any HIP call, q4_last_error() for details).
 *
 * Sources of the method (cited by page title and section):
 *  [CH]   "量化：PTQ、GPTQ、AWQ 与 SmoothQuant" (charles2530.github.io), the closing
 *         quick code example: per output channel, scale = amax / 127,
 *         q = clamp(round(w / scale), -127, 127), w_hat = q * scale.
 *  [IOC]  "模型量化技术工程实践：GPTQ/AWQ/QLoRA深度解析" (www.iopencloud.com),
 *         section 2.1: symmetric INT8, scale = max|W| / 127, range [-127, 127].
 *  [ARG]  "Post-training quantization: GPTQ, AWQ and rotation" (arganzheng.life),
 *         section 四.3: per-channel INT8 RTN is nearly lossless and the W8A16
 *         default; section 二.3: weight-only quantization keeps 16-bit
 *         activations and dequantizes on chip.
 *
 * Shapes: W [out][in] float16, x [B][in] float16, y [B][out] float16, row-major.
 * out and in in [1, 2^30); in must be a multiple of 8 (16-byte rows).
 *
 * Device layout of the codes (opaque; q8_to_canonical / q8_from_canonical
 * convert). With Np = ceil(out/16)*16, Kp = ceil(in/128)*128, S = Kp/128, code
 * (n, k) with t = n/16, r = n%16, s = k/128, h = (k%128)/64, j = (k%64)/32,
 * c = (k%32)/8, e = k%8 is the byte
 *     ((t*S + s)*2 + h)*1024 + (r + 16*c)*16 + 8*j + e
 * holding q + 128. Padding (rows >= out, channels >= in) holds 128 (code 0).
 * A 16-row x 128-channel tile is one 2 KiB block: two 16-byte loads per lane of a
 * 64-lane wavefront, each giving two MFMA A operands. Scales: float16 [Np],
 * padding rows 0.
 *
 * Canonical layout: codes int8 [out][in] (two's complement), scales float16 [out].
 */
#ifndef Q8_H
#define Q8_H

#include "q4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the device-layout code buffer: ceil(out/16)*16 * ceil(in/128)*128.
 * 0 if out or in is out of range or in % 8 != 0. */
size_t q8_packed_bytes(int64_t out, int64_t in);

/* float16 elements of the device-layout scale array: ceil(out/16)*16 (0 if out
 * is out of range). */
size_t q8_scales_count(int64_t out);

/* Per-channel INT8 quantize + pack ([CH] quick code example; [IOC] section 2.1):
 *   s16[n] = float16_rne(float32(max_k |W[n][k]|) / 127.0f)
 *   q[n][k] = clamp(rint_half_even(float32(W[n][k]) / float32(s16[n])), -127, 127),
 *             q = 0 wherever s16 == 0 (an all-zero row, or amax / 127 below
 *             float16's range; the example's clamp of amax at 1e-6 changes no
 *             float16 scale).
 * IEEE float32 division. Writes q8_packed_bytes(out, in) bytes to `packed`
 * (16-byte aligned) and q8_scales_count(out) float16 to `scales` (2-byte
 * aligned), padding included. W: [out][in] float16, 16-byte aligned. Reads W
 * twice (row maxima, then codes). */
q4_status q8_quantize_pack(const void* W, int64_t out, int64_t in, void* packed, void* scales, void* stream);

/* Bytes of device workspace q8_gemm needs for this shape (float32 partial sums
 * when the channel range is split over workgroups); 0 when none is needed.
 * Contents on entry are ignored and undefined on return. */
size_t q8_workspace_bytes(int64_t B, int64_t out, int64_t in);

/* Fused W8A16 product ([ARG] section 二.3):
 *   y[b][n] = float16_rne( sum over 128-channel blocks of s16[n] * sum_k x[b][k] * q[n][k] )
 * float16 x and codes, float32 accumulation. B <= 16 runs the GEMV kernel (one
 * 16-column MFMA tile), a larger B the skinny MFMA GEMM (column tiles of 16 batch
 * rows sharing each dequantized code fragment). x: [B][in] float16, 16-byte
 * aligned; packed/scales as written by q8_quantize_pack; y: [B][out] float16,
 * 2-byte aligned; `workspace` (16-byte aligned) must hold
 * q8_workspace_bytes(B, out, in) bytes (NULL allowed when that is 0, else
 * Q4_ERR_WORKSPACE). Deterministic. */
q4_status q8_gemm(const void* x, int64_t B, const void* packed, const void* scales, int64_t out, int64_t in,
                  void* y, void* workspace, size_t workspace_bytes, void* stream);

/* q8_gemm with an explicit GEMV launch shape (B <= 16), for tuning: `rows_per_wave`
 * 1, 2 or 4 row tiles of 16 per wavefront, `waves_per_group` 1..16 (at most 8 used
 * with rows_per_wave 2 or 4), `k_splits` workgroups splitting the channel range (at
 * most ceil(in/128); the activation slice of one split must fit the device's LDS).
 * Needs k_splits * B * out * 4 bytes of workspace when k_splits > 1.
 * Q4_ERR_UNSUPPORTED for B > 16 and for shapes the kernel cannot run. */
q4_status q8_gemm_config(const void* x, int64_t B, const void* packed, const void* scales, int64_t out,
                         int64_t in, void* y, int32_t rows_per_wave, int32_t waves_per_group, int32_t k_splits,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Device layout -> canonical layout: canon_codes int8 [out][in], canon_scales
 * float16 [out]. */
q4_status q8_to_canonical(const void* packed, const void* scales, int64_t out, int64_t in, void* canon_codes,
                          void* canon_scales, void* stream);

/* Canonical layout -> device layout, padding included (imports INT8 weights
 * quantized elsewhere; every int8 code, -128 included, multiplies as itself). */
q4_status q8_from_canonical(const void* canon_codes, const void* canon_scales, int64_t out, int64_t in,
                            void* packed, void* scales, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q8_H */
