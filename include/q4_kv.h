/*
 * q4_kv.h -- C ABI of libq4, INT4 group-wise quantization of a KV cache, for AMD
 * Instinct MI355X (gfx950). Same library, status codes and conventions as q4.h
 * (device pointers owned by the caller, enqueue-only on `stream`, host-side
 * validation before any HIP call, q4_last_error() for details).
 *
 * Sources (cited by page title and section):
 *  [WIKI] "压缩算法" (cs-knowledge-wiki.pages.dev), section 7.4.1.2,
 *         quantize_kv_cache_int4: K or V [batch, heads, seq_len, head_dim], groups
 *         of group_size channels along head_dim, scale = group amax / 7, codes
 *         round(x / scale) clamped to [-8, 7], two INT4 codes packed per byte (the
 *         page leaves pack_int4 undefined; the packing below is this library's).
 *  [YBB]  "LLM 后训练量化深度实战…" (www.ybb.press), section 七: KV bytes per token
 *         (2 * layers * kv_heads * head_dim * bytes); scales must be at least per
 *         head and follow the tokens (and pages) they belong to.
 *
 * Cache layout (bh = batch * kv_heads sequences of max_seq positions each):
 *   codes  uint8   [bh][max_seq][head_dim / 2]: byte i of a token row holds channel
 *                  2i in its low nibble and 2i + 1 in its high nibble, 4-bit two's
 *                  complement;
 *   scales float16 [bh][max_seq][head_dim / group]: one per token, head and group.
 * Rounding: scale = float16_rne(float32(amax) / 7.0f) (0 for an all-zero group,
 * whose codes are then 0); q = clamp(rint_half_even(float32(x) / float32(scale)),
 * -8, 7) with an IEEE float32 division -- the weight quantizer's rules (q4.h).
 * group is 32, 64 or 128; head_dim a positive multiple of group; every count
 * below 2^31.
 */
#ifndef Q4_KV_H
#define Q4_KV_H

#include "q4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Quantize n new tokens of every sequence into the cache at positions
 * pos .. pos + n - 1 (prefill: pos = 0, n = prompt length; decode: n = 1, pos = the
 * current length). src: float16 [bh][n][head_dim] contiguous, 16-byte aligned;
 * codes 4-byte and scales 2-byte aligned. pos + n must not exceed max_seq. Other
 * positions of the cache are not touched. */
q4_status q4_kv_quantize_pack(const void* src, int64_t bh, int64_t n, int64_t head_dim, int32_t group,
                              void* codes, void* scales, int64_t max_seq, int64_t pos, void* stream);

/* Dequantize positions pos .. pos + n - 1 of every sequence into dst float16
 * [bh][n][head_dim] (16-byte aligned): x_hat = q * scale, the float32 product
 * rounded once to float16. */
q4_status q4_kv_dequant(const void* codes, const void* scales, int64_t bh, int64_t n, int64_t head_dim,
                        int32_t group, int64_t max_seq, int64_t pos, void* dst, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4_KV_H */
