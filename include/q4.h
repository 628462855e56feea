/*
 * q4.h -- C ABI of libq4: group-wise INT4 round-to-nearest weight quantization
 * and the fused dequantize-and-multiply W4A16 product, for AMD Instinct MI355X
 * (gfx950).
 *
 * Sources of the method (cited by page title and section):
 *  [YBB]  "LLM 后训练量化深度实战：从 GPTQ/AWQ 到 FP8 与 KV Cache 量化的显存-带宽极限工程"
 *         (www.ybb.press), section 二: quantize_per_group (scale = group amax / 7,
 *         codes rounded and clamped to [-8, 7], one scale per group of input
 *         channels, in_features must be a multiple of the group size); section 一:
 *         the decode GEMV y = x W^T is bound by the bytes of W it reads.
 *  [ARG]  "Post-training quantization: GPTQ, AWQ and rotation" (arganzheng.life),
 *         section 二.2: affine form q = clamp(round(w/s) + z, 0, 2^b - 1),
 *         w_hat = s (q - z), asymmetric s = (max - min)/(2^b - 1), integer z;
 *         per-group scales must be applied inside the k-accumulation; bits per
 *         weight. Section 二.3: W4A16 reads INT4 weights, dequantizes them on chip
 *         and multiplies with 16-bit activations; the FLOPs are unchanged.
 *  [WIKI] "压缩算法" (cs-knowledge-wiki.pages.dev), section 7.4.1.1: z = round(-min/s);
 *         section 7.4.1.2: INT4 codes in [-8, 7], two codes packed per byte.
 *  [CH]   "量化：PTQ、GPTQ、AWQ 与 SmoothQuant" (charles2530.github.io), section 1:
 *         4-bit symmetric range {-8, ..., 7}.
 *  Act-order: [ARG] sections 五.3 and 十一.2 (see the act-order calls below).
 *  Per-channel INT8 (W8A16): include/q8.h.
 *
 * Conventions common to every call
 *  - Matrices are row-major. W is [out][in] float16 (a linear layer's weight,
 *    y = x W^T); x is [B][in] float16; y is [B][out] float16.
 *  - All pointers except `stream` are DEVICE pointers owned by the caller
 *    (q4_actorder_perm, a host helper, is the one exception). The library never
 *    allocates, frees or caches device memory; its only global state is a set of
 *    lock-guarded host caches of device properties (CU counts, occupancy), so
 *    calls are thread-safe and re-entrant.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue
 *    work on it and never synchronize.
 *  - Arguments are validated on the host before any HIP call; a failed check
 *    returns its status and enqueues nothing. A HIP launch error returns
 *    Q4_ERR_HIP. q4_last_error() describes the most recent failure on the
 *    calling thread.
 *  - Supported group sizes g: 32, 64 and every multiple of 128. `in` must be a
 *    positive multiple of g. `out` >= 1; `B` >= 0 (B = 0 enqueues nothing).
 *    out and in must each be below 2^30.
 *  - Non-finite weights give unspecified codes and scales (no scan is made).
 *
 * Device layout of the packed codes (opaque to callers; q4_to_canonical and
 * q4_from_canonical convert). With Np = ceil(out/16)*16, Kp = ceil(in/128)*128
 * and S = Kp/128, code (n, k) with t = n/16, r = n%16, s = k/128,
 * m = (k%128)/32, c = (k%32)/8, e = k%8 is the nibble p(e)%2 (0 = low) of byte
 *     ((t*S + s)*64 + r + 16*c)*16 + 4*m + p(e)/2,   p(e) = e/2 (e even), 4 + (e-1)/2 (e odd).
 * Symmetric codes are stored offset-binary (q + 8), asymmetric codes as q.
 * Rows >= out and channels >= in are padding holding code 0. Each 1 KiB block
 * is one 16-row x 128-channel tile: one 16-byte load per lane of a 64-lane
 * wavefront, already in the A-operand order of v_mfma_f32_16x16x32_f16.
 *
 * Device layout of per-group arrays (float16 scales, uint8 zero points): with
 * Gp = Kp/g, element (n, j) sits at index (t*Gp + j)*16 + r; padding is 0.
 *
 * Canonical layout (what q4_to_canonical returns): codes [out][in/2] bytes,
 * byte (n, i) = (c[n][2i] & 0xF) | (c[n][2i+1] & 0xF) << 4, symmetric codes in
 * 4-bit two's complement; scales [out][in/g] float16; zeros [out][in/g] uint8.
 */
#ifndef Q4_H
#define Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  Q4_OK = 0,
  Q4_ERR_NULL = 1,        /* a required pointer is NULL                                  */
  Q4_ERR_SHAPE = 2,       /* out/in/B out of range or overflowing                        */
  Q4_ERR_GROUP = 3,       /* group unsupported, or in % group != 0 ([YBB] section 二)    */
  Q4_ERR_ALIGN = 4,       /* a pointer is not aligned as the call requires               */
  Q4_ERR_UNSUPPORTED = 5, /* a valid request the library does not handle (e.g. config)    */
  Q4_ERR_WORKSPACE = 6,   /* workspace smaller than q4_workspace_bytes() asks for        */
  Q4_ERR_HIP = 7          /* a HIP runtime call or kernel launch failed                  */
} q4_status;

/* Static English description of a status code. Never NULL. */
const char* q4_status_str(int status);

/* Description of the last failure on the calling thread ("" if none). */
const char* q4_last_error(void);

/* Library version string, "q4 1.0.0 gfx950 src <hash>": <hash> identifies the
 * sources and flags the library was built from ("unknown" when built without them). */
const char* q4_version(void);

/* 1 if `group` is a supported group size, else 0. */
int32_t q4_group_supported(int32_t group);

/* Bytes of the device-layout packed code buffer for an [out][in] matrix:
 * ceil(out/16)*16 * ceil(in/128)*128 / 2. 0 if out or in is not positive. */
size_t q4_packed_bytes(int64_t out, int64_t in);

/* Elements of a device-layout per-group array (scales or zeros):
 * ceil(out/16)*16 * ceil(in/128)*128/group. 0 on invalid arguments. */
size_t q4_groups_count(int64_t out, int64_t in, int32_t group);

/* Symmetric quantize + pack ([YBB] section 二; [WIKI] section 7.4.1.2):
 *   s16[n][j] = float16_rne(float32(max_{k in group j} |W[n][k]|) / 7.0f)
 *   q[n][k]   = clamp(rint_half_even(float32(W[n][k]) / float32(s16)), -8, 7),
 *               q = 0 wherever s16 == 0 (an all-zero or underflowing group).
 * The codes are those of the IEEE float32 quotient rounded half to even (the
 * kernel reaches the same decision without a per-weight divide: one reciprocal
 * per group and an exact tie check). Writes q4_packed_bytes(out, in) bytes to `packed`
 * (16-byte aligned) and q4_groups_count(out, in, group) float16 to `scales`
 * (8-byte aligned), both in device layout, padding included. W: [out][in]
 * float16, 16-byte aligned. */
q4_status q4_quantize_pack(const void* W, int64_t out, int64_t in, int32_t group,
                           void* packed, void* scales, void* stream);

/* Asymmetric uint4 quantize + pack ([ARG] section 二.2; [WIKI] section 7.4.1.1):
 *   s16 = float16_rne(float32(float32(max) - float32(min)) / 15.0f)
 *   z   = clamp(rint(-min / s16), 0, 15),  q = clamp(rint(w / s16) + z, 0, 15),
 *   q = z = 0 wherever s16 == 0.  w_hat = s16 * (q - z).
 * As q4_quantize_pack, plus q4_groups_count() uint8 zero points in `zeros`. */
q4_status q4_quantize_pack_asym(const void* W, int64_t out, int64_t in, int32_t group,
                                void* packed, void* scales, void* zeros, void* stream);

/* Symmetric INT4 quantize + pack with the clipping search of [ARG] section 三.2:
 * per group, for p = min_percent .. 100 (alpha = float32(p) / 100.0f):
 *   s16_p = float16_rne(float32(max(float32(amax) * alpha, 1e-12f)) / 7.0f)
 *   q_p   = clamp(rint(w / s16_p), -7, 7)   (0 where s16_p == 0)
 *   err_p = sum over the group of (s16_p * q_p - w)^2   (float64 accumulation
 *           of float32-exact differences)
 * and the p with the smallest err_p is kept, equal errors going to the larger p;
 * min_percent = 100 gives exactly q4_quantize_pack's output. Output layout and
 * alignment as q4_quantize_pack (the GEMM reads it unchanged). group must be 32,
 * 64 or 128 and min_percent in 1..100, else Q4_ERR_UNSUPPORTED. */
q4_status q4_quantize_pack_clip(const void* W, int64_t out, int64_t in, int32_t group, int32_t min_percent,
                                void* packed, void* scales, void* stream);

/* Bytes of device workspace q4_gemm / q4_gemm_asym need for this shape: float32
 * partial sums when the channel range is split over several workgroups (a long
 * `in` with B <= 16, or too few rows to fill the GPU); 0 when none is needed. The
 * workspace is scratch: its contents on entry are ignored and undefined on return. */
size_t q4_workspace_bytes(int64_t B, int64_t out, int64_t in, int32_t group);

/* The launch shape q4_gemm picks for this product on the current device, as the
 * arguments q4_gemm_config takes to run the same launch: shape[0] = rows_per_wave,
 * shape[1] = waves_per_group, shape[2] = k_splits, shape[3] = col_tiles (4 int32
 * written on success). A host-side query that touches no device memory; it holds for
 * symmetric codes (q4_gemm_asym may pick another shape). Returns Q4_ERR_NULL for a
 * NULL shape, Q4_ERR_SHAPE for B outside [1, 2^30) and the errors of q4_gemm for
 * out, in and group. */
q4_status q4_gemm_shape(int64_t B, int64_t out, int64_t in, int32_t group, int32_t* shape);

/* Fused W4A16 product ([ARG] sections 二.2 and 二.3; [YBB] section 一):
 *   y[b][n] = float16_rne( sum_j s16[n][j] * sum_{k in group j} x[b][k] * q[n][k] )
 * with float16 x and codes, float32 accumulation, the group scale applied to
 * each group's partial sum inside the k-loop. Any B >= 0: B <= 16 runs the
 * GEMV kernel (one 16-column MFMA tile, padded), larger B the skinny-GEMM
 * tiling. x: [B][in] float16, 16-byte aligned; packed/scales as written by
 * q4_quantize_pack; y: [B][out] float16, 2-byte aligned.
 * `workspace` (16-byte aligned) must hold q4_workspace_bytes(B, out, in, group)
 * bytes; it may be NULL when that is 0, else Q4_ERR_WORKSPACE is returned.
 * Results are deterministic: partial sums are added in a fixed order. */
q4_status q4_gemm(const void* x, int64_t B, const void* packed, const void* scales,
                  int64_t out, int64_t in, int32_t group, void* y,
                  void* workspace, size_t workspace_bytes, void* stream);

/* q4_gemm for callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture that must not call hipMalloc, tight serving loops,
 * harnesses that forbid allocation). Same product, same kernels and same results as
 * q4_gemm; the split partial sums that q4_gemm keeps in the caller's workspace go to
 * a library-owned device array of Q4_NOALLOC_SCRATCH_BYTES instead, one per GPU,
 * reserved when the library is loaded and held until the process ends. The call
 * allocates nothing. Shapes needing more than that (q4_workspace_bytes(B, out, in,
 * group) > Q4_NOALLOC_SCRATCH_BYTES) return Q4_ERR_WORKSPACE. The array is shared by
 * every q4_gemm_noalloc call on a GPU and keeps the last call's contents (each call
 * overwrites what it reads): calls that overlap on one GPU, on different streams or
 * host threads, race and must be serialized by the caller. */
#define Q4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
q4_status q4_gemm_noalloc(const void* x, int64_t B, const void* packed, const void* scales,
                          int64_t out, int64_t in, int32_t group, void* y, void* stream);

/* As q4_gemm for asymmetric weights: the inner sum uses (q - z[n][j]). */
q4_status q4_gemm_asym(const void* x, int64_t B, const void* packed, const void* scales,
                       const void* zeros, int64_t out, int64_t in, int32_t group, void* y,
                       void* workspace, size_t workspace_bytes, void* stream);

/* q4_gemm with an explicit launch shape, for tuning. `asym` selects q4_gemm_asym
 * semantics (zeros used). Returns Q4_ERR_UNSUPPORTED for shapes the kernels
 * cannot run.
 * B <= 16 (GEMV): `rows_per_wave` row tiles of 16 per wavefront (1, 2 or 4),
 *   `waves_per_group` wavefronts per workgroup (1..16; at most 8 are used with
 *   group < 128 or rows_per_wave 4) sharing its work, `k_splits` workgroups
 *   splitting the channel range, `col_tiles` must be 1. The activation slice of
 *   one split must fit the device's LDS per workgroup. Needs
 *   k_splits * B * out * 4 bytes of workspace when k_splits > 1.
 * B > 16 (skinny GEMM): `rows_per_wave` 1, 2 or 4, `waves_per_group` 4 or 8
 *   (8 only with rows_per_wave <= 2),
 *   `col_tiles` 2, 3, 4, 6 or 8 tiles of 16 batch rows per workgroup, with
 *   rows_per_wave * col_tiles * max(1, 128 / group) <= 16 (accumulator
 *   registers), `k_splits` workgroups splitting the channel range in chunks of
 *   max(2, 8 / col_tiles) blocks of 128 (at most as many splits as chunks). Needs
 *   k_splits * B * out * 4 bytes of workspace when k_splits > 1. */
q4_status q4_gemm_config(const void* x, int64_t B, const void* packed, const void* scales,
                         const void* zeros, int32_t asym, int64_t out, int64_t in, int32_t group,
                         void* y, int32_t rows_per_wave, int32_t waves_per_group, int32_t k_splits,
                         int32_t col_tiles, void* workspace, size_t workspace_bytes, void* stream);

/* Device layout -> canonical layout (see above). `zeros`/`canon_zeros` are used
 * only when asym != 0. canon_codes: out*in/2 bytes; canon_scales: out*(in/group)
 * float16; canon_zeros: out*(in/group) bytes. */
q4_status q4_to_canonical(const void* packed, const void* scales, const void* zeros, int32_t asym,
                          int64_t out, int64_t in, int32_t group,
                          void* canon_codes, void* canon_scales, void* canon_zeros, void* stream);

/* Canonical layout -> device layout, padding included: imports codes and scales
 * produced elsewhere (e.g. by another quantizer with the same format). */
q4_status q4_from_canonical(const void* canon_codes, const void* canon_scales, const void* canon_zeros,
                            int32_t asym, int64_t out, int64_t in, int32_t group,
                            void* packed, void* scales, void* zeros, void* stream);

/* Measurement helper: read `bytes` (a positive multiple of 8192) from the device
 * buffer `buf` (16-byte aligned) with a plain streaming read kernel (one workgroup of
 * 4 wavefronts per CU, 8 KiB bursts per wavefront, pieces assigned round-robin: the
 * fastest plain read measured), so the GEMV's bytes / time can be compared with the read rate the same
 * device sustains ([YBB] section 一: decode is bound by the bytes it reads). `sink`
 * is a device uint32 the kernel writes only in a case random data never produces.
 * Returns Q4_ERR_SHAPE for other sizes, Q4_ERR_NULL / Q4_ERR_ALIGN as usual. */
q4_status q4_read_probe(const void* buf, size_t bytes, void* sink, void* stream);

/* Self-check of the quantizers' code decision on this device ([YBB] section 二:
 * q = round(w / scale), half to even). The quantizers take it from one hardware
 * reciprocal per scale and a tie test instead of a divide per weight; this runs that
 * decision on every positive finite float16 scale s and every finite float16 weight
 * w (31,743 x 63,488 = 2,015,299,584 pairs) against rint of the correctly rounded
 * float32 quotient, and counts the pairs with |w / s| < 341 (every clamp range used
 * lies inside) where the two differ. `counts` is a device array of two uint64 that
 * the call overwrites: counts[0] = pairs checked, counts[1] = mismatches (0 on a
 * correct device). Enqueued on `stream` (a few milliseconds); Q4_ERR_NULL and
 * Q4_ERR_ALIGN (8 bytes) as usual. */
q4_status q4_rtn_check(uint64_t* counts, void* stream);

/* ---- act-order (GPTQ desc_act) weights ----------------------------------------
 * [ARG] section 五.3: channels may be quantized in descending order of the Hessian
 * diagonal, groups of g being formed along that order, so a kernel needs a per-
 * channel group index g_idx[k]; section 十一.2: the reorder is a gather. The library
 * stores such weights with their input channels permuted so that every group is a
 * contiguous run of g columns (column i of the stored matrix is channel perm[i]),
 * and gathers the activations through perm inside the product. Scales keep the
 * group index: scale (n, j) belongs to the channels k with g_idx[k] == j. */

/* HOST function (host pointers, no HIP call): the permutation listing the channels
 * of group 0 in ascending order, then those of group 1, ...: perm[in] from
 * g_idx[in]. Every g_idx value must lie in [0, in/group) and every group must hold
 * exactly `group` channels, else Q4_ERR_SHAPE (nothing is written past the checks
 * that failed; perm's contents are then unspecified). Group rules as q4_quantize_pack. */
q4_status q4_actorder_perm(const int32_t* g_idx, int64_t in, int32_t group, int32_t* perm);

/* Symmetric INT4 quantize + pack of the column-permuted matrix W[:, perm]: as
 * q4_quantize_pack applied to the matrix whose column i is W[:, perm[i]], so group
 * j of the output holds channels perm[j*group .. (j+1)*group - 1]. perm: DEVICE
 * int32 [in], 16-byte aligned, a permutation of 0..in-1 (entries outside [0, in)
 * are clamped into the row: no out-of-bounds access, meaningless codes). */
q4_status q4_quantize_pack_perm(const void* W, int64_t out, int64_t in, int32_t group, const int32_t* perm,
                                void* packed, void* scales, void* stream);

/* Workspace q4_gemm_perm needs: the gathered activations (B * in * 2 bytes rounded
 * up to 256) followed by q4_workspace_bytes' split partials. */
size_t q4_workspace_bytes_perm(int64_t B, int64_t out, int64_t in, int32_t group);

/* Act-order product: y[b][n] = float16_rne( sum_j s16[n][j] * sum_{i in group j}
 * x[b][perm[i]] * q[n][i] ), i.e. x . W_hat^T with W_hat's channels in their
 * original order (each channel scaled by its group's scale, the g_idx gather).
 * packed/scales as written by q4_quantize_pack_perm with the same perm (DEVICE
 * int32 [in], 16-byte aligned). A gather kernel writes x[:, perm] into the
 * workspace, then the GEMV (B <= 16) or skinny GEMM runs on it unchanged; the
 * workspace is therefore always needed (q4_workspace_bytes_perm). Other arguments
 * as q4_gemm. */
q4_status q4_gemm_perm(const void* x, int64_t B, const void* packed, const void* scales, const int32_t* perm,
                       int64_t out, int64_t in, int32_t group, void* y, void* workspace, size_t workspace_bytes,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4_H */
