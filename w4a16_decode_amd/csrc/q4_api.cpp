// C ABI front end of libq4: argument validation, launch-shape selection and
// error reporting. Every check runs on the host before any HIP call, so an
// invalid request returns a status without touching the device.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "../../include/q4.h"
#include "q4_internal.h"

namespace {

thread_local char g_last_error[256] = "";

q4_status fail(q4_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
q4_status fail(q4_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

q4_status ok() {
  g_last_error[0] = '\0';
  return Q4_OK;
}

constexpr int64_t kMaxDim = int64_t(1) << 30;

bool group_ok(int32_t g) { return g == 32 || g == 64 || (g >= 128 && g % 128 == 0); }

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Dims {
  int N, K, group, Np, Kp, Gp;
};

q4_status check_dims(int64_t out, int64_t in, int32_t group, Dims* d) {
  if (out <= 0 || in <= 0 || out >= kMaxDim || in >= kMaxDim)
    return fail(Q4_ERR_SHAPE, "out=%lld, in=%lld: each must be in [1, 2^30)", (long long)out, (long long)in);
  if (!group_ok(group)) return fail(Q4_ERR_GROUP, "group %d unsupported (32, 64 or a multiple of 128)", (int)group);
  if (in % group != 0) return fail(Q4_ERR_GROUP, "in=%lld is not a multiple of group %d", (long long)in, (int)group);
  d->N = (int)out;
  d->K = (int)in;
  d->group = group;
  d->Np = (int)round_up(out, 16);
  d->Kp = (int)round_up(in, 128);
  d->Gp = d->Kp / group;
  if ((int64_t)d->Np * d->Kp / 2 > (int64_t(1) << 40))
    return fail(Q4_ERR_SHAPE, "matrix too large");
  return Q4_OK;
}

q4_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(Q4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Launch shape for y = x W^T with B rows (the kernel is described at the top of
// q4_gemm.hip). Aim for several thousand wavefronts so every CU keeps enough
// 16-byte loads in flight, with at least two 1 KiB blocks per wavefront.
void pick_shape(int B, const Dims& d, q4::GemmArgs* a) {
  const int T = d.Np / 16;
  const int S = d.Kp / 128;
  const int col_tiles_total = (B + 15) / 16;
  a->col_tiles = col_tiles_total <= 1 ? 1 : col_tiles_total == 2 ? 2 : 4;
  const int col_groups = (col_tiles_total + a->col_tiles - 1) / a->col_tiles;
  int R = (T >= 2048) ? 4 : (T >= 512 ? 2 : 1);
  if (a->col_tiles == 4 && R > 2) R = 2;
  const int64_t wgs = (int64_t)((T + R - 1) / R) * col_groups;
  int W = 1;
  while (W < 8 && wgs * W < 4096 && S / (2 * W) >= 1) W *= 2;
  while (W > 1 && (int64_t)W * R * a->col_tiles * 1024 > 64 * 1024) W /= 2;
  a->rows_per_wave = R;
  a->waves_per_group = W;
}

}  // namespace

extern "C" {

const char* q4_status_str(int status) {
  switch (status) {
    case Q4_OK: return "ok";
    case Q4_ERR_NULL: return "a required pointer is NULL";
    case Q4_ERR_SHAPE: return "invalid or overflowing shape";
    case Q4_ERR_GROUP: return "unsupported group size or in % group != 0";
    case Q4_ERR_ALIGN: return "misaligned pointer";
    case Q4_ERR_UNSUPPORTED: return "unsupported request";
    case Q4_ERR_WORKSPACE: return "workspace too small";
    case Q4_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* q4_last_error(void) { return g_last_error; }

const char* q4_version(void) { return "q4 1.0.0 gfx950"; }

int32_t q4_group_supported(int32_t group) { return group_ok(group) ? 1 : 0; }

size_t q4_packed_bytes(int64_t out, int64_t in) {
  if (out <= 0 || in <= 0 || out >= kMaxDim || in >= kMaxDim) return 0;
  return (size_t)(round_up(out, 16) * round_up(in, 128) / 2);
}

size_t q4_groups_count(int64_t out, int64_t in, int32_t group) {
  Dims d;
  if (check_dims(out, in, group, &d) != Q4_OK) return 0;
  return (size_t)d.Np * (size_t)d.Gp;
}

size_t q4_workspace_bytes(int64_t, int64_t, int64_t, int32_t) { return 0; }

static q4_status quantize_common(const void* W, int64_t out, int64_t in, int32_t group, void* packed, void* scales,
                                 void* zeros, bool asym, void* stream) {
  if (!W || !packed || !scales || (asym && !zeros)) return fail(Q4_ERR_NULL, "W, packed, scales%s must be non-NULL", asym ? ", zeros" : "");
  Dims d;
  q4_status st = check_dims(out, in, group, &d);
  if (st != Q4_OK) return st;
  if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(scales, 8))
    return fail(Q4_ERR_ALIGN, "W and packed need 16-byte, scales 8-byte alignment");
  q4::QuantArgs a{W, d.N, d.K, d.group, d.Np, d.Kp, d.Gp, asym, packed, scales, zeros};
  return hip_status(q4::launch_quantize(a, static_cast<hipStream_t>(stream)), "quantize launch");
}

q4_status q4_quantize_pack(const void* W, int64_t out, int64_t in, int32_t group, void* packed, void* scales,
                           void* stream) {
  return quantize_common(W, out, in, group, packed, scales, nullptr, false, stream);
}

q4_status q4_quantize_pack_asym(const void* W, int64_t out, int64_t in, int32_t group, void* packed, void* scales,
                                void* zeros, void* stream) {
  return quantize_common(W, out, in, group, packed, scales, zeros, true, stream);
}

static q4_status gemm_common(const void* x, int64_t B, const void* packed, const void* scales, const void* zeros,
                             bool asym, int64_t out, int64_t in, int32_t group, void* y, int rows_per_wave,
                             int waves_per_group, void* stream) {
  if (B < 0 || B >= kMaxDim) return fail(Q4_ERR_SHAPE, "B=%lld out of range", (long long)B);
  Dims d;
  q4_status st = check_dims(out, in, group, &d);
  if (st != Q4_OK) return st;
  if (B == 0) return ok();
  if (!x || !packed || !scales || !y || (asym && !zeros))
    return fail(Q4_ERR_NULL, "x, packed, scales, y%s must be non-NULL", asym ? ", zeros" : "");
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 8) || !aligned(y, 2))
    return fail(Q4_ERR_ALIGN, "x and packed need 16-byte, scales 8-byte, y 2-byte alignment");
  if ((int64_t)B * in >= (int64_t(1) << 40) || (int64_t)B * out >= (int64_t(1) << 40))
    return fail(Q4_ERR_SHAPE, "B*in or B*out too large");
  q4::GemmArgs a{};
  a.x = x;
  a.B = (int)B;
  a.packed = packed;
  a.scales = scales;
  a.zeros = zeros;
  a.asym = asym;
  a.N = d.N;
  a.K = d.K;
  a.group = d.group;
  a.Np = d.Np;
  a.Kp = d.Kp;
  a.Gp = d.Gp;
  a.y = y;
  pick_shape((int)B, d, &a);
  if (rows_per_wave > 0 || waves_per_group > 0) {
    if (rows_per_wave != 1 && rows_per_wave != 2 && rows_per_wave != 4)
      return fail(Q4_ERR_UNSUPPORTED, "rows_per_wave must be 1, 2 or 4");
    if (waves_per_group < 1 || waves_per_group > 8)
      return fail(Q4_ERR_UNSUPPORTED, "waves_per_group must be in [1, 8]");
    if ((int64_t)waves_per_group * rows_per_wave * a.col_tiles * 1024 > 64 * 1024)
      return fail(Q4_ERR_UNSUPPORTED, "waves_per_group * rows_per_wave * column tiles exceeds the 64 KiB reduction buffer");
    a.rows_per_wave = rows_per_wave;
    a.waves_per_group = waves_per_group;
  }
  return hip_status(q4::launch_gemm(a, static_cast<hipStream_t>(stream)), "gemm launch");
}

q4_status q4_gemm(const void* x, int64_t B, const void* packed, const void* scales, int64_t out, int64_t in,
                  int32_t group, void* y, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  return gemm_common(x, B, packed, scales, nullptr, false, out, in, group, y, 0, 0, stream);
}

q4_status q4_gemm_asym(const void* x, int64_t B, const void* packed, const void* scales, const void* zeros,
                       int64_t out, int64_t in, int32_t group, void* y, void* workspace, size_t workspace_bytes,
                       void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  return gemm_common(x, B, packed, scales, zeros, true, out, in, group, y, 0, 0, stream);
}

q4_status q4_gemm_config(const void* x, int64_t B, const void* packed, const void* scales, const void* zeros,
                         int32_t asym, int64_t out, int64_t in, int32_t group, void* y, int32_t rows_per_wave,
                         int32_t waves_per_group, void* stream) {
  if (rows_per_wave <= 0 || waves_per_group <= 0)
    return fail(Q4_ERR_UNSUPPORTED, "rows_per_wave and waves_per_group must be positive");
  return gemm_common(x, B, packed, scales, zeros, asym != 0, out, in, group, y, rows_per_wave, waves_per_group,
                     stream);
}

q4_status q4_to_canonical(const void* packed, const void* scales, const void* zeros, int32_t asym, int64_t out,
                          int64_t in, int32_t group, void* canon_codes, void* canon_scales, void* canon_zeros,
                          void* stream) {
  if (!packed || !scales || !canon_codes || !canon_scales || (asym && (!zeros || !canon_zeros)))
    return fail(Q4_ERR_NULL, "a required pointer is NULL");
  Dims d;
  q4_status st = check_dims(out, in, group, &d);
  if (st != Q4_OK) return st;
  if (!aligned(packed, 4) || !aligned(scales, 2) || !aligned(canon_scales, 2))
    return fail(Q4_ERR_ALIGN, "packed needs 4-byte, scales 2-byte alignment");
  q4::LayoutArgs a{d.N, d.K, d.group, d.Np, d.Kp, d.Gp, asym != 0, const_cast<void*>(packed),
                   const_cast<void*>(scales), const_cast<void*>(zeros), canon_codes, canon_scales, canon_zeros};
  return hip_status(q4::launch_to_canonical(a, static_cast<hipStream_t>(stream)), "to_canonical launch");
}

q4_status q4_from_canonical(const void* canon_codes, const void* canon_scales, const void* canon_zeros,
                            int32_t asym, int64_t out, int64_t in, int32_t group, void* packed, void* scales,
                            void* zeros, void* stream) {
  if (!packed || !scales || !canon_codes || !canon_scales || (asym && (!zeros || !canon_zeros)))
    return fail(Q4_ERR_NULL, "a required pointer is NULL");
  Dims d;
  q4_status st = check_dims(out, in, group, &d);
  if (st != Q4_OK) return st;
  if (!aligned(packed, 4) || !aligned(scales, 2) || !aligned(canon_scales, 2))
    return fail(Q4_ERR_ALIGN, "packed needs 4-byte, scales 2-byte alignment");
  q4::LayoutArgs a{d.N, d.K, d.group, d.Np, d.Kp, d.Gp, asym != 0, packed, scales, zeros,
                   const_cast<void*>(canon_codes), const_cast<void*>(canon_scales), const_cast<void*>(canon_zeros)};
  return hip_status(q4::launch_from_canonical(a, static_cast<hipStream_t>(stream)), "from_canonical launch");
}

}  // extern "C"
