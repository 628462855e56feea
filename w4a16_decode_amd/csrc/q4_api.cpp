// C ABI front end of libq4: argument validation, launch-shape selection and
// error reporting. Every check runs on the host before any HIP call, so an
// invalid request returns a status without touching the device.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include <hip/hip_runtime.h>

#include "../../include/q4.h"
#include "../../include/q8.h"
#include "../../include/q4_kv.h"
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
static_assert(Q4_NOALLOC_SCRATCH_BYTES == q4::kNoAllocScratchBytes, "q4.h and the scratch array agree");

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

// Launch shape for y = x W^T with B rows (the kernels are described at the top of
// q4_gemm.hip). B <= 16 runs the persistent GEMV kernel: every workgroup keeps its
// slice of x (B rows x its channel range) in LDS next to its wavefronts' partial
// sums, so the channel range is split over KS workgroups until that fits the
// device's LDS.
constexpr int kGemvXChunks = 8;          // x chunks of 16 B per thread (kXChunksPerThread)
constexpr size_t kLdsFallback = 64 * 1024;

// LDS a workgroup may allocate on the current device (64 KiB if it cannot be queried).
size_t lds_per_block() {
  static std::mutex mu;
  static std::map<int, size_t> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return kLdsFallback;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int v = 0;
  size_t lim = kLdsFallback;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0)
    lim = (size_t)v;
  cache[dev] = lim;
  return lim;
}

// LDS of one GEMV workgroup with a single unit of work (q4_gemm.hip, GemvLds): x
// slice + zero row, the per-unit biases of symmetric codes, the partial sums of
// one unit and the unit counter. The launch fits as many units as the limit holds.
size_t gemv_lds(int B, int S, int KS, int R, int group, bool asym) {
  const size_t nsb = (size_t)((S + KS - 1) / KS);
  const size_t gsub = group >= 128 ? 1 : (size_t)(128 / group);
  const size_t x = (((size_t)B * (nsb * 128 + q4::kGemmRowPad) + 128) * 2 + 15) & ~(size_t)15;
  const size_t beta = asym ? 0 : ((size_t)B * nsb * gsub + 1 + 3) / 4 * 4 * sizeof(float);
  return x + beta + (size_t)R * 16 * B * 4 + 16;
}

// Wavefronts a GEMV workgroup runs with (gemv_max_waves in q4_gemm.hip).
int gemv_max_waves(int R, int group, bool q8 = false) { return (group < 128 || R > 2 || (q8 && R > 1)) ? 8 : 16; }

bool gemv_shape_ok(int B, int S, int KS, int W, int R, int group, bool asym, size_t lds_limit, bool q8 = false) {
  if (KS < 1 || KS > S || W < 1 || W > 16) return false;
  W = std::min(W, gemv_max_waves(R, group, q8));
  const int nsb = (S + KS - 1) / KS;
  if (gemv_lds(B, S, KS, R, group, asym) > lds_limit) return false;
  return (int64_t)B * nsb * 16 <= (int64_t)kGemvXChunks * W * 64;
}

// Modelled time (us) of a GEMV launch shape at 4 <= B <= 16 (symmetric INT4 codes,
// one scale per block): a linear model of the busiest CU's work, fitted to launches of
// every shape R in {1, 2}, W in {8, 16}, KS in {1, 2, 4, 8} on 16 weight matrices
// (1024 to 57344 rows, 4096 to 28672 channels) at B = 4 to 16 on MI355X. Terms: KiB
// of codes the busiest CU streams (0.0555 us each, 4.7 TB/s over 256 CUs); KiB of
// activations it stages into LDS before streaming (0.0263 us each); the separate
// split reduction (1.99 us, plus 0.92 us per MB of float32 partials); and a credit
// for longer streams per wavefront (-0.297 us per KiB of codes per wavefront).
// Picking the lowest-cost shape came within 1.4% on average (10.7% at worst) of the
// fastest measured shape of each matrix and batch size.
double gemv_model_us(int B, int T, int S, int N, int R, int W, int KS, size_t lds, size_t lds_limit, int cus) {
  const int64_t nRB = (T + R - 1) / R;
  const int64_t nsb = (S + KS - 1) / KS;
  const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(16 / W, (int64_t)(lds_limit / std::max<size_t>(lds, 1))));
  const int64_t per_split = std::max<int64_t>(1, std::min<int64_t>(nRB, per_cu * cus / KS));
  const int64_t n_rb = (nRB + per_split - 1) / per_split;
  const int64_t wgs_cu = (per_split * KS + cus - 1) / cus;  // workgroups on the busiest CU
  const double codes = (double)(n_rb * R * nsb * wgs_cu);  // KiB
  const double xs = (double)B * nsb / 4.0 * wgs_cu;        // KiB
  const double red = KS > 1 ? 1.99 + 0.92 * ((double)KS * B * N * 4 / 1e6) : 0.0;
  return 0.0555 * codes + 0.0263 * xs + red - 0.297 * codes / (W * wgs_cu);
}

// LDS of one skinny-GEMM workgroup (q4_internal.h).
size_t mfma_lds(int col_tiles) { return q4::mfma_lds_bytes(col_tiles); }

// Modelled time (us) of a skinny-GEMM launch shape (symmetric INT4 codes, one scale
// per block, 8 wavefronts per workgroup): a linear model of the busiest CU's work,
// fitted to launches of every shape R in {1, 2}, KS in {1, 2, 3, 4, 6, 8}, CT in
// {2, 3, 4, 6, 8} on 9 weight matrices (4096 to 57344 rows, 4096 to 28672 channels) at
// B = 17 to 256 on MI355X. Terms: KiB of codes the busiest CU streams and dequantizes
// (0.0035 us each), the same times the column tiles (its MFMA work, 0.0060 us), the
// activation tile-blocks it stages into LDS (0.098 us each), the separate split
// reduction (0.69 us, plus 0.74 us per MB of float32 partials), the KiB of codes per
// wavefront the CU holds at once (0.155 us: latency that fewer resident wavefronts
// leave exposed) and a constant 7.3 us. Picking the lowest-cost shape came within 0.4%
// on average (11.6% at worst) of the fastest measured shape of each matrix and batch
// size, and 8.7% faster on average than the earlier fixed rules (3% slower at worst).
double skinny_model_us(int B, int T, int S, int N, int R, int KS, int CT, int per_cu, int cus) {
  const int nb = q4::mfma_chunk_blocks(CT);
  const int64_t chunks = (S + nb - 1) / nb;
  const int64_t nsb = std::min<int64_t>(S, (chunks + KS - 1) / KS * nb);  // blocks per split
  const int64_t groups = ((B + 15) / 16 + CT - 1) / CT;
  const int64_t G = (T + 8 * R - 1) / (8 * R) * groups * KS;
  const int64_t wg = (G + cus - 1) / cus;  // workgroups on the busiest CU
  const double codes = (double)(wg * 8 * R * nsb);  // KiB
  const double staged = (double)(wg * CT * nsb);
  const double conc = (double)std::min<int64_t>(wg, std::max(per_cu, 1));
  const double red = KS > 1 ? 0.68698 + 0.73563 * ((double)KS * B * N * 4 / 1e6) : 0.0;
  return 0.0035114 * codes + 0.0059675 * codes * CT + 0.097773 * staged + red + 0.15473 * codes / (8 * conc) +
         7.3183;
}

// Skinny GEMM launch shapes: R x CT accumulator tiles and one partial tile per
// group of a 128-channel block must fit the registers, the two activation tiles
// the LDS, and every k-split must get at least one chunk (q4::mfma_chunk_blocks).
bool mfma_shape_ok(int R, int W, int KS, int CT, int group, int S, bool q8 = false) {
  if (W != 4 && W != 8) return false;
  if (W == 8 && R > 2) return false;
  if (R != 1 && R != 2 && R != 4) return false;
  // INT8 codes stage twice the bytes per block: the ring of one chunk must fit
  if (q8 && (R == 4 || (R == 2 && CT == 2))) return false;
  if (CT != 2 && CT != 3 && CT != 4 && CT != 6 && CT != 8) return false;
  const int nb = q4::mfma_chunk_blocks(CT);
  const int chunks = (S + nb - 1) / nb;
  if (KS < 1 || KS > chunks) return false;
  const int gsub = group >= 128 ? 1 : 128 / group;
  return R * CT * gsub <= 16 && mfma_lds(CT) <= lds_per_block();
}

void pick_shape(int B, const Dims& d, q4::GemmArgs* a) {
  const int T = d.Np / 16;
  const int S = d.Kp / 128;
  const int col_tiles_total = (B + 15) / 16;
  if (B <= 16) {
    // a workgroup may use the CU's whole LDS (the activation slice decides how many
    // stay resident per CU)
    const size_t lim = lds_per_block();
    a->col_tiles = 1;
    // two row tiles per wavefront for square-ish matrices of 512 to 2047 tiles (the
    // extra tile per load keeps more bytes in flight where there are few row
    // blocks), else one: tall matrices, small groups (several scales per block) and
    // matrices so small that two tiles per row block would leave CUs idle
    // (INT8 codes: always one; 2 KiB blocks already keep 6 KiB per wavefront in flight)
    const int R = (a->q8 || T >= 2048 || d.group < 128 || T > S * 8 || T < 512) ? 1 : 2;
    // 8 wavefronts (two workgroups per CU) stream best for B <= 4; 16 hold twice
    // the activation slice, which keeps larger batches from splitting the channels.
    // At B <= 2 on short rows (<= 4096 channels; INT8 codes: <= 8192 channels and
    // fewer than 1024 row tiles) 4 wavefronts: twice the workgroups, and units long
    // enough that every wavefront keeps streaming.
    const bool w4 = B <= 2 && (S <= 32 || (a->q8 && T < 1024 && S <= 64));
    const int W = w4 ? 4 : B <= 4 ? 8 : gemv_max_waves(R, d.group, a->q8);
    int KS = 1;
    // two row tiles per wavefront at B <= 3 stream x per unit (no activation slice
    // to fit in LDS, so no channel split); otherwise the fewest splits whose slice fits
    // (B = 4 takes the model's pick below; the launch streams x where that pick is two
    // row tiles without a split and the burst form runs)
    const bool streamed = !a->q8 && B <= 3 && q4::gemv_streams_x(B, d.Kp, R, 1, false);
    while (!streamed && KS < S && !gemv_shape_ok(B, S, KS, W, R, d.group, a->asym, lim, a->q8)) ++KS;
    a->rows_per_wave = R;
    a->waves_per_group = W;
    a->k_splits = KS;
    a->lds_limit = lim;
    if (B >= 4 && !streamed && !a->q8 && !a->asym && d.group >= 128) {
      // the shape of lowest modelled time (gemv_model_us); ties keep fewer splits
      const int cus = q4::device_cu_count_cached();
      double best = 1e30;
      for (int ks : {1, 2, 4, 8})
        for (int r : {1, 2})
          for (int w : {8, 16}) {
            if (ks > S || !gemv_shape_ok(B, S, ks, w, r, d.group, false, lim)) continue;
            const double t = gemv_model_us(B, T, S, d.Np, r, w, ks, gemv_lds(B, S, ks, r, d.group, false), lim, cus);
            if (t < best) {
              best = t;
              a->rows_per_wave = r;
              a->waves_per_group = w;
              a->k_splits = ks;
            }
          }
    }
    return;
  }
  // B > 16: skinny MFMA GEMM, 8 wavefronts per workgroup sharing CT column tiles of
  // 16 batch rows (double-buffered activation chunks in LDS). Symmetric INT4 codes
  // with one scale per block or fewer take the shape of lowest modelled time
  // (skinny_model_us). Asymmetric codes, groups of 32 or 64 and INT8 codes keep fixed
  // rules: 2 column tiles up to B = 32, 4 up to 128 (8 when that needs more than 256
  // workgroups), else 8; 2 row
  // tiles per wavefront; the channel range split over up to `cap` workgroups (8 for
  // rows of >= 112 blocks, else 4) until there are about 256 of them, with 1 row tile
  // per wavefront when even that leaves too few. Short rows (<= 64 blocks) at B > 128
  // take 2 column tiles and no split where that gives at most 256 workgroups: the
  // column groups re-read a matrix that small from the caches, and no reduction runs
  // (6144x4096 at B = 256: 31 vs 42 us; 8192x8192: 54 vs 59 us). Measured on a grid of
  // launch shapes over 7 matrices at B = 17-256: within 1.2% of the fastest measured
  // shape on average (the rule without the two refinements: 6.1%).
  if (!a->q8 && !a->asym && d.group >= 128) {
    // the shape of lowest modelled time (skinny_model_us); column tiles that would
    // leave two or more 16-row tiles of one group empty are not considered; ties keep
    // the first in the order column tiles, row tiles, splits
    const int cus = q4::device_cu_count_cached();
    double best = 1e30;
    for (int ct : {2, 3, 4, 6, 8}) {
      if (ct > 2 && ct > col_tiles_total + 1) continue;
      for (int r : {1, 2}) {
        if (!mfma_shape_ok(r, 8, 1, ct, d.group, S)) continue;
        const int per_cu = q4::mfma_resident_per_cu(r, ct);
        for (int ks : {1, 2, 3, 4, 6, 8}) {
          if (!mfma_shape_ok(r, 8, ks, ct, d.group, S)) continue;
          const double t = skinny_model_us(B, T, S, d.N, r, ks, ct, per_cu, cus);
          if (t < best) {
            best = t;
            a->rows_per_wave = r;
            a->waves_per_group = 8;
            a->k_splits = ks;
            a->col_tiles = ct;
          }
        }
      }
    }
    if (best < 1e30) return;
  }
  const int64_t rw2 = (T + 15) / 16;  // row workgroups at 2 row tiles per wavefront
  if (S <= 64 && col_tiles_total > 8 && rw2 * ((col_tiles_total + 1) / 2) <= 256 &&
      mfma_shape_ok(2, 8, 1, 2, d.group, S, a->q8)) {
    a->col_tiles = 2;
    a->rows_per_wave = 2;
    a->waves_per_group = 8;
    a->k_splits = 1;
    return;
  }
  const int cap = S >= 112 ? 8 : 4;
  int CT = col_tiles_total <= 2 ? 2 : (col_tiles_total <= 8 ? 4 : 8);
  int R = 2;
  auto wgs = [&](int r) { return (int64_t)((T + 8 * r - 1) / (8 * r)) * ((col_tiles_total + CT - 1) / CT); };
  if (256 / wgs(R) > cap) R = 1;
  while (!mfma_shape_ok(R, 8, 1, CT, d.group, S, a->q8)) {
    if (R > 1) R /= 2;
    else if (CT > 2) CT /= 2;
    else break;  // unreachable: R = 1, CT = 2 always fits
  }
  // where the grid would need a second, partial round (57344 rows at B = 128: 448
  // workgroups), wider column groups halve it (gate/up at B = 128: INT4 175 -> 149 us, INT8
  // 215 -> 168 us)
  while (CT < 8 && CT < col_tiles_total && wgs(R) > 256 && mfma_shape_ok(R, 8, 1, CT * 2, d.group, S, a->q8)) CT *= 2;
  int KS = (int)std::min<int64_t>(cap, std::max<int64_t>(1, 256 / wgs(R)));
  while (KS > 1 && !mfma_shape_ok(R, 8, KS, CT, d.group, S, a->q8)) --KS;
  a->col_tiles = CT;
  a->rows_per_wave = R;
  a->waves_per_group = 8;
  a->k_splits = KS;
}

size_t splits_workspace(const q4::GemmArgs& a) {
  return a.k_splits > 1 ? (size_t)a.k_splits * a.B * a.N * sizeof(float) : 0;
}

// Act-order products gather x into the front of the workspace first.
size_t perm_x_bytes(int64_t B, int64_t in) { return (size_t)round_up(B * in * 2, 256); }

}  // namespace

namespace q4 {

namespace {
int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  return dev;
}
std::mutex g_dev_mu;
std::map<int, int> g_cus;                                              // device -> CUs
std::map<std::tuple<const void*, int, size_t, int>, int> g_resident;  // (kernel, block, lds, device) -> per CU
}  // namespace

int device_cu_count_cached() {
  const int dev = current_device();
  std::lock_guard<std::mutex> lk(g_dev_mu);
  auto it = g_cus.find(dev);
  if (it != g_cus.end()) return it->second;
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1) v = 256;
  g_cus[dev] = v;
  return v;
}

int resident_per_cu(const void* fn, int block, size_t lds) {
  const auto key = std::make_tuple(fn, block, lds, current_device());
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    auto it = g_resident.find(key);
    if (it != g_resident.end()) return it->second;
  }
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, block, lds) != hipSuccess || nb < 1) nb = 1;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  g_resident[key] = nb;
  return nb;
}

int resident_grid(const void* fn, int block) { return resident_per_cu(fn, block, 0) * device_cu_count_cached(); }

}  // namespace q4

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

#ifndef Q4_SOURCE_HASH
#define Q4_SOURCE_HASH "unknown"
#endif
const char* q4_version(void) { return "q4 1.0.0 gfx950 src " Q4_SOURCE_HASH; }

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

// The larger of the split workspaces q4_gemm and q4_gemm_asym need: the two may pick
// different launch shapes (symmetric codes stream x at B = 4 where asymmetric ones split).
static size_t splits_workspace_any(int64_t B, const Dims& d) {
  size_t need = 0;
  for (bool asym : {false, true}) {
    q4::GemmArgs a{};
    a.B = (int)B;
    a.N = d.N;
    a.asym = asym;
    pick_shape((int)B, d, &a);
    need = std::max(need, splits_workspace(a));
  }
  return need;
}

size_t q4_workspace_bytes(int64_t B, int64_t out, int64_t in, int32_t group) {
  Dims d;
  if (B <= 0 || B >= kMaxDim || check_dims(out, in, group, &d) != Q4_OK) return 0;
  return splits_workspace_any(B, d);
}

q4_status q4_gemm_shape(int64_t B, int64_t out, int64_t in, int32_t group, int32_t* shape) {
  if (shape == nullptr) return fail(Q4_ERR_NULL, "shape is NULL");
  if (B <= 0 || B >= kMaxDim) return fail(Q4_ERR_SHAPE, "B=%lld must be in [1, 2^30)", (long long)B);
  Dims d;
  q4_status st = check_dims(out, in, group, &d);
  if (st != Q4_OK) return st;
  q4::GemmArgs a{};
  a.B = (int)B;
  a.N = d.N;
  pick_shape((int)B, d, &a);
  shape[0] = a.rows_per_wave;
  shape[1] = a.waves_per_group;
  shape[2] = a.k_splits;
  shape[3] = a.col_tiles;
  return ok();
}

static q4_status quantize_common(const void* W, int64_t out, int64_t in, int32_t group, void* packed, void* scales,
                                 void* zeros, bool asym, int clip_pmin, void* stream, const int32_t* perm = nullptr) {
  if (!W || !packed || !scales || (asym && !zeros)) return fail(Q4_ERR_NULL, "W, packed, scales%s must be non-NULL", asym ? ", zeros" : "");
  Dims d;
  q4_status st = check_dims(out, in, group, &d);
  if (st != Q4_OK) return st;
  if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(scales, 8))
    return fail(Q4_ERR_ALIGN, "W and packed need 16-byte, scales 8-byte alignment");
  q4::QuantArgs a{W, d.N, d.K, d.group, d.Np, d.Kp, d.Gp, asym, packed, scales, zeros, clip_pmin, perm};
  return hip_status(q4::launch_quantize(a, static_cast<hipStream_t>(stream)), "quantize launch");
}

q4_status q4_quantize_pack(const void* W, int64_t out, int64_t in, int32_t group, void* packed, void* scales,
                           void* stream) {
  return quantize_common(W, out, in, group, packed, scales, nullptr, false, 0, stream);
}

q4_status q4_quantize_pack_asym(const void* W, int64_t out, int64_t in, int32_t group, void* packed, void* scales,
                                void* zeros, void* stream) {
  return quantize_common(W, out, in, group, packed, scales, zeros, true, 0, stream);
}

q4_status q4_quantize_pack_clip(const void* W, int64_t out, int64_t in, int32_t group, int32_t min_percent,
                                void* packed, void* scales, void* stream) {
  if (min_percent < 1 || min_percent > 100) return fail(Q4_ERR_UNSUPPORTED, "min_percent=%d not in 1..100", (int)min_percent);
  if (group != 32 && group != 64 && group != 128)
    return fail(Q4_ERR_UNSUPPORTED, "the clipping search runs for group 32, 64 or 128 (got %d)", (int)group);
  return quantize_common(W, out, in, group, packed, scales, nullptr, false, min_percent, stream);
}

static q4_status gemm_common(const void* x, int64_t B, const void* packed, const void* scales, const void* zeros,
                             bool asym, int64_t out, int64_t in, int32_t group, void* y, int rows_per_wave,
                             int waves_per_group, int k_splits, int col_tiles, void* workspace,
                             size_t workspace_bytes, void* stream, const int32_t* perm = nullptr,
                             bool noalloc = false) {
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
  a.perm = perm;
  pick_shape((int)B, d, &a);
  if (rows_per_wave > 0 || waves_per_group > 0 || k_splits > 0 || col_tiles > 0) {
    if (rows_per_wave != 1 && rows_per_wave != 2 && rows_per_wave != 4)
      return fail(Q4_ERR_UNSUPPORTED, "rows_per_wave must be 1, 2 or 4");
    if (waves_per_group < 1 || waves_per_group > 16)
      return fail(Q4_ERR_UNSUPPORTED, "waves_per_group must be in [1, 16]");
    if (B <= 16) {
      if (col_tiles != 1) return fail(Q4_ERR_UNSUPPORTED, "col_tiles must be 1 for B <= 16");
      a.lds_limit = lds_per_block();
      // the streaming kernel (two row tiles, B <= 3, no split) stages no activation slice
      const bool streamed = q4::gemv_streams_x(
          (int)B, d.Kp, rows_per_wave, k_splits,
          q4::gemv_stream_burst_ok(d.Np, d.group, asym != 0, false, q4::device_cu_count_cached()));
      if (!streamed &&
          !gemv_shape_ok((int)B, d.Kp / 128, k_splits, waves_per_group, rows_per_wave, d.group, asym, a.lds_limit))
        return fail(Q4_ERR_UNSUPPORTED, "k_splits=%d, waves_per_group=%d: more splits than 128-channel blocks, "
                    "or the activation slice of B=%lld does not fit LDS or the copy",
                    (int)k_splits, (int)waves_per_group, (long long)B);
    } else if (!mfma_shape_ok(rows_per_wave, waves_per_group, k_splits, col_tiles, d.group, d.Kp / 128)) {
      return fail(Q4_ERR_UNSUPPORTED, "for B > 16: waves_per_group must be 4 or 8 (8 only with rows_per_wave <= 2), "
                  "col_tiles 2, 3, 4, 6 or 8 (within LDS), "
                  "rows_per_wave * col_tiles * max(1, 128 / group) <= 16, k_splits at most the chunks of "
                  "max(2, 8 / col_tiles) blocks");
    }
    a.col_tiles = col_tiles;
    a.rows_per_wave = rows_per_wave;
    a.waves_per_group = waves_per_group;
    a.k_splits = k_splits;
  }
  const size_t need = splits_workspace(a) + (perm ? perm_x_bytes(B, in) : 0);
  if (noalloc) {
    // the library's own scratch array stands in for the workspace
    if (need > q4::kNoAllocScratchBytes)
      return fail(Q4_ERR_WORKSPACE, "this shape needs %zu bytes of scratch, more than the %zu q4_gemm_noalloc holds",
                  need, q4::kNoAllocScratchBytes);
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      q4_status st2 = hip_status(q4::noalloc_scratch(&workspace), "scratch address lookup");
      if (st2 != Q4_OK) return st2;
      workspace_bytes = q4::kNoAllocScratchBytes;
    }
  }
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(Q4_ERR_WORKSPACE, "this shape needs %zu bytes of workspace (q4_workspace_bytes%s), got %zu", need,
                  perm ? "_perm" : "", workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(Q4_ERR_ALIGN, "workspace needs 16-byte alignment");
  }
  a.workspace = workspace;
  return hip_status(q4::launch_gemm(a, static_cast<hipStream_t>(stream)), "gemm launch");
}

q4_status q4_gemm(const void* x, int64_t B, const void* packed, const void* scales, int64_t out, int64_t in,
                  int32_t group, void* y, void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_common(x, B, packed, scales, nullptr, false, out, in, group, y, 0, 0, 0, 0, workspace, workspace_bytes,
                     stream);
}

q4_status q4_gemm_noalloc(const void* x, int64_t B, const void* packed, const void* scales, int64_t out, int64_t in,
                          int32_t group, void* y, void* stream) {
  return gemm_common(x, B, packed, scales, nullptr, false, out, in, group, y, 0, 0, 0, 0, nullptr, 0, stream, nullptr,
                     true);
}

q4_status q4_gemm_asym(const void* x, int64_t B, const void* packed, const void* scales, const void* zeros,
                       int64_t out, int64_t in, int32_t group, void* y, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return gemm_common(x, B, packed, scales, zeros, true, out, in, group, y, 0, 0, 0, 0, workspace, workspace_bytes,
                     stream);
}

q4_status q4_gemm_config(const void* x, int64_t B, const void* packed, const void* scales, const void* zeros,
                         int32_t asym, int64_t out, int64_t in, int32_t group, void* y, int32_t rows_per_wave,
                         int32_t waves_per_group, int32_t k_splits, int32_t col_tiles, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (rows_per_wave <= 0 || waves_per_group <= 0 || k_splits <= 0 || col_tiles <= 0)
    return fail(Q4_ERR_UNSUPPORTED, "rows_per_wave, waves_per_group, k_splits and col_tiles must be positive");
  return gemm_common(x, B, packed, scales, zeros, asym != 0, out, in, group, y, rows_per_wave, waves_per_group,
                     k_splits, col_tiles, workspace, workspace_bytes, stream);
}

// ---- act-order (g_idx) --------------------------------------------------------

q4_status q4_actorder_perm(const int32_t* g_idx, int64_t in, int32_t group, int32_t* perm) {
  if (!g_idx || !perm) return fail(Q4_ERR_NULL, "g_idx and perm must be non-NULL");
  if (in <= 0 || in >= kMaxDim) return fail(Q4_ERR_SHAPE, "in=%lld must be in [1, 2^30)", (long long)in);
  if (!group_ok(group)) return fail(Q4_ERR_GROUP, "group %d unsupported (32, 64 or a multiple of 128)", (int)group);
  if (in % group != 0) return fail(Q4_ERR_GROUP, "in=%lld is not a multiple of group %d", (long long)in, (int)group);
  const int64_t G = in / group;
  std::vector<int64_t> start(G + 1, 0);  // counting sort: group sizes, then offsets
  for (int64_t k = 0; k < in; ++k) {
    const int64_t j = g_idx[k];
    if (j < 0 || j >= G)
      return fail(Q4_ERR_SHAPE, "g_idx[%lld] = %lld outside [0, %lld)", (long long)k, (long long)j, (long long)G);
    ++start[j + 1];
  }
  for (int64_t j = 0; j < G; ++j) {
    if (start[j + 1] != group)
      return fail(Q4_ERR_SHAPE, "group %lld holds %lld channels, not %d", (long long)j, (long long)start[j + 1],
                  (int)group);
    start[j + 1] += start[j];
  }
  for (int64_t k = 0; k < in; ++k) perm[start[g_idx[k]]++] = (int32_t)k;
  return ok();
}

q4_status q4_quantize_pack_perm(const void* W, int64_t out, int64_t in, int32_t group, const int32_t* perm,
                                void* packed, void* scales, void* stream) {
  if (!perm) return fail(Q4_ERR_NULL, "perm must be non-NULL");
  if (!aligned(perm, 16)) return fail(Q4_ERR_ALIGN, "perm needs 16-byte alignment");
  return quantize_common(W, out, in, group, packed, scales, nullptr, false, 0, stream, perm);
}

size_t q4_workspace_bytes_perm(int64_t B, int64_t out, int64_t in, int32_t group) {
  Dims d;
  if (B <= 0 || B >= kMaxDim || check_dims(out, in, group, &d) != Q4_OK) return 0;
  return splits_workspace_any(B, d) + perm_x_bytes(B, in);
}

q4_status q4_gemm_perm(const void* x, int64_t B, const void* packed, const void* scales, const int32_t* perm,
                       int64_t out, int64_t in, int32_t group, void* y, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (B > 0 && !perm) return fail(Q4_ERR_NULL, "perm must be non-NULL");
  if (perm && !aligned(perm, 16)) return fail(Q4_ERR_ALIGN, "perm needs 16-byte alignment");
  return gemm_common(x, B, packed, scales, nullptr, false, out, in, group, y, 0, 0, 0, 0, workspace, workspace_bytes,
                     stream, perm);
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

// ---- per-channel INT8 (W8A16) ------------------------------------------------

static q4_status check_w8_dims(int64_t out, int64_t in, Dims* d) {
  if (out <= 0 || in <= 0 || out >= kMaxDim || in >= kMaxDim)
    return fail(Q4_ERR_SHAPE, "out=%lld, in=%lld: each must be in [1, 2^30)", (long long)out, (long long)in);
  if (in % 8 != 0) return fail(Q4_ERR_SHAPE, "in=%lld must be a multiple of 8", (long long)in);
  d->N = (int)out;
  d->K = (int)in;
  d->Np = (int)round_up(out, 16);
  d->Kp = (int)round_up(in, 128);
  d->group = d->Kp;  // one scale per row: a single group spanning the padded row
  d->Gp = 1;
  return Q4_OK;
}

size_t q8_packed_bytes(int64_t out, int64_t in) {
  Dims d;
  if (out <= 0 || in <= 0 || out >= kMaxDim || in >= kMaxDim || in % 8 != 0) return 0;
  check_w8_dims(out, in, &d);
  return (size_t)d.Np * (size_t)d.Kp;
}

size_t q8_scales_count(int64_t out) {
  if (out <= 0 || out >= kMaxDim) return 0;
  return (size_t)round_up(out, 16);
}

q4_status q8_quantize_pack(const void* W, int64_t out, int64_t in, void* packed, void* scales, void* stream) {
  if (!W || !packed || !scales) return fail(Q4_ERR_NULL, "W, packed, scales must be non-NULL");
  Dims d;
  q4_status st = check_w8_dims(out, in, &d);
  if (st != Q4_OK) return st;
  if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(scales, 2))
    return fail(Q4_ERR_ALIGN, "W and packed need 16-byte, scales 2-byte alignment");
  q4::W8Args a{W, d.N, d.K, d.Np, d.Kp, packed, scales, nullptr, nullptr};
  return hip_status(q4::launch_quantize_w8(a, static_cast<hipStream_t>(stream)), "q8 quantize launch");
}

size_t q8_workspace_bytes(int64_t B, int64_t out, int64_t in) {
  Dims d;
  if (B <= 0 || B >= kMaxDim || out <= 0 || in <= 0 || out >= kMaxDim || in >= kMaxDim || in % 8 != 0) return 0;
  check_w8_dims(out, in, &d);
  q4::GemmArgs a{};
  a.B = (int)B;
  a.N = d.N;
  a.q8 = true;
  pick_shape(a.B, d, &a);
  return splits_workspace(a);
}

static q4_status q8_gemm_common(const void* x, int64_t B, const void* packed, const void* scales, int64_t out,
                                int64_t in, void* y, int rows_per_wave, int waves_per_group, int k_splits,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || B >= kMaxDim) return fail(Q4_ERR_SHAPE, "B=%lld out of range", (long long)B);
  Dims d;
  q4_status st = check_w8_dims(out, in, &d);
  if (st != Q4_OK) return st;
  if (B == 0) return ok();
  if (!x || !packed || !scales || !y) return fail(Q4_ERR_NULL, "x, packed, scales, y must be non-NULL");
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 2) || !aligned(y, 2))
    return fail(Q4_ERR_ALIGN, "x and packed need 16-byte, scales and y 2-byte alignment");
  if ((int64_t)B * in >= (int64_t(1) << 40) || (int64_t)B * out >= (int64_t(1) << 40))
    return fail(Q4_ERR_SHAPE, "B*in or B*out too large");
  q4::GemmArgs a{};
  a.x = x;
  a.B = (int)B;
  a.y = y;
  a.packed = packed;
  a.scales = scales;
  a.q8 = true;
  a.N = d.N;
  a.K = d.K;
  a.group = d.group;
  a.Np = d.Np;
  a.Kp = d.Kp;
  a.Gp = d.Gp;
  pick_shape((int)B, d, &a);
  if (rows_per_wave > 0 || waves_per_group > 0 || k_splits > 0) {
    if (B > 16) return fail(Q4_ERR_UNSUPPORTED, "q8_gemm_config sets GEMV shapes (B <= 16); B=%lld runs the skinny GEMM",
                            (long long)B);
    const int B16 = (int)B;
    if (rows_per_wave != 1 && rows_per_wave != 2 && rows_per_wave != 4)
      return fail(Q4_ERR_UNSUPPORTED, "rows_per_wave must be 1, 2 or 4");
    if (waves_per_group < 1 || waves_per_group > 16)
      return fail(Q4_ERR_UNSUPPORTED, "waves_per_group must be in [1, 16]");
    a.lds_limit = lds_per_block();
    if (!gemv_shape_ok(B16, d.Kp / 128, k_splits, waves_per_group, rows_per_wave, d.group, false, a.lds_limit, true))
      return fail(Q4_ERR_UNSUPPORTED, "k_splits=%d, waves_per_group=%d: more splits than 128-channel blocks, "
                  "or the activation slice of %d rows does not fit LDS or the copy",
                  (int)k_splits, (int)waves_per_group, B16);
    a.rows_per_wave = rows_per_wave;
    a.waves_per_group = waves_per_group;
    a.k_splits = k_splits;
  }
  const size_t need = splits_workspace(a);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(Q4_ERR_WORKSPACE, "this shape needs %zu bytes of workspace (q8_workspace_bytes), got %zu", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(Q4_ERR_ALIGN, "workspace needs 16-byte alignment");
  }
  a.workspace = workspace;
  return hip_status(q4::launch_gemm(a, static_cast<hipStream_t>(stream)), "q8 gemm launch");
}

q4_status q8_gemm(const void* x, int64_t B, const void* packed, const void* scales, int64_t out, int64_t in,
                  void* y, void* workspace, size_t workspace_bytes, void* stream) {
  return q8_gemm_common(x, B, packed, scales, out, in, y, 0, 0, 0, workspace, workspace_bytes, stream);
}

q4_status q8_gemm_config(const void* x, int64_t B, const void* packed, const void* scales, int64_t out,
                         int64_t in, void* y, int32_t rows_per_wave, int32_t waves_per_group, int32_t k_splits,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (rows_per_wave <= 0 || waves_per_group <= 0 || k_splits <= 0)
    return fail(Q4_ERR_UNSUPPORTED, "rows_per_wave, waves_per_group and k_splits must be positive");
  return q8_gemm_common(x, B, packed, scales, out, in, y, rows_per_wave, waves_per_group, k_splits, workspace,
                        workspace_bytes, stream);
}

q4_status q8_to_canonical(const void* packed, const void* scales, int64_t out, int64_t in, void* canon_codes,
                          void* canon_scales, void* stream) {
  if (!packed || !scales || !canon_codes || !canon_scales) return fail(Q4_ERR_NULL, "a required pointer is NULL");
  Dims d;
  q4_status st = check_w8_dims(out, in, &d);
  if (st != Q4_OK) return st;
  if (!aligned(scales, 2) || !aligned(canon_scales, 2)) return fail(Q4_ERR_ALIGN, "scales need 2-byte alignment");
  q4::W8Args a{nullptr, d.N, d.K, d.Np, d.Kp, const_cast<void*>(packed), const_cast<void*>(scales), canon_codes,
               canon_scales};
  return hip_status(q4::launch_w8_to_canonical(a, static_cast<hipStream_t>(stream)), "q8 to_canonical launch");
}

q4_status q8_from_canonical(const void* canon_codes, const void* canon_scales, int64_t out, int64_t in,
                            void* packed, void* scales, void* stream) {
  if (!packed || !scales || !canon_codes || !canon_scales) return fail(Q4_ERR_NULL, "a required pointer is NULL");
  Dims d;
  q4_status st = check_w8_dims(out, in, &d);
  if (st != Q4_OK) return st;
  if (!aligned(packed, 4) || !aligned(scales, 2) || !aligned(canon_scales, 2))
    return fail(Q4_ERR_ALIGN, "packed needs 4-byte, scales 2-byte alignment");
  q4::W8Args a{nullptr, d.N, d.K, d.Np, d.Kp, packed, scales, const_cast<void*>(canon_codes),
               const_cast<void*>(canon_scales)};
  return hip_status(q4::launch_w8_from_canonical(a, static_cast<hipStream_t>(stream)), "q8 from_canonical launch");
}

// ---- INT4 KV cache ---------------------------------------------------------------

static q4_status check_kv(int64_t bh, int64_t n, int64_t head_dim, int32_t group, int64_t max_seq, int64_t pos) {
  constexpr int64_t kMax31 = int64_t(1) << 31;
  if (group != 32 && group != 64 && group != 128)
    return fail(Q4_ERR_GROUP, "KV group %d unsupported (32, 64 or 128)", (int)group);
  if (head_dim <= 0 || head_dim % group != 0 || head_dim >= kMax31)
    return fail(Q4_ERR_GROUP, "head_dim=%lld must be a positive multiple of group %d", (long long)head_dim, (int)group);
  if (bh < 0 || n < 0 || pos < 0 || max_seq <= 0 || bh >= kMax31 || n >= kMax31 || max_seq >= kMax31)
    return fail(Q4_ERR_SHAPE, "bh=%lld, n=%lld, pos=%lld, max_seq=%lld out of range", (long long)bh, (long long)n,
                (long long)pos, (long long)max_seq);
  if (pos + n > max_seq)
    return fail(Q4_ERR_SHAPE, "pos + n = %lld exceeds max_seq = %lld", (long long)(pos + n), (long long)max_seq);
  int64_t cells = 0, elems = 0;  // each factor is below 2^31, but their product may not fit 64 bits
  if (__builtin_mul_overflow(bh, max_seq, &cells) || __builtin_mul_overflow(cells, head_dim, &elems) ||
      elems >= (int64_t(1) << 46))
    return fail(Q4_ERR_SHAPE, "cache too large");
  return Q4_OK;
}

q4_status q4_kv_quantize_pack(const void* src, int64_t bh, int64_t n, int64_t head_dim, int32_t group, void* codes,
                              void* scales, int64_t max_seq, int64_t pos, void* stream) {
  q4_status st = check_kv(bh, n, head_dim, group, max_seq, pos);
  if (st != Q4_OK) return st;
  if (bh == 0 || n == 0) return ok();
  if (!src || !codes || !scales) return fail(Q4_ERR_NULL, "src, codes, scales must be non-NULL");
  if (!aligned(src, 16) || !aligned(codes, 4) || !aligned(scales, 2))
    return fail(Q4_ERR_ALIGN, "src needs 16-byte, codes 4-byte, scales 2-byte alignment");
  q4::KvArgs a{src, bh, n, (int)head_dim, group, max_seq, pos, codes, scales, nullptr};
  return hip_status(q4::launch_kv_quantize(a, static_cast<hipStream_t>(stream)), "kv quantize launch");
}

q4_status q4_kv_dequant(const void* codes, const void* scales, int64_t bh, int64_t n, int64_t head_dim, int32_t group,
                        int64_t max_seq, int64_t pos, void* dst, void* stream) {
  q4_status st = check_kv(bh, n, head_dim, group, max_seq, pos);
  if (st != Q4_OK) return st;
  if (bh == 0 || n == 0) return ok();
  if (!codes || !scales || !dst) return fail(Q4_ERR_NULL, "codes, scales, dst must be non-NULL");
  if (!aligned(codes, 4) || !aligned(scales, 2) || !aligned(dst, 16))
    return fail(Q4_ERR_ALIGN, "codes need 4-byte, scales 2-byte, dst 16-byte alignment");
  q4::KvArgs a{nullptr, bh, n, (int)head_dim, group, max_seq, pos, const_cast<void*>(codes), const_cast<void*>(scales),
               dst};
  return hip_status(q4::launch_kv_dequant(a, static_cast<hipStream_t>(stream)), "kv dequant launch");
}

// ---- read probe ----------------------------------------------------------------

q4_status q4_read_probe(const void* buf, size_t bytes, void* sink, void* stream) {
  if (!buf || !sink) return fail(Q4_ERR_NULL, "buf and sink must be non-NULL");
  if (bytes == 0 || bytes % 8192 != 0) return fail(Q4_ERR_SHAPE, "bytes=%zu must be a positive multiple of 8192", bytes);
  if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(Q4_ERR_ALIGN, "buf needs 16-byte, sink 4-byte alignment");
  return hip_status(q4::launch_read_probe(buf, (int64_t)(bytes / 8192), sink, q4::device_cu_count_cached(),
                                          static_cast<hipStream_t>(stream)), "read probe launch");
}

q4_status q4_rtn_check(uint64_t* counts, void* stream) {
  if (!counts) return fail(Q4_ERR_NULL, "counts must be non-NULL");
  if (!aligned(counts, 8)) return fail(Q4_ERR_ALIGN, "counts needs 8-byte alignment");
  return hip_status(q4::launch_rtn_check(reinterpret_cast<unsigned long long*>(counts),
                                         static_cast<hipStream_t>(stream)),
                    "rtn check launch");
}

}  // extern "C"
