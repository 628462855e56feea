// Host-side checks of libq4's C ABI front end (q4_api.cpp), built with gcc under
// AddressSanitizer and UndefinedBehaviorSanitizer, without a GPU or a HIP runtime.
//
// The kernel launchers (q4::launch_*) and the few HIP runtime calls q4_api.cpp makes
// are replaced by the stubs below: a launcher records that it was reached and
// returns g_launch_result, which a test sets to a HIP error to inject a launch
// failure. The checks then cover, for every entry point:
//   * invalid arguments return their status and reach no launcher;
//   * a valid call reaches exactly one launcher (two for an act-order product) and,
//     when the launcher fails, returns Q4_ERR_HIP with the HIP error in q4_last_error;
//   * shape products that overflow 64 bits are rejected (KV cache sizes);
//   * the act-order permutation, computed on the host, is right.
// Exit status 0 means every check passed; the sanitizers abort on the first error.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "q4.h"
#include "q4_kv.h"
#include "q8.h"
#include "../../w4a16_decode_amd/csrc/q4_internal.h"

// ---- stubs ---------------------------------------------------------------------
static hipError_t g_launch_result = hipSuccess;
static int g_launches = 0;

namespace q4 {
#define Q4_STUB(name, argtype) \
  hipError_t name(const argtype&, hipStream_t) { ++g_launches; return g_launch_result; }
Q4_STUB(launch_kv_quantize, KvArgs)
Q4_STUB(launch_kv_dequant, KvArgs)
Q4_STUB(launch_quantize, QuantArgs)
Q4_STUB(launch_quantize_w8, W8Args)
Q4_STUB(launch_w8_to_canonical, W8Args)
Q4_STUB(launch_w8_from_canonical, W8Args)
Q4_STUB(launch_to_canonical, LayoutArgs)
Q4_STUB(launch_from_canonical, LayoutArgs)
Q4_STUB(launch_gemm, GemmArgs)
#undef Q4_STUB
hipError_t launch_read_probe(const void*, int64_t, void*, int, hipStream_t) {
  ++g_launches;
  return g_launch_result;
}
hipError_t launch_rtn_check(unsigned long long*, hipStream_t) {
  ++g_launches;
  return g_launch_result;
}
// the MI355X residency of the skinny GEMM's symmetric kernels: one row tile per
// wavefront with at most 4 column tiles (90-104 VGPRs, <= 68 KiB of LDS) fits two
// 8-wavefront workgroups per CU, every other shape one
int mfma_resident_per_cu(int rows_per_wave, int col_tiles) { return rows_per_wave == 1 && col_tiles <= 4 ? 2 : 1; }
int g_scratch_lookups = 0;
hipError_t noalloc_scratch(void** out) {
  ++g_scratch_lookups;
  *out = reinterpret_cast<void*>(0x7000000);
  return hipSuccess;
}
}  // namespace q4

extern "C" {
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int) {
  *v = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 160 * 1024;
  return hipSuccess;
}
hipError_t hipOccupancyMaxActiveBlocksPerMultiprocessor(int* n, const void*, int, size_t) {
  *n = 1;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "hipSuccess" : "injected launch failure"; }
}

// ---- checks ----------------------------------------------------------------------
static int g_failed = 0;

#define EXPECT(cond, what)                                                        \
  do {                                                                            \
    if (!(cond)) {                                                                \
      fprintf(stderr, "FAILED %s:%d %s (%s)\n", __FILE__, __LINE__, what, q4_last_error()); \
      ++g_failed;                                                                 \
    }                                                                             \
  } while (0)

// `call` must return `want` and reach `launches` launchers.
#define CHECK_CALL(call, want, launches)                                                       \
  do {                                                                                         \
    g_launches = 0;                                                                            \
    const int st_ = (int)(call);                                                               \
    if (st_ != (int)(want) || g_launches != (launches)) {                                      \
      fprintf(stderr, "FAILED %s:%d %s -> %d (want %d), %d launches (want %d): %s\n", __FILE__, \
              __LINE__, #call, st_, (int)(want), g_launches, (int)(launches), q4_last_error()); \
      ++g_failed;                                                                              \
    }                                                                                          \
  } while (0)

static char* const P = reinterpret_cast<char*>(0x100000);  // aligned, never dereferenced

// Each valid call: once succeeding (one launch), once with the launch failing.
#define VALID(call, launches)                                                            \
  do {                                                                                   \
    g_launch_result = hipSuccess;                                                        \
    CHECK_CALL(call, Q4_OK, launches);                                                   \
    g_launch_result = hipErrorLaunchFailure;                                             \
    CHECK_CALL(call, Q4_ERR_HIP, launches);                                              \
    EXPECT(strstr(q4_last_error(), "injected launch failure") != nullptr, "HIP error text"); \
    g_launch_result = hipSuccess;                                                        \
  } while (0)

// `host_sanitize shapes`: reads "B out in group" lines from stdin and prints the
// launch shape q4_gemm_shape reports for each ("R W KS CT", or "error <status>"),
// with the device limits the stubs above stand in for (256 CUs, 160 KiB of LDS).
static int print_shapes() {
  long long B, N, K;
  int g;
  while (scanf("%lld %lld %lld %d", &B, &N, &K, &g) == 4) {
    int32_t sh[4] = {0, 0, 0, 0};
    const q4_status st = q4_gemm_shape(B, N, K, g, sh);
    if (st != Q4_OK) printf("error %d\n", (int)st);
    else printf("%d %d %d %d\n", (int)sh[0], (int)sh[1], (int)sh[2], (int)sh[3]);
  }
  return 0;
}

int main(int argc, char** argv) {
  if (argc > 1 && strcmp(argv[1], "shapes") == 0) return print_shapes();
  // quantize
  VALID(q4_quantize_pack(P, 4096, 4096, 128, P, P, nullptr), 1);
  VALID(q4_quantize_pack_asym(P, 300, 1024, 64, P, P, P, nullptr), 1);
  VALID(q4_quantize_pack_clip(P, 300, 1024, 32, 80, P, P, nullptr), 1);
  VALID(q4_quantize_pack_perm(P, 300, 1024, 128, reinterpret_cast<const int32_t*>(P), P, P, nullptr), 1);
  CHECK_CALL(q4_quantize_pack(nullptr, 16, 128, 128, P, P, nullptr), Q4_ERR_NULL, 0);
  CHECK_CALL(q4_quantize_pack(P, 16, 96, 64, P, P, nullptr), Q4_ERR_GROUP, 0);
  CHECK_CALL(q4_quantize_pack(P, 16, 128, 48, P, P, nullptr), Q4_ERR_GROUP, 0);
  CHECK_CALL(q4_quantize_pack(P + 2, 16, 128, 128, P, P, nullptr), Q4_ERR_ALIGN, 0);
  CHECK_CALL(q4_quantize_pack(P, int64_t(1) << 30, 128, 128, P, P, nullptr), Q4_ERR_SHAPE, 0);
  CHECK_CALL(q4_quantize_pack(P, INT64_MAX, INT64_MAX, 128, P, P, nullptr), Q4_ERR_SHAPE, 0);
  CHECK_CALL(q4_quantize_pack(P, -1, 128, 128, P, P, nullptr), Q4_ERR_SHAPE, 0);
  CHECK_CALL(q4_quantize_pack_clip(P, 16, 128, 128, 0, P, P, nullptr), Q4_ERR_UNSUPPORTED, 0);
  CHECK_CALL(q4_quantize_pack_clip(P, 16, 256, 256, 80, P, P, nullptr), Q4_ERR_UNSUPPORTED, 0);
  CHECK_CALL(q4_quantize_pack_asym(P, 16, 128, 128, P, P, nullptr, nullptr), Q4_ERR_NULL, 0);

  // products: every path of the shape selection, with enough workspace
  static const int64_t shapes[][3] = {{1, 57344, 8192}, {1, 8192, 28672}, {4, 8192, 28672}, {8, 10240, 8192},
                                      {16, 4096, 4096}, {32, 28672, 8192}, {256, 28672, 8192}, {3, 17, 96},
                                      {48, 4096, 14336}, {192, 8192, 8192}, {256, 6144, 4096}};
  for (const auto& sh : shapes) {
    const int64_t B = sh[0], N = sh[1], K = sh[2];
    const int32_t g = K % 128 == 0 ? 128 : 32;
    const size_t ws = q4_workspace_bytes(B, N, K, g);
    VALID(q4_gemm(P, B, P, P, N, K, g, P, P, ws, nullptr), 1);
    VALID(q4_gemm_asym(P, B, P, P, P, N, K, g, P, P, ws, nullptr), 1);
    const size_t wsp = q4_workspace_bytes_perm(B, N, K, g);
    EXPECT(wsp >= ws + (size_t)(B * K * 2), "act-order workspace holds the gathered x");
    VALID(q4_gemm_perm(P, B, P, P, reinterpret_cast<const int32_t*>(P), N, K, g, P, P, wsp, nullptr), 1);
    if (ws > 0) {
      // ws covers both products; it is exact for at least one of them (symmetric codes
      // stream x at B = 4 without a split where asymmetric ones split)
      const int before = g_launches;
      const bool sym_short = q4_gemm(P, B, P, P, N, K, g, P, P, ws - 1, nullptr) == Q4_ERR_WORKSPACE;
      const bool asym_short = q4_gemm_asym(P, B, P, P, P, N, K, g, P, P, ws - 1, nullptr) == Q4_ERR_WORKSPACE;
      EXPECT(sym_short || asym_short, "q4_workspace_bytes is the larger of the two products' needs");
      EXPECT(g_launches - before == (sym_short ? 0 : 1) + (asym_short ? 0 : 1), "a short workspace launches nothing");
    }
    const size_t w8 = q8_workspace_bytes(B, N, K);
    VALID(q8_gemm(P, B, P, P, N, K, P, P, w8, nullptr), 1);
  }
  // launch-shape query: host only, argument errors as q4_gemm's
  {
    int32_t sh[4] = {0, 0, 0, 0};
    CHECK_CALL(q4_gemm_shape(1, 57344, 8192, 128, sh), Q4_OK, 0);
    EXPECT(sh[3] == 1 && sh[0] >= 1 && sh[1] >= 1 && sh[2] >= 1, "B <= 16 runs the GEMV (one column tile)");
    CHECK_CALL(q4_gemm_shape(96, 28672, 8192, 128, sh), Q4_OK, 0);
    EXPECT(sh[1] == 8 && (sh[3] == 3 || sh[3] == 6), "B = 96: six 16-row tiles, in groups of 3 or 6");
    CHECK_CALL(q4_gemm_shape(96, 28672, 8192, 128, nullptr), Q4_ERR_NULL, 0);
    CHECK_CALL(q4_gemm_shape(0, 28672, 8192, 128, sh), Q4_ERR_SHAPE, 0);
    CHECK_CALL(q4_gemm_shape(int64_t(1) << 30, 28672, 8192, 128, sh), Q4_ERR_SHAPE, 0);
    CHECK_CALL(q4_gemm_shape(4, 28672, 8192, 48, sh), Q4_ERR_GROUP, 0);
    CHECK_CALL(q4_gemm_shape(4, 0, 8192, 128, sh), Q4_ERR_SHAPE, 0);
  }
  // the no-allocation product: the library scratch stands in for the workspace
  q4::g_scratch_lookups = 0;
  VALID(q4_gemm_noalloc(P, 1, P, P, 4096, 4096, 128, P, nullptr), 1);
  EXPECT(q4::g_scratch_lookups == 0, "no scratch lookup where no split needs it");
  VALID(q4_gemm_noalloc(P, 8, P, P, 8192, 28672, 128, P, nullptr), 1);
  EXPECT(q4::g_scratch_lookups > 0, "scratch looked up for a split product");
  EXPECT(q4_workspace_bytes(16, 65536, 262144, 128) > Q4_NOALLOC_SCRATCH_BYTES, "a split beyond the scratch");
  CHECK_CALL(q4_gemm_noalloc(P, 16, P, P, 65536, 262144, 128, P, nullptr), Q4_ERR_WORKSPACE, 0);
  CHECK_CALL(q4_gemm_noalloc(nullptr, 4, P, P, 8192, 28672, 128, P, nullptr), Q4_ERR_NULL, 0);
  CHECK_CALL(q4_gemm(P, 0, nullptr, nullptr, 16, 128, 128, nullptr, nullptr, 0, nullptr), Q4_OK, 0);
  CHECK_CALL(q4_gemm(P, -1, P, P, 16, 128, 128, P, nullptr, 0, nullptr), Q4_ERR_SHAPE, 0);
  CHECK_CALL(q4_gemm(P, 1, P, P, 16, 128, 128, nullptr, nullptr, 0, nullptr), Q4_ERR_NULL, 0);
  CHECK_CALL(q4_gemm(P + 8, 1, P, P, 16, 128, 128, P, nullptr, 0, nullptr), Q4_ERR_ALIGN, 0);
  CHECK_CALL(q4_gemm(P, 1, P, P, 16, 128, 128, P + 1, nullptr, 0, nullptr), Q4_ERR_ALIGN, 0);
  CHECK_CALL(q4_gemm(P, int64_t(1) << 29, P, P, 1 << 20, 4096, 128, P, nullptr, 0, nullptr), Q4_ERR_SHAPE, 0);
  CHECK_CALL(q4_gemm_config(P, 1, P, P, nullptr, 0, 4096, 4096, 128, P, 3, 8, 1, 1, nullptr, 0, nullptr),
             Q4_ERR_UNSUPPORTED, 0);
  CHECK_CALL(q4_gemm_config(P, 1, P, P, nullptr, 0, 4096, 4096, 128, P, 1, 8, 0, 1, nullptr, 0, nullptr),
             Q4_ERR_UNSUPPORTED, 0);
  CHECK_CALL(q4_gemm_config(P, 64, P, P, nullptr, 0, 4096, 4096, 128, P, 4, 8, 1, 4, nullptr, 0, nullptr),
             Q4_ERR_UNSUPPORTED, 0);
  VALID(q4_gemm_config(P, 1, P, P, nullptr, 0, 4096, 4096, 128, P, 1, 8, 1, 1, nullptr, 0, nullptr), 1);
  VALID(q4_gemm_config(P, 64, P, P, P, 1, 4096, 4096, 128, P, 2, 8, 1, 4, nullptr, 0, nullptr), 1);

  // layout converters, INT8, KV, read probe
  VALID(q4_to_canonical(P, P, nullptr, 0, 300, 1024, 128, P, P, nullptr, nullptr), 1);
  VALID(q4_from_canonical(P, P, P, 1, 300, 1024, 128, P, P, P, nullptr), 1);
  CHECK_CALL(q4_to_canonical(P, P, nullptr, 1, 300, 1024, 128, P, P, P, nullptr), Q4_ERR_NULL, 0);
  VALID(q8_quantize_pack(P, 300, 1024, P, P, nullptr), 1);
  VALID(q8_to_canonical(P, P, 300, 1024, P, P, nullptr), 1);
  VALID(q8_from_canonical(P, P, 300, 1024, P, P, nullptr), 1);
  CHECK_CALL(q8_quantize_pack(P, 300, 1020, P, P, nullptr), Q4_ERR_SHAPE, 0);
  VALID(q4_kv_quantize_pack(P, 64, 128, 128, 128, P, P, 4096, 100, nullptr), 1);
  VALID(q4_kv_dequant(P, P, 64, 128, 128, 64, 4096, 100, P, nullptr), 1);
  CHECK_CALL(q4_kv_quantize_pack(P, 64, 128, 128, 128, P, P, 4096, 4000, nullptr), Q4_ERR_SHAPE, 0);
  // bh * max_seq * head_dim overflows 64 bits (2^64 and 2^63): rejected, not wrapped
  CHECK_CALL(q4_kv_quantize_pack(P, int64_t(1) << 20, 1, int64_t(1) << 24, 128, P, P, int64_t(1) << 20, 0, nullptr),
             Q4_ERR_SHAPE, 0);
  CHECK_CALL(q4_kv_quantize_pack(P, int64_t(1) << 20, 1, int64_t(1) << 23, 128, P, P, int64_t(1) << 20, 0, nullptr),
             Q4_ERR_SHAPE, 0);
  CHECK_CALL(q4_kv_dequant(P, P, int64_t(1) << 20, 1, int64_t(1) << 24, 128, int64_t(1) << 20, 0, P, nullptr),
             Q4_ERR_SHAPE, 0);
  VALID(q4_read_probe(P, 8192 * 4, P, nullptr), 1);
  CHECK_CALL(q4_read_probe(P, 8191, P, nullptr), Q4_ERR_SHAPE, 0);
  VALID(q4_rtn_check(reinterpret_cast<uint64_t*>(P), nullptr), 1);
  CHECK_CALL(q4_rtn_check(nullptr, nullptr), Q4_ERR_NULL, 0);
  CHECK_CALL(q4_rtn_check(reinterpret_cast<uint64_t*>(P + 4), nullptr), Q4_ERR_ALIGN, 0);

  // act-order permutation (host code): channel k in group (5k + 3) % 16, 4096 channels
  {
    static int32_t g_idx[4096], perm[4096];
    for (int k = 0; k < 4096; ++k) g_idx[k] = (5 * k + 3) % 16;
    g_launches = 0;
    EXPECT(q4_actorder_perm(g_idx, 4096, 256, perm) == Q4_OK, "actorder_perm");
    EXPECT(g_launches == 0, "actorder_perm launches nothing");
    int prev = -1;
    for (int i = 0; i < 4096; ++i) {
      EXPECT(g_idx[perm[i]] == i / 256, "perm groups");
      if (i % 256 != 0) EXPECT(perm[i] > prev, "ascending inside a group");
      prev = perm[i];
    }
    g_idx[7] = 16;
    EXPECT(q4_actorder_perm(g_idx, 4096, 256, perm) == Q4_ERR_SHAPE, "g_idx out of range");
    g_idx[7] = g_idx[8];
    EXPECT(q4_actorder_perm(g_idx, 4096, 256, perm) == Q4_ERR_SHAPE, "unequal groups");
  }

  if (g_failed) {
    fprintf(stderr, "%d check(s) failed\n", g_failed);
    return 1;
  }
  printf("host checks ok\n");
  return 0;
}
