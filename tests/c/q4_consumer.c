/*
 * A plain C99 consumer of libq4's C ABI (include/q4.h): no C++, no torch.
 *
 *   q4_consumer host            host-side calls only (sizes, status strings, act-order
 *                               permutation, argument checks); exits 0 when they agree
 *                               with the header's definitions
 *   q4_consumer gpu IN OUT      reads W, x from IN, runs q4_quantize_pack, q4_to_canonical
 *                               and q4_gemm on the GPU with the caller's own hipMalloc'd
 *                               buffers and stream, writes codes, scales and y to OUT
 *
 * IN:  int32 N, K, B, group; float16 W[N][K]; float16 x[B][K]
 * OUT: uint8 codes[N][K/2]; float16 scales[N][K/group]; float16 y[B][N]
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "q4.h"

static int fail(const char* what) {
  fprintf(stderr, "q4_consumer: %s (%s)\n", what, q4_last_error());
  return 1;
}

static int host_checks(void) {
  int32_t g_idx[256], perm[256];
  int k, j;
  if (q4_packed_bytes(4096, 4096) != (size_t)4096 * 4096 / 2) return fail("q4_packed_bytes");
  if (q4_packed_bytes(17, 96) != (size_t)32 * 128 / 2) return fail("q4_packed_bytes padding");
  if (q4_groups_count(4096, 4096, 128) != (size_t)4096 * 32) return fail("q4_groups_count");
  if (!q4_group_supported(128) || q4_group_supported(96)) return fail("q4_group_supported");
  if (strcmp(q4_status_str(Q4_OK), "ok") != 0) return fail("q4_status_str");
  /* channel k belongs to group (k * 7) % 8: every group holds 32 of the 256 channels */
  for (k = 0; k < 256; ++k) g_idx[k] = (k * 7) % 8;
  if (q4_actorder_perm(g_idx, 256, 32, perm) != Q4_OK) return fail("q4_actorder_perm");
  for (j = 0; j < 256; ++j) {
    if (g_idx[perm[j]] != j / 32) return fail("perm groups");
    if (j % 32 && perm[j] <= perm[j - 1]) return fail("perm order");
  }
  /* rejected on the host before any HIP call */
  if (q4_quantize_pack(NULL, 16, 128, 128, NULL, NULL, NULL) != Q4_ERR_NULL) return fail("null check");
  if (q4_gemm((void*)0x100000, 1, (void*)0x100000, (void*)0x100000, 16, 100, 32, (void*)0x100000, NULL, 0, NULL) !=
      Q4_ERR_GROUP)
    return fail("group check");
  printf("host ok: %s\n", q4_version());
  return 0;
}

#define HIP_OK(call) do { if ((call) != hipSuccess) { fprintf(stderr, "q4_consumer: %s failed\n", #call); return 1; } } while (0)

static int gpu_run(const char* in_path, const char* out_path) {
  int32_t hdr[4];
  FILE* f = fopen(in_path, "rb");
  if (!f || fread(hdr, sizeof(int32_t), 4, f) != 4) return fail("reading the input header");
  const int64_t N = hdr[0], K = hdr[1], B = hdr[2];
  const int32_t group = hdr[3];
  const size_t wn = (size_t)N * K, xn = (size_t)B * K;
  uint16_t* W = malloc(wn * 2);
  uint16_t* x = malloc(xn * 2);
  if (!W || !x || fread(W, 2, wn, f) != wn || fread(x, 2, xn, f) != xn) return fail("reading W and x");
  fclose(f);

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  const size_t pb = q4_packed_bytes(N, K), ng = q4_groups_count(N, K, group);
  const size_t ws_bytes = q4_workspace_bytes(B, N, K, group);
  void *dW, *dx, *dp, *ds, *dy, *dws = NULL, *dcodes, *dscales;
  HIP_OK(hipMalloc(&dW, wn * 2));
  HIP_OK(hipMalloc(&dx, xn * 2));
  HIP_OK(hipMalloc(&dp, pb));
  HIP_OK(hipMalloc(&ds, ng * 2));
  HIP_OK(hipMalloc(&dy, (size_t)B * N * 2));
  HIP_OK(hipMalloc(&dcodes, wn / 2));
  HIP_OK(hipMalloc(&dscales, (size_t)N * (K / group) * 2));
  if (ws_bytes) HIP_OK(hipMalloc(&dws, ws_bytes));
  HIP_OK(hipMemcpy(dW, W, wn * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dx, x, xn * 2, hipMemcpyHostToDevice));

  if (q4_quantize_pack(dW, N, K, group, dp, ds, stream) != Q4_OK) return fail("q4_quantize_pack");
  if (q4_to_canonical(dp, ds, NULL, 0, N, K, group, dcodes, dscales, NULL, stream) != Q4_OK)
    return fail("q4_to_canonical");
  if (q4_gemm(dx, B, dp, ds, N, K, group, dy, dws, ws_bytes, stream) != Q4_OK) return fail("q4_gemm");
  HIP_OK(hipStreamSynchronize(stream));

  uint8_t* codes = malloc(wn / 2);
  uint16_t* scales = malloc((size_t)N * (K / group) * 2);
  uint16_t* y = malloc((size_t)B * N * 2);
  if (!codes || !scales || !y) return fail("host buffers");
  HIP_OK(hipMemcpy(codes, dcodes, wn / 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(scales, dscales, (size_t)N * (K / group) * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(y, dy, (size_t)B * N * 2, hipMemcpyDeviceToHost));
  f = fopen(out_path, "wb");
  if (!f) return fail("opening the output");
  fwrite(codes, 1, wn / 2, f);
  fwrite(scales, 2, (size_t)N * (K / group), f);
  fwrite(y, 2, (size_t)B * N, f);
  fclose(f);
  hipFree(dW); hipFree(dx); hipFree(dp); hipFree(ds); hipFree(dy); hipFree(dcodes); hipFree(dscales);
  if (dws) hipFree(dws);
  hipStreamDestroy(stream);
  free(W); free(x); free(codes); free(scales); free(y);
  printf("gpu ok\n");
  return 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "host") == 0) return host_checks();
  if (argc >= 4 && strcmp(argv[1], "gpu") == 0) return gpu_run(argv[2], argv[3]);
  fprintf(stderr, "usage: q4_consumer host | q4_consumer gpu IN OUT\n");
  return 2;
}
