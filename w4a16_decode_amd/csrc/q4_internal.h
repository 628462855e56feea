// Host-side launch interfaces between the C ABI front end (q4_api.cpp) and the
// kernel translation units. Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

struct QuantArgs {
  const void* W;
  int N, K, group;
  int Np, Kp, Gp;
  bool asym;
  void* packed;
  void* scales;
  void* zeros;
  int clip_pmin;  // > 0: symmetric clipping search over alpha = p/100, p = clip_pmin..100
  const int32_t* perm;  // non-NULL: act-order, quantize the columns in the order perm[0..K) (symmetric)
};

struct LayoutArgs {
  int N, K, group;
  int Np, Kp, Gp;
  bool asym;
  // Device layout: read by to_canonical, written by from_canonical.
  void* packed;
  void* scales;
  void* zeros;
  // Canonical layout: written by to_canonical, read by from_canonical.
  void* canon_codes;
  void* canon_scales;
  void* canon_zeros;
};

struct GemmArgs {
  const void* x;
  int B;
  const void* packed;
  const void* scales;
  const void* zeros;
  bool asym;
  bool q8;  // per-channel INT8 codes (B <= 16 GEMV only); group = Kp, Gp = 1
  const int32_t* perm;  // non-NULL: act-order codes; x is read through perm (x[:, perm])
  int N, K, group;
  int Np, Kp, Gp;
  void* y;
  // launch shape
  int rows_per_wave;    // row tiles of 16 per wavefront: 1, 2 or 4
  int waves_per_group;  // wavefronts per workgroup: 1..16 (GEMV), 4 (skinny GEMM)
  int col_tiles;        // 16-column batch tiles per wavefront: 1, 2 or 4
  int k_splits;         // workgroups splitting the channels (B <= 16 path); > 1 needs workspace
  void* workspace;      // float32 [k_splits][B][N] partial sums when k_splits > 1
  int grid_limit;       // B <= 16: cap on the persistent grid (0 = as many as are resident)
  size_t lds_limit;     // B <= 16: LDS a workgroup may use (sizes the per-workgroup result buffer)
};

// Per-channel INT8 (W8A16): codes [Np * Kp] bytes in 2 KiB blocks, scales float16 [Np].
struct W8Args {
  const void* W;  // float16 [N, K] (quantize)
  int N, K, Np, Kp;
  void* packed;
  void* scales;
  void* canon_codes;   // int8 [N, K]
  void* canon_scales;  // float16 [N]
};

// INT4 KV cache: src [bh][n][d] float16 -> codes [bh][max_seq][d/2], scales
// [bh][max_seq][d/group] at positions pos .. pos + n - 1 (dequant: the reverse into dst).
struct KvArgs {
  const void* src;
  int64_t bh, n;
  int d, group;
  int64_t max_seq, pos;
  void* codes;
  void* scales;
  void* dst;
};

hipError_t launch_kv_quantize(const KvArgs& a, hipStream_t stream);
// Read `pieces` x 8 KiB from buf with one workgroup of 8 wavefronts per CU.
hipError_t launch_read_probe(const void* buf, int64_t pieces, void* sink, int cus, hipStream_t stream);
hipError_t launch_kv_dequant(const KvArgs& a, hipStream_t stream);
hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);
hipError_t launch_quantize_w8(const W8Args& a, hipStream_t stream);
hipError_t launch_w8_to_canonical(const W8Args& a, hipStream_t stream);
hipError_t launch_w8_from_canonical(const W8Args& a, hipStream_t stream);
hipError_t launch_to_canonical(const LayoutArgs& a, hipStream_t stream);
hipError_t launch_from_canonical(const LayoutArgs& a, hipStream_t stream);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);
// Whether the GEMV for this shape streams x per unit (B <= 3, one split, two row
// tiles per wavefront, a multiple of 1024 channels) instead of staging the whole slice.
bool gemv_streams_x(int B, int Kp, int rows_per_wave, int k_splits);
// Compute units of the current device, and the workgroups of `block` threads of
// kernel fn it holds at once (both cached, lock-guarded).
int device_cu_count_cached();
int resident_grid(const void* fn, int block);

}  // namespace q4
