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
  int waves_per_group;  // wavefronts per workgroup: 1..16 (GEMV), 4 or 8 (skinny GEMM)
  int col_tiles;        // 16-column batch tiles per workgroup: 1 (GEMV), 2, 3, 4, 6 or 8 (skinny GEMM)
  int k_splits;         // workgroups splitting the channels; > 1 needs workspace
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
// Read `pieces` x 8 KiB from buf with one workgroup of 4 wavefronts per CU.
hipError_t launch_read_probe(const void* buf, int64_t pieces, void* sink, int cus, hipStream_t stream);
hipError_t launch_rtn_check(unsigned long long* counts, hipStream_t stream);
hipError_t launch_kv_dequant(const KvArgs& a, hipStream_t stream);
hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);
hipError_t launch_quantize_w8(const W8Args& a, hipStream_t stream);
hipError_t launch_w8_to_canonical(const W8Args& a, hipStream_t stream);
hipError_t launch_w8_from_canonical(const W8Args& a, hipStream_t stream);
hipError_t launch_to_canonical(const LayoutArgs& a, hipStream_t stream);
hipError_t launch_from_canonical(const LayoutArgs& a, hipStream_t stream);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);
// Device address (on the current device) of the library-owned scratch array that
// q4_gemm_noalloc uses in place of a workspace; looked up once per device.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void** out);
// Blocks of 128 channels in one unit of the streaming GEMV.
constexpr int kStreamUnitBlocks = 8;

// Activation rows in LDS (GEMV slices and units, skinny-GEMM tiles) are padded by 16
// halfs (32 bytes): the 16 lanes of a B-operand read (16 rows, 16 bytes each) then
// hit distinct banks; a 16-byte pad leaves 2-way conflicts, which halved the LDS
// read rate in a plain read loop.
constexpr int kGemmRowPad = 16;

// Skinny GEMM: the channel range is walked in chunks of 8 / col_tiles blocks, at least
// 2 (the ring of codes in flight is one chunk long). LDS: two activation tiles of
// col_tiles * 16 batch rows by one chunk, padded rows -- ~51 KiB for 3 column tiles,
// ~66-68 KiB for 2 or 4 (room for two workgroups per CU), ~102 KiB for 6 and ~136 KiB
// for 8. Chunks of 16 / col_tiles blocks (~132 KiB at every width) measured 5-12%
// slower at B = 24-32.
constexpr int mfma_chunk_blocks(int col_tiles) { return col_tiles >= 4 ? 2 : 8 / col_tiles; }
constexpr size_t mfma_lds_bytes(int col_tiles) {
  return (size_t)2 * col_tiles * 16 * (mfma_chunk_blocks(col_tiles) * 128 + kGemmRowPad) * 2;
}

// Whether the streaming GEMV runs in its burst form (gemv_stream_burst_kernel): symmetric
// INT4 codes, groups of 128, and at most one workgroup per CU (row blocks of two tiles
// <= CUs), the grid its register budget allows.
inline bool gemv_stream_burst_ok(int Np, int group, bool asym, bool q8, int cus) {
  return !asym && !q8 && group == 128 && (Np / 16 + 1) / 2 <= cus;
}

// Whether the GEMV for this launch shape streams x per unit (one split, two row tiles
// per wavefront, a multiple of 1024 channels; B <= 3, or B = 4 in the burst form, where
// streaming measured faster than the staged kernel with two row tiles) instead of
// staging the whole slice. The host's own pick streams at B <= 3 only; at B = 4 its
// launch model decides the shape (streamed where that is two row tiles, no split).
inline bool gemv_streams_x(int B, int Kp, int rows_per_wave, int k_splits, bool burst_form) {
  const int S = Kp / 128;
  return B >= 1 && (B <= 3 || (B == 4 && burst_form)) && k_splits == 1 && rows_per_wave == 2 &&
         S % kStreamUnitBlocks == 0;
}
// Facts of the current device, each looked up once per device and kept in one
// lock-guarded cache (q4_api.cpp): its compute units, the workgroups of `block`
// threads with `lds` bytes of dynamic LDS of kernel fn one CU holds at once, and
// the same times the CU count for kernels without dynamic LDS.
int device_cu_count_cached();
int resident_per_cu(const void* fn, int block, size_t lds);
int resident_grid(const void* fn, int block);

// Workgroups of the skinny GEMM for symmetric INT4 codes with one scale per block
// (8 wavefronts, rows_per_wave 1 or 2, col_tiles 2, 3, 4, 6 or 8) that one CU of the
// current device holds at once (q4_gemm.hip); 1 where the device cannot be queried.
int mfma_resident_per_cu(int rows_per_wave, int col_tiles);

}  // namespace q4
