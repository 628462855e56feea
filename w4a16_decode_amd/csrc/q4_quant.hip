// Quantize + pack kernels and the canonical <-> device layout converters.
//
// Method: group-wise round-to-nearest INT4 ("LLM 后训练量化深度实战…", www.ybb.press,
// section 二: scale = group amax / 7, codes clamped to [-8, 7]); asymmetric uint4 with
// integer zero point ("Post-training quantization: GPTQ, AWQ and rotation",
// arganzheng.life, section 二.2; "压缩算法", cs-knowledge-wiki, section 7.4.1.1).
//
// One wavefront handles one 16-row x 128-channel tile (one 1 KiB output block):
// lane l = r + 16*c reads, for m = 0..3, the 8 float16 weights of row r at
// channels 32*m + 8*c .. +7 (16 bytes), which are exactly the 32 codes it will
// store as its 16-byte slice of the block. A group of 128 channels of a row is
// spread over the four lanes r, r+16, r+32, r+48; its amax is reduced across
// them with two cross-lane exchanges. Codes round the quotient w / s half to even,
// which for float16 w and s is the decision of the exact rational quotient (and of
// the IEEE float32 one); it is taken from one reciprocal per scale and a multiply
// per weight (q4_rtn.h).
#include <algorithm>

#include "q4_device.h"
#include "q4_internal.h"
#include "q4_rtn.h"

namespace q4 {

namespace {

struct Row8 {
  float v[8];
};

// 8 float16 weights of row n at channels k..k+7 (zeros outside the matrix)
__device__ __forceinline__ uint4 load_raw8(const uint16_t* __restrict__ W, int n, int N, int k, int K) {
  return (n < N && k < K) ? *reinterpret_cast<const uint4*>(W + (size_t)n * K + k) : make_uint4(0u, 0u, 0u, 0u);
}

__device__ __forceinline__ Row8 row8_of(uint4 raw) {
  Row8 o;
  const half8_t h = as_half8(raw);
#pragma unroll
  for (int e = 0; e < 8; ++e) o.v[e] = (float)h[e];
  return o;
}

__device__ __forceinline__ Row8 load_row8(const uint16_t* __restrict__ W, int n, int N, int k, int K) {
  return row8_of(load_raw8(W, n, N, k, K));
}

// Act-order columns ("Post-training quantization: GPTQ, AWQ and rotation",
// arganzheng.life, sections 五.3 and 十一.2): the quantizer reads the matrix with
// its columns permuted, column k of the permuted matrix being channel perm[k], so
// every act-order group is a contiguous run of g permuted columns. Each of the 8
// weights is a 2-byte gather from row n; indices are clamped into the row.
__device__ __forceinline__ Row8 load_row8_perm(const uint16_t* __restrict__ W, int n, int N, int k, int K,
                                               const int32_t* __restrict__ perm) {
  Row8 o;
  if (n < N && k < K) {
    const int4 p0 = *reinterpret_cast<const int4*>(perm + k);
    const int4 p1 = *reinterpret_cast<const int4*>(perm + k + 4);
    const int idx[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    const uint16_t* row = W + (size_t)n * K;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      o.v[e] = (float)__builtin_bit_cast(_Float16, row[min((unsigned)idx[e], (unsigned)(K - 1))]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) o.v[e] = 0.0f;
  }
  return o;
}

template <bool PERM>
__device__ __forceinline__ Row8 load_w8(const uint16_t* __restrict__ W, int n, int N, int k, int K,
                                        const int32_t* __restrict__ perm) {
  return PERM ? load_row8_perm(W, n, N, k, K, perm) : load_row8(W, n, N, k, K);
}

__device__ __forceinline__ float wave_max4(float a) {
  // maximum over lanes l, l^16, l^32, l^48 (the four k-quarters of one row)
  a = fmaxf(a, __shfl_xor(a, 16, 64));
  a = fmaxf(a, __shfl_xor(a, 32, 64));
  return a;
}
__device__ __forceinline__ float wave_min4(float a) {
  a = fminf(a, __shfl_xor(a, 16, 64));
  a = fminf(a, __shfl_xor(a, 32, 64));
  return a;
}

__device__ __forceinline__ uint16_t half_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }

// Symmetric scale of a group from its amax: fp16(fp32(amax) / 7), RNE to float16, formed
// as the product with the float32 constant fl(1/7), which rounds to the same float16 as
// the IEEE quotient for every positive float16 amax (checked for all of them on the
// host), so no divide is needed
__device__ __forceinline__ _Float16 sym_scale(float amax) { return (_Float16)(fmaxf(amax, 1e-12f) * (1.0f / 7.0f)); }

// r = rtn_recip(s): 0 for s == 0, which gives the code of q = 0 (and z = 0)
__device__ __forceinline__ uint32_t sym_code(float w, float r) {
  // offset-binary nibble q + 8, q = clamp(rint(w / s), -8, 7)
  const float q = fminf(fmaxf(rtn_quot(w, r), -8.0f), 7.0f);
  return (uint32_t)((int)q + 8);
}

__device__ __forceinline__ uint32_t asym_code(float w, float r, float z) {
  const float q = fminf(fmaxf(rtn_quot(w, r) + z, 0.0f), 15.0f);
  return (uint32_t)q;
}

__device__ __forceinline__ uint32_t pack_dword(const uint32_t nib[8]) {
  uint32_t d = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) d |= nib[e] << (4 * nibble_of(e));
  return d;
}

// GSUB = groups per 128-channel block (4: g = 32, 2: g = 64, 1: g = 128).
// Without act-order the grid holds only resident wavefronts, and each one walks its
// units with the next unit's weights already in flight, so loads overlap the coding
// of the current unit.
template <int GSUB, bool ASYM, bool PERM = false>
__global__ __launch_bounds__(256) void quant_block_kernel(const uint16_t* __restrict__ W, int N, int K, int S,
                                                          int Gp, int64_t units, uint4* __restrict__ packed,
                                                          uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros,
                                                          const int32_t* __restrict__ perm) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, c = lane >> 4;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  constexpr int MPG = 4 / GSUB;  // 32-channel steps per group

  // code one unit (tile t, block s) from its 32 weights per lane, store codes and scales
  auto code_unit = [&](const Row8 (&w)[4], int t, int s) __attribute__((always_inline)) {
    uint32_t dw[4];
#pragma unroll
    for (int gs = 0; gs < GSUB; ++gs) {
      float scale_f;
      float zero_f = 0.0f;
      _Float16 s16;
      if (!ASYM) {
        float a = 0.0f;
#pragma unroll
        for (int m = gs * MPG; m < (gs + 1) * MPG; ++m)
#pragma unroll
          for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(w[m].v[e]));
        a = wave_max4(a);
        s16 = sym_scale(a);
        scale_f = (float)s16;
      } else {
        float lo = INFINITY, hi = -INFINITY;
#pragma unroll
        for (int m = gs * MPG; m < (gs + 1) * MPG; ++m)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            lo = fminf(lo, w[m].v[e]);
            hi = fmaxf(hi, w[m].v[e]);
          }
        lo = wave_min4(lo);
        hi = wave_max4(hi);
        s16 = (_Float16)((hi - lo) / 15.0f);
        scale_f = (float)s16;
        // z = clamp(rint(-lo / s), 0, 15) by the same exact decision as the codes (-lo
        // is a float16 value); s == 0 gives z = 0
        zero_f = fminf(fmaxf(rtn_quot(-lo, rtn_recip(scale_f)), 0.0f), 15.0f);
      }
      const float rcp = rtn_recip(scale_f);
#pragma unroll
      for (int m = gs * MPG; m < (gs + 1) * MPG; ++m) {
        uint32_t nib[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          nib[e] = ASYM ? asym_code(w[m].v[e], rcp, zero_f) : sym_code(w[m].v[e], rcp);
        dw[m] = pack_dword(nib);
      }
      if (c == 0) {
        const size_t gi = ((size_t)t * Gp + (size_t)s * GSUB + gs) * kTileRows + r;
        scales[gi] = half_bits(s16);
        if (ASYM) zeros[gi] = (uint8_t)zero_f;
      }
    }
    packed[((size_t)t * S + s) * kWave + lane] = make_uint4(dw[0], dw[1], dw[2], dw[3]);
  };

  if constexpr (PERM) {
    for (int64_t u = wave; u < units; u += nwaves) {
      const int t = (int)(u / S), s = (int)(u % S);
      Row8 w[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        w[m] = load_row8_perm(W, t * kTileRows + r, N, s * kSuperK + m * kBlockK + 8 * c, K, perm);
      code_unit(w, t, s);
    }
  } else {
    // units u = wave, wave + nwaves, ...: the (tile, block) cursor advances by a fixed
    // step, and two register sets alternate so that the next unit's loads are in
    // flight while the current one is coded
    const int dt = (int)(nwaves / S), ds = (int)(nwaves % S);
    auto advance = [&](int& t, int& s) __attribute__((always_inline)) {
      s += ds;
      t += dt;
      if (s >= S) {
        s -= S;
        ++t;
      }
    };
    auto fetch = [&](uint4 (&dst)[4], int t, int s) __attribute__((always_inline)) {
      const int n = t * kTileRows + r;
      const int k0 = s * kSuperK + 8 * c;
      const uint16_t* base = W + (size_t)min(n, N - 1) * K + k0;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        dst[m] = (n < N && k0 + m * kBlockK < K) ? *reinterpret_cast<const uint4*>(base + m * kBlockK)
                                                 : make_uint4(0u, 0u, 0u, 0u);
    };
    auto code_raw = [&](const uint4 (&raw)[4], int t, int s) __attribute__((always_inline)) {
      Row8 w[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) w[m] = row8_of(raw[m]);
      code_unit(w, t, s);
    };
    int64_t u = wave;
    int t = (int)(u / S), s = (int)(u % S);
    uint4 ra[4], rb[4];
    if (u < units) fetch(ra, t, s);
    while (u < units) {
      int tn = t, sn = s;
      advance(tn, sn);
      const bool more = u + nwaves < units;
      if (more) fetch(rb, tn, sn);
      code_raw(ra, t, s);
      u += nwaves;
      t = tn;
      s = sn;
      if (!more) break;
      advance(tn, sn);
      const bool more2 = u + nwaves < units;
      if (more2) fetch(ra, tn, sn);
      code_raw(rb, t, s);
      u += nwaves;
      t = tn;
      s = sn;
    }
  }
}

// Symmetric INT4 with the clipping search of "Post-training quantization: GPTQ, AWQ
// and rotation" (arganzheng.life), section 三.2: per group, the ranges
// alpha * amax for alpha = p / 100, p = pmin .. 100, are tried; each gives the RTN
// scale of that range and codes clipped to the symmetric grid -7 .. 7, and the range
// whose codes reconstruct the group with the smallest squared error is kept (equal
// errors go to the larger alpha, so pmin = 100 is plain RTN). Same tile mapping as
// quant_block_kernel. The error of a candidate: every s16 * q - w is exact in
// float32, its square exact in float64; each lane sums its weights of the group in
// float64 and the four lanes of a row exchange partial sums (the same pairs on
// every lane, so the four agree on the choice).
__device__ __forceinline__ double wave_sum4(double a) {
  a += __shfl_xor(a, 16, 64);
  a += __shfl_xor(a, 32, 64);
  return a;
}

// clamp(rint(w / s), -7, 7) with r = rtn_recip(s) (0 for s == 0)
__device__ __forceinline__ float clip_q(float w, float r) { return fminf(fmaxf(rtn_quot(w, r), -7.0f), 7.0f); }

template <int GSUB>
__global__ __launch_bounds__(256) void quant_clip_kernel(const uint16_t* __restrict__ W, int N, int K, int S, int Gp,
                                                         int64_t units, int pmin, uint4* __restrict__ packed,
                                                         uint16_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, c = lane >> 4;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  constexpr int MPG = 4 / GSUB;

  for (int64_t u = wave; u < units; u += nwaves) {
    const int t = (int)(u / S), s = (int)(u % S);
    const int n = t * kTileRows + r;
    Row8 w[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) w[m] = load_row8(W, n, N, s * kSuperK + m * kBlockK + 8 * c, K);

    uint32_t dw[4];
#pragma unroll
    for (int gs = 0; gs < GSUB; ++gs) {
      float a = 0.0f;
#pragma unroll
      for (int m = gs * MPG; m < (gs + 1) * MPG; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(w[m].v[e]));
      a = wave_max4(a);
      double best_err = INFINITY;
      _Float16 s16 = (_Float16)0.0f;
      for (int p = pmin; p <= 100; ++p) {
        const float alpha = (float)p / 100.0f;
        const _Float16 sp = (_Float16)(fmaxf(a * alpha, 1e-12f) / 7.0f);
        const float sf = (float)sp;
        const float rp = rtn_recip(sf);
        double err = 0.0;
#pragma unroll
        for (int m = gs * MPG; m < (gs + 1) * MPG; ++m)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const double d = (double)(sf * clip_q(w[m].v[e], rp) - w[m].v[e]);
            err = __builtin_fma(d, d, err);
          }
        err = wave_sum4(err);
        if (err <= best_err) {  // ascending p: ties go to the larger alpha
          best_err = err;
          s16 = sp;
        }
      }
      const float rcp = rtn_recip((float)s16);
#pragma unroll
      for (int m = gs * MPG; m < (gs + 1) * MPG; ++m) {
        uint32_t nib[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) nib[e] = (uint32_t)((int)clip_q(w[m].v[e], rcp) + 8);
        dw[m] = pack_dword(nib);
      }
      if (c == 0) scales[((size_t)t * Gp + (size_t)s * GSUB + gs) * kTileRows + r] = half_bits(s16);
    }
    packed[((size_t)t * S + s) * kWave + lane] = make_uint4(dw[0], dw[1], dw[2], dw[3]);
  }
}

// Groups of g = 128*J channels, J >= 2: one wavefront per (tile, group); the
// group's blocks are read twice (reduction pass, then coding pass).
template <bool ASYM, bool PERM = false>
__global__ __launch_bounds__(256) void quant_wide_kernel(const uint16_t* __restrict__ W, int N, int K, int S, int J,
                                                         int Gp, int64_t units, uint4* __restrict__ packed,
                                                         uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros,
                                                         const int32_t* __restrict__ perm) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, c = lane >> 4;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);

  for (int64_t u = wave; u < units; u += nwaves) {
    const int t = (int)(u / Gp), j = (int)(u % Gp);
    const int n = t * kTileRows + r;
    float a = 0.0f, lo = INFINITY, hi = -INFINITY;
    for (int sb = 0; sb < J; ++sb) {
      const int s = j * J + sb;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const Row8 w = load_w8<PERM>(W, n, N, s * kSuperK + m * kBlockK + 8 * c, K, perm);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          a = fmaxf(a, fabsf(w.v[e]));
          lo = fminf(lo, w.v[e]);
          hi = fmaxf(hi, w.v[e]);
        }
      }
    }
    _Float16 s16;
    float scale_f, zero_f = 0.0f;
    if (!ASYM) {
      s16 = sym_scale(wave_max4(a));
      scale_f = (float)s16;
    } else {
      lo = wave_min4(lo);
      hi = wave_max4(hi);
      s16 = (_Float16)((hi - lo) / 15.0f);
      scale_f = (float)s16;
      zero_f = fminf(fmaxf(rtn_quot(-lo, rtn_recip(scale_f)), 0.0f), 15.0f);  // as in quant_block_kernel
    }
    const float rcp = rtn_recip(scale_f);
    for (int sb = 0; sb < J; ++sb) {
      const int s = j * J + sb;
      uint32_t dw[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const Row8 w = load_w8<PERM>(W, n, N, s * kSuperK + m * kBlockK + 8 * c, K, perm);
        uint32_t nib[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) nib[e] = ASYM ? asym_code(w.v[e], rcp, zero_f) : sym_code(w.v[e], rcp);
        dw[m] = pack_dword(nib);
      }
      packed[((size_t)t * S + s) * kWave + lane] = make_uint4(dw[0], dw[1], dw[2], dw[3]);
    }
    if (c == 0) {
      const size_t gi = ((size_t)t * Gp + j) * kTileRows + r;
      scales[gi] = half_bits(s16);
      if (ASYM) zeros[gi] = (uint8_t)zero_f;
    }
  }
}

// ---- per-channel INT8 (W8A16) -------------------------------------------------
//
// Symmetric INT8 with one scale per output channel: s = row amax / 127,
// q = clamp(round(w / s), -127, 127) ("量化：PTQ、GPTQ、AWQ 与 SmoothQuant",
// charles2530.github.io, the closing quick code example; "模型量化技术工程实践",
// www.iopencloud.com, section 2.1). A code needs its row's amax, so every 16-row
// tile is read twice: once for the row maxima, then per 16-row x 128-channel block,
// which is written as two 1 KiB halves (lane l = r + 16c stores row r, channels
// 64h + 32j + 8c + e at byte 8j + e of its 16 bytes in half h), codes offset by 128.

__device__ __forceinline__ uint32_t w8_code(float w, float r) {
  // offset-binary byte q + 128, q = clamp(rint(w / s), -127, 127), r = rtn_recip(s)
  // (code 0 for s == 0)
  const float q = fminf(fmaxf(rtn_quot(w, r), -127.0f), 127.0f);
  return (uint32_t)((int)q + 128);
}

// Both reads in one kernel: a workgroup of 8 wavefronts takes one 16-row tile at a
// time (persistent; two workgroups per CU). Wavefront w reduces the maxima of rows
// 2w and 2w+1 (8 loads of 16 bytes per lane in flight; rows past N get scale 0),
// the 16 reciprocal scales go through LDS, then wavefront w codes blocks w, w + 8,
// ... of the tile, re-reading it while it is still in the caches (two tiles per CU
// are in flight), so W mostly crosses HBM once.
__global__ __launch_bounds__(512) void w8_fused_kernel(const uint16_t* __restrict__ W, int N, int K, int S, int T,
                                                       uint16_t* __restrict__ scales, uint4* __restrict__ packed) {
  __shared__ float rcp_s[kTileRows];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;  // 0 .. 7
  const int r = lane & 15, c = lane >> 4;
  for (int t = blockIdx.x; t < T; t += gridDim.x) {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int n = t * kTileRows + 2 * wave + rr;
      float a = 0.0f;
      if (n < N) {
        const uint16_t* row = W + (size_t)n * K;  // K % 8 == 0: 16-byte aligned rows
#pragma unroll 8
        for (int k = lane * 8; k < K; k += kWave * 8) {
          const half8_t h = as_half8(*reinterpret_cast<const uint4*>(row + k));
#pragma unroll
          for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf((float)h[e]));
        }
      }
#pragma unroll
      for (int m = 1; m < kWave; m <<= 1) a = fmaxf(a, __shfl_xor(a, m, 64));
      // fp16(fp32(amax) / 127) through the constant fl(1/127): the same float16 for every
      // float16 amax (checked for all of them on the host); rows past N: 0
      const _Float16 s16 = (_Float16)(a * (1.0f / 127.0f));
      if (lane == 0) {
        scales[n] = half_bits(s16);
        rcp_s[2 * wave + rr] = rtn_recip((float)s16);
      }
    }
    __syncthreads();
    const float rcp = rcp_s[r];
    const int n = t * kTileRows + r;
    for (int s = wave; s < S; s += 8) {
      uint32_t d[8];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const Row8 w = load_row8(W, n, N, s * kSuperK + m * kBlockK + 8 * c, K);
#pragma unroll
        for (int i = 0; i < 2; ++i)
          d[2 * m + i] = w8_code(w.v[4 * i], rcp) | (w8_code(w.v[4 * i + 1], rcp) << 8) |
                         (w8_code(w.v[4 * i + 2], rcp) << 16) | (w8_code(w.v[4 * i + 3], rcp) << 24);
      }
      uint4* out = packed + ((size_t)t * S + s) * 2 * kWave + lane;
      out[0] = make_uint4(d[0], d[1], d[2], d[3]);
      out[kWave] = make_uint4(d[4], d[5], d[6], d[7]);
    }
    __syncthreads();  // rcp_s is rewritten for the next tile
  }
}

__device__ __forceinline__ size_t w8_dev_byte(int n, int k, int S) {
  const int t = n >> 4, r = n & 15, s = k >> 7, h = (k & 127) >> 6, j = (k & 63) >> 5, c = (k & 31) >> 3;
  return (((size_t)t * S + s) * 2 + h) * 1024 + (size_t)(r + 16 * c) * 16 + 8 * j + (k & 7);
}

__global__ void w8_to_canonical_kernel(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
                                       int N, int K, int S, int8_t* __restrict__ canon,
                                       uint16_t* __restrict__ canon_scales) {
  const int64_t total = (int64_t)N * K;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int n = (int)(i / K), k = (int)(i % K);
    canon[i] = (int8_t)((int)packed[w8_dev_byte(n, k, S)] - 128);
    if (k == 0) canon_scales[n] = scales[n];
  }
}

__global__ void w8_from_canonical_kernel(const int8_t* __restrict__ canon, const uint16_t* __restrict__ canon_scales,
                                         int N, int K, int S, int Np, int64_t dwords, uint32_t* __restrict__ packed,
                                         uint16_t* __restrict__ scales) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < dwords; i += (int64_t)gridDim.x * blockDim.x) {
    // dword i: block (t, s), half h, lane l, dword d of the lane's 16 bytes
    const int d = (int)(i & 3), l = (int)((i >> 2) & 63), h = (int)((i >> 8) & 1);
    const int64_t ts = i >> 9;
    const int t = (int)(ts / S), s = (int)(ts % S);
    const int n = t * 16 + (l & 15);
    const int k0 = s * 128 + 64 * h + 32 * (d >> 1) + 8 * (l >> 4) + 4 * (d & 1);
    uint32_t v = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = k0 + e;
      const uint32_t b = (n < N && k < K) ? (uint32_t)((int)canon[(size_t)n * K + k] + 128) : 128u;
      v |= b << (8 * e);
    }
    packed[i] = v;
    if (i < Np) scales[i] = i < N ? canon_scales[i] : (uint16_t)0;
  }
}

// ---- layout converters -------------------------------------------------------

__device__ __forceinline__ size_t dev_dword_index(int n, int k, int S) {
  const int t = n >> 4, r = n & 15, s = k >> 7, m = (k & 127) >> 5, c = (k & 31) >> 3;
  return (((size_t)t * S + s) * kWave + r + 16 * c) * 4 + m;
}

__global__ void to_canonical_codes_kernel(const uint32_t* __restrict__ packed, int N, int K, int S, bool asym,
                                          uint8_t* __restrict__ canon) {
  const int64_t total = (int64_t)N * (K / 2);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int n = (int)(i / (K / 2));
    const int k = (int)(i % (K / 2)) * 2;
    const uint32_t d = packed[dev_dword_index(n, k, S)];
    uint32_t lo = (d >> (4 * nibble_of(k & 7))) & 0xF;
    uint32_t hi = (d >> (4 * nibble_of((k + 1) & 7))) & 0xF;
    if (!asym) {  // offset binary -> 4-bit two's complement: (v - 8) mod 16 == v ^ 8
      lo ^= 8u;
      hi ^= 8u;
    }
    canon[i] = (uint8_t)(lo | (hi << 4));
  }
}

__global__ void from_canonical_codes_kernel(const uint8_t* __restrict__ canon, int N, int K, int S, bool asym,
                                            int64_t dwords, uint32_t* __restrict__ packed) {
  for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < dwords; d += (int64_t)gridDim.x * blockDim.x) {
    const int m = (int)(d & 3);
    const int64_t chunk = d >> 2;
    const int lane = (int)(chunk & 63);
    const int64_t ts = chunk >> 6;
    const int t = (int)(ts / S), s = (int)(ts % S);
    const int n = t * 16 + (lane & 15);
    const int k0 = s * kSuperK + m * kBlockK + 8 * (lane >> 4);
    uint32_t out = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = k0 + e;
      uint32_t v;
      if (n < N && k < K) {
        v = (canon[(size_t)n * (K / 2) + (k >> 1)] >> (4 * (k & 1))) & 0xF;
        if (!asym) v ^= 8u;
      } else {
        v = asym ? 0u : 8u;
      }
      out |= v << (4 * nibble_of(e));
    }
    packed[d] = out;
  }
}

template <typename T>
__global__ void groups_to_canonical_kernel(const T* __restrict__ dev, int N, int G, int Gp, T* __restrict__ canon) {
  const int64_t total = (int64_t)N * G;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int n = (int)(i / G), j = (int)(i % G);
    canon[i] = dev[((size_t)(n >> 4) * Gp + j) * 16 + (n & 15)];
  }
}

template <typename T>
__global__ void groups_from_canonical_kernel(const T* __restrict__ canon, int N, int G, int Gp, int64_t total,
                                             T* __restrict__ dev) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(i & 15);
    const int64_t tj = i >> 4;
    const int t = (int)(tj / Gp), j = (int)(tj % Gp);
    const int n = t * 16 + r;
    dev[i] = (n < N && j < G) ? canon[(size_t)n * G + j] : (T)0;
  }
}

inline int grid_for(int64_t work, int block) {
  int64_t g = (work + block - 1) / block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

// quant_block_kernel without act-order: a persistent grid of resident wavefronts
template <int GSUB, bool ASYM>
void launch_block(const QuantArgs& a, int S, int64_t units, hipStream_t stream) {
  const int block = 256;
  const void* fn = reinterpret_cast<const void*>(&quant_block_kernel<GSUB, ASYM, false>);
  const int grid = std::min(grid_for(units * kWave, block), resident_grid(fn, block));
  hipLaunchKernelGGL((quant_block_kernel<GSUB, ASYM, false>), dim3(grid), dim3(block), 0, stream,
                     static_cast<const uint16_t*>(a.W), a.N, a.K, S, a.Gp, units, static_cast<uint4*>(a.packed),
                     static_cast<uint16_t*>(a.scales), static_cast<uint8_t*>(a.zeros), nullptr);
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream) {
  const int S = a.Kp / kSuperK;
  const int T = a.Np / kTileRows;
  const int block = 256;
  const uint16_t* W = static_cast<const uint16_t*>(a.W);
  uint4* P = static_cast<uint4*>(a.packed);
  uint16_t* Sc = static_cast<uint16_t*>(a.scales);
  uint8_t* Z = static_cast<uint8_t*>(a.zeros);
  if (a.clip_pmin > 0) {  // symmetric, g <= 128 (checked by the caller)
    const int64_t units = (int64_t)T * S;
    const int grid = grid_for(units * kWave, block);
    if (a.group == 32)
      hipLaunchKernelGGL((quant_clip_kernel<4>), dim3(grid), dim3(block), 0, stream, W, a.N, a.K, S, a.Gp, units, a.clip_pmin, P, Sc);
    else if (a.group == 64)
      hipLaunchKernelGGL((quant_clip_kernel<2>), dim3(grid), dim3(block), 0, stream, W, a.N, a.K, S, a.Gp, units, a.clip_pmin, P, Sc);
    else
      hipLaunchKernelGGL((quant_clip_kernel<1>), dim3(grid), dim3(block), 0, stream, W, a.N, a.K, S, a.Gp, units, a.clip_pmin, P, Sc);
    return hipGetLastError();
  }
  const int32_t* perm = a.perm;
  if (a.group <= kSuperK) {
    const int64_t units = (int64_t)T * S;
    const int grid = grid_for(units * kWave, block);
    if (perm) {  // act-order: symmetric codes of the column-permuted matrix
      if (a.group == 32)
        hipLaunchKernelGGL((quant_block_kernel<4, false, true>), dim3(grid), dim3(block), 0, stream, W, a.N, a.K, S, a.Gp, units, P, Sc, Z, perm);
      else if (a.group == 64)
        hipLaunchKernelGGL((quant_block_kernel<2, false, true>), dim3(grid), dim3(block), 0, stream, W, a.N, a.K, S, a.Gp, units, P, Sc, Z, perm);
      else
        hipLaunchKernelGGL((quant_block_kernel<1, false, true>), dim3(grid), dim3(block), 0, stream, W, a.N, a.K, S, a.Gp, units, P, Sc, Z, perm);
    } else if (a.group == 32) {
      if (a.asym) launch_block<4, true>(a, S, units, stream);
      else launch_block<4, false>(a, S, units, stream);
    } else if (a.group == 64) {
      if (a.asym) launch_block<2, true>(a, S, units, stream);
      else launch_block<2, false>(a, S, units, stream);
    } else {
      if (a.asym) launch_block<1, true>(a, S, units, stream);
      else launch_block<1, false>(a, S, units, stream);
    }
  } else {
    const int J = a.group / kSuperK;
    const int64_t units = (int64_t)T * a.Gp;
    const int grid = grid_for(units * kWave, block);
    if (perm) hipLaunchKernelGGL((quant_wide_kernel<false, true>), dim3(grid), dim3(block), 0, stream, W, a.N, a.K, S, J, a.Gp, units, P, Sc, Z, perm);
    else if (a.asym) hipLaunchKernelGGL((quant_wide_kernel<true>), dim3(grid), dim3(block), 0, stream, W, a.N, a.K, S, J, a.Gp, units, P, Sc, Z, perm);
    else hipLaunchKernelGGL((quant_wide_kernel<false>), dim3(grid), dim3(block), 0, stream, W, a.N, a.K, S, J, a.Gp, units, P, Sc, Z, perm);
  }
  return hipGetLastError();
}

hipError_t launch_to_canonical(const LayoutArgs& a, hipStream_t stream) {
  const int S = a.Kp / kSuperK;
  const int G = a.K / a.group;
  const int block = 256;
  hipLaunchKernelGGL(to_canonical_codes_kernel, dim3(grid_for((int64_t)a.N * (a.K / 2), block)), dim3(block), 0,
                     stream, static_cast<const uint32_t*>(a.packed), a.N, a.K, S, a.asym,
                     static_cast<uint8_t*>(a.canon_codes));
  hipLaunchKernelGGL((groups_to_canonical_kernel<uint16_t>), dim3(grid_for((int64_t)a.N * G, block)), dim3(block), 0,
                     stream, static_cast<const uint16_t*>(a.scales), a.N, G, a.Gp,
                     static_cast<uint16_t*>(a.canon_scales));
  if (a.asym)
    hipLaunchKernelGGL((groups_to_canonical_kernel<uint8_t>), dim3(grid_for((int64_t)a.N * G, block)), dim3(block), 0,
                       stream, static_cast<const uint8_t*>(a.zeros), a.N, G, a.Gp,
                       static_cast<uint8_t*>(a.canon_zeros));
  return hipGetLastError();
}

hipError_t launch_from_canonical(const LayoutArgs& a, hipStream_t stream) {
  const int S = a.Kp / kSuperK;
  const int G = a.K / a.group;
  const int block = 256;
  const int64_t dwords = (int64_t)a.Np * a.Kp / 8;
  const int64_t gtotal = (int64_t)a.Np * a.Gp;
  hipLaunchKernelGGL(from_canonical_codes_kernel, dim3(grid_for(dwords, block)), dim3(block), 0, stream,
                     static_cast<const uint8_t*>(a.canon_codes), a.N, a.K, S, a.asym, dwords,
                     static_cast<uint32_t*>(a.packed));
  hipLaunchKernelGGL((groups_from_canonical_kernel<uint16_t>), dim3(grid_for(gtotal, block)), dim3(block), 0, stream,
                     static_cast<const uint16_t*>(a.canon_scales), a.N, G, a.Gp, gtotal,
                     static_cast<uint16_t*>(a.scales));
  if (a.asym)
    hipLaunchKernelGGL((groups_from_canonical_kernel<uint8_t>), dim3(grid_for(gtotal, block)), dim3(block), 0, stream,
                       static_cast<const uint8_t*>(a.canon_zeros), a.N, G, a.Gp, gtotal,
                       static_cast<uint8_t*>(a.zeros));
  return hipGetLastError();
}

hipError_t launch_quantize_w8(const W8Args& a, hipStream_t stream) {
  const int S = a.Kp / kSuperK;
  const int T = a.Np / kTileRows;
  const int block = 256;
  (void)block;
  const int grid = std::max(1, std::min(T, 2 * device_cu_count_cached()));
  hipLaunchKernelGGL(w8_fused_kernel, dim3(grid), dim3(512), 0, stream, static_cast<const uint16_t*>(a.W), a.N, a.K,
                     S, T, static_cast<uint16_t*>(a.scales), static_cast<uint4*>(a.packed));
  return hipGetLastError();
}

hipError_t launch_w8_to_canonical(const W8Args& a, hipStream_t stream) {
  const int block = 256;
  hipLaunchKernelGGL(w8_to_canonical_kernel, dim3(grid_for((int64_t)a.N * a.K, block)), dim3(block), 0, stream,
                     static_cast<const uint8_t*>(a.packed), static_cast<const uint16_t*>(a.scales), a.N, a.K,
                     a.Kp / kSuperK, static_cast<int8_t*>(a.canon_codes), static_cast<uint16_t*>(a.canon_scales));
  return hipGetLastError();
}

hipError_t launch_w8_from_canonical(const W8Args& a, hipStream_t stream) {
  const int block = 256;
  const int64_t dwords = (int64_t)a.Np * a.Kp / 4;
  hipLaunchKernelGGL(w8_from_canonical_kernel, dim3(grid_for(dwords, block)), dim3(block), 0, stream,
                     static_cast<const int8_t*>(a.canon_codes), static_cast<const uint16_t*>(a.canon_scales), a.N,
                     a.K, a.Kp / kSuperK, a.Np, dwords, static_cast<uint32_t*>(a.packed),
                     static_cast<uint16_t*>(a.scales));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Self-check of the division-free decision (q4_rtn.h) on the device: for every
// positive finite float16 scale s (one workgroup each) and every finite float16
// weight w, rtn_quot(w, rtn_recip(s)) against rintf of the correctly rounded float32
// quotient w / s (this file is built with correctly rounded division), counting the
// pairs with |w / s| < 341 where the two differ. counts[0] += pairs checked,
// counts[1] += mismatches (zeroed by the first kernel).
namespace {

constexpr int kPosFiniteFp16 = 0x7BFF;  // positive finite float16 bit patterns 0x0001..0x7BFF

__global__ void rtn_check_zero_kernel(unsigned long long* counts) {
  if (threadIdx.x < 2) counts[threadIdx.x] = 0ull;
}

__global__ __launch_bounds__(256) void rtn_check_kernel(unsigned long long* counts) {
  const uint16_t sb = (uint16_t)(blockIdx.x + 1);
  const float s = (float)__builtin_bit_cast(_Float16, sb);
  const float r = rtn_recip(s);
  unsigned int bad = 0, checked = 0;
  for (int i = threadIdx.x; i < 2 * (kPosFiniteFp16 + 1); i += blockDim.x) {
    const uint16_t wb = (uint16_t)(i <= kPosFiniteFp16 ? i : 0x8000 + (i - kPosFiniteFp16 - 1));
    const float w = (float)__builtin_bit_cast(_Float16, wb);
    const float q = w / s;
    ++checked;
    if (fabsf(q) < 341.0f && rtn_quot(w, r) != rintf(q)) ++bad;
  }
  // wavefront sums, then one atomic per wavefront
  for (int m = 32; m >= 1; m >>= 1) {
    bad += __shfl_xor(bad, m);
    checked += __shfl_xor(checked, m);
  }
  if ((threadIdx.x & 63) == 0) {
    atomicAdd(&counts[0], (unsigned long long)checked);
    atomicAdd(&counts[1], (unsigned long long)bad);
  }
}

}  // namespace

hipError_t launch_rtn_check(unsigned long long* counts, hipStream_t stream) {
  hipLaunchKernelGGL(rtn_check_zero_kernel, dim3(1), dim3(64), 0, stream, counts);
  hipLaunchKernelGGL(rtn_check_kernel, dim3(kPosFiniteFp16), dim3(256), 0, stream, counts);
  return hipGetLastError();
}

}  // namespace q4
