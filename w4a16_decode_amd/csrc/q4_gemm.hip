// Fused dequantize-and-multiply W4A16 kernel: y[b][n] = sum_k x[b][k] * w_hat[n][k].
//
// The weight GEMM of decode reads every weight once per step and is bound by those
// bytes ("LLM 后训练量化深度实战…", www.ybb.press, section 一); under W4A16 the INT4
// weights are read from HBM, dequantized on chip and multiplied with the 16-bit
// activations, and a per-group scale has to be applied inside the k-accumulation
// rather than in an epilogue ("Post-training quantization: GPTQ, AWQ and rotation",
// arganzheng.life, sections 二.2 and 二.3).
//
// Mapping onto gfx950:
//  * One 16-row x 128-channel block of packed codes (1 KiB) is one 16-byte load per
//    lane of a wavefront; the device layout puts each lane's 16 bytes in the A-operand
//    order of v_mfma_f32_16x16x32_f16 (lane l -> row l%16, channels 8*(l/16)..+7 of
//    each 32-channel step), so codes go HBM -> VGPR -> dequant -> MFMA with no LDS.
//  * Dequantization is exact in float16 (magic-number OR + one packed add/fma per
//    pair, see dequant8), so the MFMA contracts the integer codes against float16 x
//    with float32 accumulation; each group's partial is scaled in float32.
//  * The batch (B <= 16) fills the 16 MFMA columns; larger B uses up to 4 column
//    tiles per wavefront and more workgroups along y.
//  * A workgroup owns R row tiles; its wavefronts split the channel range and the
//    partial sums are reduced through LDS in a fixed order (deterministic).
#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {
namespace {

__device__ __forceinline__ uint32_t lane_dword(const uint4& v, int m) {
  return m == 0 ? v.x : m == 1 ? v.y : m == 2 ? v.z : v.w;
}

__device__ __forceinline__ float4_t mfma16x16x32(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// GSUB: groups per 128-channel block (4: g = 32, 2: g = 64, 1: g = 128*J).
template <int R, int NT, int GSUB, bool ASYM>
__global__ __launch_bounds__(512) void gemm_kernel(const uint16_t* __restrict__ x, int B,
                                                   const uint4* __restrict__ packed,
                                                   const uint16_t* __restrict__ scales,
                                                   const uint8_t* __restrict__ zeros, int N, int K, int T, int S,
                                                   int Gp, int J, uint16_t* __restrict__ y) {
  extern __shared__ float red[];
  constexpr int MPG = 4 / GSUB;  // 32-channel steps per group inside a block
  const int W = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tile0 = blockIdx.x * R;
  const int col0 = blockIdx.y * NT;
  const int sb0 = (int)(((int64_t)S * wave) / W);
  const int sb1 = (int)(((int64_t)S * (wave + 1)) / W);
  const int kq = lane >> 4;        // 8-channel slice fed by this lane in each 32-channel step
  const int crow = 4 * (lane >> 4);  // first of the 4 accumulator rows held by this lane
  const int arow = lane & 15;        // A-operand row (weight row) held by this lane

  int tiles[R];
#pragma unroll
  for (int r = 0; r < R; ++r) tiles[r] = min(tile0 + r, T - 1);  // clamped: loads stay in bounds

  float4_t acc[R][NT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[r][c] = float4_t{0.f, 0.f, 0.f, 0.f};

  const half8_t zero8 = {};
  const half2_t sym_lo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const half2_t sym_hi = {(_Float16)-72.0f, (_Float16)-72.0f};

  for (int s = sb0; s < sb1; ++s) {
    uint4 wq[R];
#pragma unroll
    for (int r = 0; r < R; ++r) wq[r] = packed[((size_t)tiles[r] * S + s) * kWave + lane];

    half8_t xb[NT][4];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      const int b = (col0 + c) * 16 + (lane & 15);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int k = s * kSuperK + m * kBlockK + 8 * kq;
        xb[c][m] = (b < B && k < K) ? as_half8(*reinterpret_cast<const uint4*>(x + (size_t)b * K + k)) : zero8;
      }
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int gs = 0; gs < GSUB; ++gs) {
        const int j = (GSUB == 1) ? s / J : s * GSUB + gs;
        const size_t gbase = ((size_t)tiles[r] * Gp + j) * 16;
        const uint2 sraw = *reinterpret_cast<const uint2*>(scales + gbase + crow);
        const half4_t sh = __builtin_bit_cast(half4_t, sraw);
        const float4_t sc = {(float)sh[0], (float)sh[1], (float)sh[2], (float)sh[3]};
        half2_t blo = sym_lo, bhi = sym_hi;
        if (ASYM) {
          const _Float16 z = (_Float16)(float)zeros[gbase + arow];
          blo = half2_t{(_Float16)-1024.0f - z, (_Float16)-1024.0f - z};
          bhi = half2_t{(_Float16)-64.0f - z, (_Float16)-64.0f - z};
        }
        half8_t a[MPG];
#pragma unroll
        for (int mm = 0; mm < MPG; ++mm) a[mm] = dequant8(lane_dword(wq[r], gs * MPG + mm), blo, bhi);
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          float4_t part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int mm = 0; mm < MPG; ++mm) part = mfma16x16x32(a[mm], xb[c][gs * MPG + mm], part);
          acc[r][c] += sc * part;
        }
      }
    }
  }

  // Output: accumulator element i of lane l in tile (r, c) is row 16*tile + crow + i,
  // batch column 16*(col0 + c) + l%16.
  if (W == 1) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (tile0 + r >= T) continue;
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        const int b = (col0 + c) * 16 + (lane & 15);
        if (b >= B) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = (tile0 + r) * 16 + crow + i;
          if (n < N) y[(size_t)b * N + n] = __builtin_bit_cast(uint16_t, (_Float16)acc[r][c][i]);
        }
      }
    }
    return;
  }

  constexpr int PER_WAVE = R * NT * 256;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave * PER_WAVE + (r * NT + c) * 256 + i * 64 + lane] = acc[r][c][i];
  __syncthreads();
  for (int e = threadIdx.x; e < PER_WAVE; e += blockDim.x) {
    float sum = 0.f;
    for (int w = 0; w < W; ++w) sum += red[w * PER_WAVE + e];
    const int rc = e >> 8, i = (e >> 6) & 3, ln = e & 63;
    const int r = rc / NT, c = rc % NT;
    const int n = (tile0 + r) * 16 + 4 * (ln >> 4) + i;
    const int b = (col0 + c) * 16 + (ln & 15);
    if (tile0 + r < T && n < N && b < B) y[(size_t)b * N + n] = __builtin_bit_cast(uint16_t, (_Float16)sum);
  }
}

template <int R, int NT, int GSUB, bool ASYM>
hipError_t launch_t(const GemmArgs& a, hipStream_t stream) {
  const int T = a.Np / kTileRows;
  const int S = a.Kp / kSuperK;
  const int J = a.group >= kSuperK ? a.group / kSuperK : 1;
  const int W = a.waves_per_group;
  const int col_tiles_total = (a.B + 15) / 16;
  dim3 grid((T + R - 1) / R, (col_tiles_total + NT - 1) / NT);
  dim3 block(W * kWave);
  const size_t lds = W > 1 ? (size_t)W * R * NT * 256 * sizeof(float) : 0;
  hipLaunchKernelGGL((gemm_kernel<R, NT, GSUB, ASYM>), grid, block, lds, stream,
                     static_cast<const uint16_t*>(a.x), a.B, static_cast<const uint4*>(a.packed),
                     static_cast<const uint16_t*>(a.scales), static_cast<const uint8_t*>(a.zeros), a.N, a.K, T, S,
                     a.Gp, J, static_cast<uint16_t*>(a.y));
  return hipGetLastError();
}

template <int R, int NT, bool ASYM>
hipError_t launch_g(const GemmArgs& a, hipStream_t stream) {
  if (a.group == 32) return launch_t<R, NT, 4, ASYM>(a, stream);
  if (a.group == 64) return launch_t<R, NT, 2, ASYM>(a, stream);
  return launch_t<R, NT, 1, ASYM>(a, stream);
}

template <int R, int NT>
hipError_t launch_a(const GemmArgs& a, hipStream_t stream) {
  return a.asym ? launch_g<R, NT, true>(a, stream) : launch_g<R, NT, false>(a, stream);
}

template <int NT>
hipError_t launch_r(const GemmArgs& a, hipStream_t stream) {
  switch (a.rows_per_wave) {
    case 1: return launch_a<1, NT>(a, stream);
    case 2: return launch_a<2, NT>(a, stream);
    default: return launch_a<4, NT>(a, stream);
  }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  switch (a.col_tiles) {
    case 1: return launch_r<1>(a, stream);
    case 2: return launch_r<2>(a, stream);
    default: return launch_r<4>(a, stream);
  }
}

}  // namespace q4
