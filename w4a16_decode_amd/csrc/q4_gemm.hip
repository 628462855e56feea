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
//  * The batch (B <= 16) fills the 16 MFMA columns of the GEMV; its wavefronts
//    split the channel range and their partial sums are reduced through LDS in a
//    fixed order (deterministic). Larger B runs the skinny GEMM: 2 to 8 column
//    tiles of 16 batch rows per workgroup, staged through LDS and shared by its
//    four wavefronts, each owning whole row tiles.
#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>

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

// ---------------------------------------------------------------------------------
// GEMV kernel for B <= 16 (one 16-column MFMA tile), persistent.
//
// The grid is sized to what the GPU holds at once. Workgroup g owns k-split
// ks = g % KS of the channel range and the row blocks (R tiles of 16 rows)
// g/KS, g/KS + G/KS, ... Its W wavefronts split the k-split's channel range; each
// wavefront streams its blocks of codes and scales for one row block after the
// other with P-1 blocks in flight (vector loads retire in order, so only weights
// ride that pipeline), and reads its activation operands from LDS: the workgroup
// copies its slice of x (all B rows) into LDS once, for all its row blocks. After
// the last block of a row block the wavefronts' partial sums are reduced through
// LDS (double-buffered, one barrier per row block) while the loads for the next
// row block are already in flight. With KS > 1 the workgroups write float32
// partials to the workspace and reduce_splits_kernel adds them in a fixed order.
template <int R, int GSUB, bool ASYM>
struct WStage {
  uint4 w[R];
  uint2 sc[R][GSUB];
  uint32_t z[R][GSUB];
};

constexpr int kXChunksPerThread = 8;  // x slice <= 8 * 16 B * blockDim

// LDS layout of one GEMV workgroup, in bytes (shared with the host-side sizing).
struct GemvLds {
  size_t x, beta, red, out, total;
  __host__ __device__ GemvLds(int B, int nsb, int GSUB, bool bias, int W, int R, int n_rb) {
    x = ((((size_t)B * (nsb * kSuperK + 8) + kSuperK) * 2) + 15) & ~(size_t)15;  // x rows + zero row
    beta = bias ? (((size_t)B * nsb * GSUB + 1 + 3) / 4 * 4) * 4 : 0;            // per-unit biases + a zero
    red = 2 * (size_t)W * R * 256 * 4;                                           // two reduction buffers
    out = (size_t)n_rb * R * 16 * B * 4;                                         // results until the final store
    total = x + beta + red + out;
  }
};

#ifndef Q4_GEMV_WAVES_R1
#define Q4_GEMV_WAVES_R1 4
#endif
#ifndef Q4_GEMV_WAVES_R2
#define Q4_GEMV_WAVES_R2 4
#endif
// Register budget for one group per block (g >= 128): at least Q4_GEMV_WAVES_R*
// wavefronts per SIMD (512 / waves VGPRs). Smaller groups keep more scales per
// block and run without a budget rather than spill.
template <int R, int GSUB, bool ASYM, int P, bool NTL>
__global__ __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu((GSUB > 1 || R > 2) ? 1 : (R == 1 ? Q4_GEMV_WAVES_R1 : Q4_GEMV_WAVES_R2), 8)))
void gemv_kernel(const uint16_t* __restrict__ x, int B,
                                                   const uint4* __restrict__ packed,
                                                   const uint16_t* __restrict__ scales,
                                                   const uint8_t* __restrict__ zeros, int N, int K, int T, int S,
                                                   int Gp, int J, int KS, int nRB, uint16_t* __restrict__ y,
                                                   float* __restrict__ ws) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int MPG = 4 / GSUB;
  constexpr int PER_WAVE = R * 256;  // floats of one wavefront's partial sums
  // Symmetric codes skip the per-pair bias removal (magic8r) and subtract a
  // per-unit bias from the float32 partial instead; a unit is the channel run one
  // partial covers (128 / GSUB).
  constexpr bool BIAS = !ASYM;
  constexpr int UNIT = kSuperK / GSUB;
  const int W = blockDim.x >> 6;
  // readfirstlane: the wavefront index is uniform, and saying so keeps every value
  // derived from it (block ranges, addresses, loop bounds) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ks = blockIdx.x % KS;
  const int rb_first = blockIdx.x / KS;
  const int rb_stride = gridDim.x / KS;
  const int wsb0 = (int)(((int64_t)S * ks) / KS);
  const int wsb1 = (int)(((int64_t)S * (ks + 1)) / KS);
  const int nsb = wsb1 - wsb0;
  const int sb0 = wsb0 + (int)(((int64_t)nsb * wave) / W);
  const int sb1 = wsb0 + (int)(((int64_t)nsb * (wave + 1)) / W);
  const int nsw = sb1 - sb0;  // >= 1: the host keeps W <= S / KS
  const int n_rb = rb_first < nRB ? (nRB - 1 - rb_first) / rb_stride + 1 : 0;
  const int total = n_rb * nsw;  // blocks this wavefront streams
  const int KR = nsb * kSuperK;
  const int xstride = KR + 8;  // halfs per x row in LDS (16-byte pad against bank conflicts)
  const int nunits = nsb * GSUB;
  const GemvLds lay(B, nsb, GSUB, BIAS, W, R, n_rb);
  uint16_t* xl = reinterpret_cast<uint16_t*>(smem);      // x (x/16 at the scaled elements when BIAS)
  uint16_t* xzero = xl + B * xstride;                     // 128 zero halfs for absent batch rows
  float* beta = reinterpret_cast<float*>(smem + lay.x);
  float* red0 = reinterpret_cast<float*>(smem + lay.x + lay.beta);
  float* outb = reinterpret_cast<float*>(smem + lay.x + lay.beta + lay.red);
  const int kq = lane >> 4;
  const int crow = 4 * (lane >> 4);
  const int arow = lane & 15;
  const int bcol = lane & 15;

  // 1. the workgroup's x slice -> registers. Every load is issued (indices clamped
  //    into x) so the wait before the LDS copy counts exactly these loads, not the
  //    weight loads issued after them.
  const int row_chunks = KR >> 3;
  const int xchunks = B * row_chunks;
  uint4 xr[kXChunksPerThread];
#pragma unroll
  for (int i = 0; i < kXChunksPerThread; ++i) {
    const int idx = min((int)threadIdx.x + i * (int)blockDim.x, xchunks - 1);
    const int b = idx / row_chunks;
    const int k = min(wsb0 * kSuperK + (idx - b * row_chunks) * 8, K - 8);
    xr[i] = *reinterpret_cast<const uint4*>(x + (size_t)b * K + k);
  }

  // 2. the first P-1 blocks of codes / scales. Block addresses are wave-uniform
  //    (tile base + 1 KiB per block); only the lane offsets live in VGPRs. Loads are
  //    unconditional: after the last block the counters stay put and the trailing
  //    prefetches re-read it, which keeps the loop free of branches around loads.
  const unsigned char* pk = reinterpret_cast<const unsigned char*>(packed);
  const uint32_t w_lane = (uint32_t)lane * 16u;
  const uint32_t s_lane = (uint32_t)crow * 2u;
  int l_rb = rb_first, l_s = sb0, loads_left = total;
  int l_j = (GSUB == 1) ? sb0 / J : sb0 * GSUB, l_jr = (GSUB == 1) ? sb0 % J : 0;
  const unsigned char* l_wt[R];
  const unsigned char* l_st[R];
  auto set_tiles = [&]() {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const size_t tile = (size_t)min(l_rb * R + r, T - 1);
      l_wt[r] = pk + tile * S * 1024;
      l_st[r] = reinterpret_cast<const unsigned char*>(scales) + tile * Gp * 32;
    }
  };
  set_tiles();
  auto load = [&](WStage<R, GSUB, ASYM>& st) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const unsigned char* wp = l_wt[r] + (size_t)l_s * 1024 + w_lane;
      if (NTL) st.w[r] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wp)));
      else st.w[r] = *reinterpret_cast<const uint4*>(wp);
#pragma unroll
      for (int gs = 0; gs < GSUB; ++gs) {
        const size_t goff = (size_t)(l_j + gs) * 32;
        st.sc[r][gs] = *reinterpret_cast<const uint2*>(l_st[r] + goff + s_lane);
        if (ASYM) st.z[r][gs] = zeros[(size_t)((l_st[r] - reinterpret_cast<const unsigned char*>(scales)) >> 1) +
                                      (goff >> 1) + arow];
      }
    }
    if (--loads_left <= 0) return;
    if (GSUB == 1) {
      if (++l_jr == J) {
        l_jr = 0;
        ++l_j;
      }
    } else {
      l_j += GSUB;
    }
    if (++l_s == sb1) {
      l_s = sb0;
      l_j = (GSUB == 1) ? sb0 / J : sb0 * GSUB;
      l_jr = (GSUB == 1) ? sb0 % J : 0;
      l_rb += rb_stride;
      set_tiles();
    }
  };
  WStage<R, GSUB, ASYM> buf[P];
#pragma unroll
  for (int p = 0; p < P - 1; ++p) load(buf[p]);

  // 3. x slice -> LDS (elements 2, 3, 6, 7 of every 8 divided by 16 when BIAS: exact
  //    powers of two; channels past K are zero), plus the zero row
#pragma unroll
  for (int i = 0; i < kXChunksPerThread; ++i) {
    const int idx = threadIdx.x + i * blockDim.x;
    if (idx < xchunks) {
      const int b = idx / row_chunks;
      const int c8 = idx - b * row_chunks;
      uint4 v = (wsb0 * kSuperK + c8 * 8 < K) ? xr[i] : make_uint4(0u, 0u, 0u, 0u);
      if (BIAS) {
        half8_t h = as_half8(v);
        h[2] *= (_Float16)0.0625f;
        h[3] *= (_Float16)0.0625f;
        h[6] *= (_Float16)0.0625f;
        h[7] *= (_Float16)0.0625f;
        v = __builtin_bit_cast(uint4, h);
      }
      *reinterpret_cast<uint4*>(xl + b * xstride + c8 * 8) = v;
    }
  }
  if (threadIdx.x < kSuperK / 8) *reinterpret_cast<uint4*>(xzero + threadIdx.x * 8) = make_uint4(0u, 0u, 0u, 0u);
  lds_barrier();
  if (BIAS) {
    // bias of every (batch row, unit): 1032 * (sum of plain elements) + 1152 * (sum of scaled elements)
    for (int e = threadIdx.x; e < B * nunits; e += blockDim.x) {
      const int b = e / nunits, u = e - b * nunits;
      const uint16_t* xs = xl + b * xstride + u * UNIT;
      float plain = 0.f, scaled = 0.f;
      for (int c = 0; c < UNIT; c += 8) {
        const half8_t h = *reinterpret_cast<const half8_t*>(xs + c);
        plain += ((float)h[0] + (float)h[1]) + ((float)h[4] + (float)h[5]);
        scaled += ((float)h[2] + (float)h[3]) + ((float)h[6] + (float)h[7]);
      }
      beta[e] = 1032.f * plain + 1152.f * scaled;
    }
    if (threadIdx.x == 0) beta[B * nunits] = 0.f;
    lds_barrier();
  }

  float4_t acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = float4_t{0.f, 0.f, 0.f, 0.f};
  const DequantRegs dq = DequantRegs::make();
  // LDS read pointers of this lane's activation operand and bias; lanes of absent
  // batch rows stay on the zero row / zero bias (step 0)
  const bool real_col = bcol < B;
  const uint16_t* xlane0 = real_col ? xl + bcol * xstride + (sb0 - wsb0) * kSuperK + 8 * kq : xzero + 8 * kq;
  const int xstep = real_col ? kSuperK : 0;
  const float* blane0 = real_col ? beta + bcol * nunits + (sb0 - wsb0) * GSUB : beta + B * nunits;
  const int bstep = real_col ? GSUB : 0;
  const uint16_t* xp = xlane0;
  const float* bp = blane0;
  int c_i = 0, c_s = sb0, parity = 0;  // row block (index among this workgroup's) and block being computed

  // activation operands (and biases) of the block being computed, read from LDS
  // one block ahead so the LDS latency hides behind the previous block's work
  half8_t xb[4];
  float bu[GSUB];
  auto read_x = [&]() {
#pragma unroll
    for (int m = 0; m < 4; ++m) xb[m] = *reinterpret_cast<const half8_t*>(xp + m * kBlockK);
    if (BIAS) {
#pragma unroll
      for (int gs = 0; gs < GSUB; ++gs) bu[gs] = bp[gs];
    }
  };
  read_x();

  auto compute = [&](const WStage<R, GSUB, ASYM>& st) {
    half8_t xc[4];
    float bc[GSUB];
#pragma unroll
    for (int m = 0; m < 4; ++m) xc[m] = xb[m];
#pragma unroll
    for (int gs = 0; gs < GSUB; ++gs) bc[gs] = BIAS ? bu[gs] : 0.f;
    // next block of the same row block, or the first block of the next one
    const bool last = c_s + 1 == sb1;
    xp = last ? xlane0 : xp + xstep;
    bp = last ? blane0 : bp + bstep;
    read_x();
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int gs = 0; gs < GSUB; ++gs) {
        const half4_t sh = __builtin_bit_cast(half4_t, st.sc[r][gs]);
        float4_t part = {0.f, 0.f, 0.f, 0.f};
        if (BIAS) {
#pragma unroll
          for (int mm = 0; mm < MPG; ++mm)
            part = mfma16x16x32(magic8r(lane_dword(st.w[r], gs * MPG + mm), dq), xc[gs * MPG + mm], part);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[r][i] = __builtin_fmaf((float)sh[i], part[i] - bc[gs], acc[r][i]);
        } else {
          const _Float16 z = (_Float16)(float)st.z[r][gs];
          const half2_t blo = {(_Float16)-1024.0f - z, (_Float16)-1024.0f - z};
          const half2_t bhi = {(_Float16)-64.0f - z, (_Float16)-64.0f - z};
#pragma unroll
          for (int mm = 0; mm < MPG; ++mm)
            part = mfma16x16x32(dequant8r(lane_dword(st.w[r], gs * MPG + mm), dq, blo, bhi), xc[gs * MPG + mm], part);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[r][i] = __builtin_fmaf((float)sh[i], part[i], acc[r][i]);
        }
      }
    }
    if (++c_s < sb1) return;
    // Row block finished: reduce the W partial sums into the LDS result buffer
    // (every wavefront gets here once per row block; no global memory access).
    float* red = red0 + parity * (W * PER_WAVE);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave * PER_WAVE + r * 256 + i * 64 + lane] = acc[r][i];
    lds_barrier();
    for (int e = threadIdx.x; e < PER_WAVE; e += blockDim.x) {
      const int ln = e & 63;
      const int b = ln & 15;
      if (b < B) {
        float sum = 0.f;
        for (int w = 0; w < W; ++w) sum += red[w * PER_WAVE + e];
        const int r = e >> 8, i = (e >> 6) & 3;
        outb[((c_i * R + r) * 16 + 4 * (ln >> 4) + i) * B + b] = sum;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = float4_t{0.f, 0.f, 0.f, 0.f};
    parity ^= 1;
    c_s = sb0;
    ++c_i;
  };

  for (int it = 0; it < total; it += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      load(buf[(p + P - 1) % P]);
      if (it + p < total) compute(buf[p]);
    }
  }

  // 4. results of all row blocks: LDS -> y (or the k-split workspace)
  lds_barrier();
  const int nout = n_rb * R * 16 * B;
  for (int e = threadIdx.x; e < nout; e += blockDim.x) {
    const int b = e % B;
    const int rowi = e / B;  // (i * R + r) * 16 + row
    const int i = rowi / (R * 16), rr = rowi % (R * 16);
    const int n = (rb_first + i * rb_stride) * R * 16 + rr;
    if (n < N) {
      if (KS == 1) y[(size_t)b * N + n] = __builtin_bit_cast(uint16_t, (_Float16)outb[e]);
      else ws[((size_t)ks * B + b) * N + n] = outb[e];
    }
  }
}

__global__ void reduce_splits_kernel(const float* __restrict__ ws, int KS, int64_t BN, uint16_t* __restrict__ y) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < BN; i += (int64_t)gridDim.x * blockDim.x) {
    float sum = 0.f;
    for (int k = 0; k < KS; ++k) sum += ws[(size_t)k * BN + i];
    y[i] = __builtin_bit_cast(uint16_t, (_Float16)sum);
  }
}

// Resident workgroups per CU for a kernel / block / LDS combination, and the CU
// count of the current device; both are fixed for a process, so they are looked
// up once and remembered.
int resident_per_cu(const void* fn, int block, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<const void*, int, size_t>, int> cache;
  std::lock_guard<std::mutex> lk(mu);
  auto key = std::make_tuple(fn, block, lds);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, block, lds) != hipSuccess || nb < 1) nb = 1;
  cache[key] = nb;
  return nb;
}

int device_cus() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  cache[dev] = cus;
  return cus;
}

template <int R, int GSUB, bool ASYM>
hipError_t launch_gemv_t(const GemmArgs& a, hipStream_t stream) {
#ifndef Q4_GEMV_DEPTH_R1
#define Q4_GEMV_DEPTH_R1 8
#endif
#ifndef Q4_GEMV_DEPTH_R2
#define Q4_GEMV_DEPTH_R2 4
#endif
  // pipeline depth (blocks of codes in flight + 1) per row-tile count; fixed at
  // build time (the macros exist so tuning builds can try other depths)
  constexpr int P = R == 1 ? Q4_GEMV_DEPTH_R1 : (R == 2 ? Q4_GEMV_DEPTH_R2 : 4);
  constexpr bool NTL = true;
  const int T = a.Np / kTileRows;
  const int S = a.Kp / kSuperK;
  const int J = a.group >= kSuperK ? a.group / kSuperK : 1;
  const int W = a.waves_per_group;
  const int KS = a.k_splits;
  const int nRB = (T + R - 1) / R;
  const int max_nsb = (S + KS - 1) / KS;
  const void* fn = reinterpret_cast<const void*>(&gemv_kernel<R, GSUB, ASYM, P, NTL>);
  // Persistent grid: as many workgroups as stay resident (measured with the LDS of
  // one row block per workgroup), with the row blocks spread evenly over them; more
  // workgroups if the per-workgroup result buffer would not fit.
  const size_t lds1 = GemvLds(a.B, max_nsb, GSUB, !ASYM, W, R, 1).total;
  const int64_t resident = (int64_t)resident_per_cu(fn, W * kWave, lds1) * device_cus();
  const int64_t units = (int64_t)nRB * KS;
  int64_t rounds = (units + resident - 1) / resident;
  // each further row block per workgroup adds its results to the LDS buffer
  const size_t out1 = (size_t)R * 16 * a.B * 4;
  const size_t lim = a.lds_limit > lds1 ? a.lds_limit : lds1;
  const int64_t max_rounds = std::max<int64_t>(1, (int64_t)((lim - lds1) / out1) + 1);
  rounds = std::min(rounds, max_rounds);
  int64_t per_split = ((int64_t)nRB + rounds - 1) / rounds;
  if (a.grid_limit > 0) per_split = std::min<int64_t>(per_split, std::max(1, a.grid_limit / KS));
  const int n_rb_max = (int)((nRB + per_split - 1) / per_split);
  const size_t lds = GemvLds(a.B, max_nsb, GSUB, !ASYM, W, R, n_rb_max).total;
  const int grid = (int)(per_split * KS);
  hipLaunchKernelGGL((gemv_kernel<R, GSUB, ASYM, P, NTL>), dim3(grid), dim3(W * kWave), lds, stream,
                     static_cast<const uint16_t*>(a.x), a.B, static_cast<const uint4*>(a.packed),
                     static_cast<const uint16_t*>(a.scales), static_cast<const uint8_t*>(a.zeros), a.N, a.K, T, S,
                     a.Gp, J, KS, nRB, static_cast<uint16_t*>(a.y), static_cast<float*>(a.workspace));
  if (KS > 1) {
    const int64_t BN = (int64_t)a.B * a.N;
    int64_t blocks = (BN + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const float*>(a.workspace), KS, BN, static_cast<uint16_t*>(a.y));
  }
  return hipGetLastError();
}

template <int R, bool ASYM>
hipError_t launch_gemv_g(const GemmArgs& a, hipStream_t stream) {
  if (a.group == 32) return launch_gemv_t<R, 4, ASYM>(a, stream);
  if (a.group == 64) return launch_gemv_t<R, 2, ASYM>(a, stream);
  return launch_gemv_t<R, 1, ASYM>(a, stream);
}

template <int R>
hipError_t launch_gemv_a(const GemmArgs& a, hipStream_t stream) {
  return a.asym ? launch_gemv_g<R, true>(a, stream) : launch_gemv_g<R, false>(a, stream);
}

hipError_t launch_gemv(const GemmArgs& a, hipStream_t stream) {
  switch (a.rows_per_wave) {
    case 1: return launch_gemv_a<1>(a, stream);
    case 2: return launch_gemv_a<2>(a, stream);
    default: return launch_gemv_a<4>(a, stream);
  }
}

// ---------------------------------------------------------------------------------
// Skinny GEMM for B > 16 (MFMA-bound from a few dozen rows of x upward).
//
// Workgroup = 4 wavefronts; wavefront w owns row tiles 4*RT*blockIdx.x + RT*w + r,
// the workgroup owns column tiles CT*blockIdx.y .. + CT - 1 (16 batch rows each).
// Codes are dequantized exactly to float16 integers (q, or q - z) in registers, as
// in the GEMV; each group's MFMA partial sum is scaled in float32 and added to the
// accumulator tile. The activation tile of each 128-channel step (CT*16 rows x 128
// channels) is staged in double-buffered, padded LDS and read by the four
// wavefronts as B operands, each read feeding RT row tiles. Codes/scales are
// prefetched PW steps ahead; the next step's activation tile is loaded into
// registers before the current step's MFMAs and written to the other LDS buffer
// after them.
constexpr int kXRow = kSuperK + 8;  // halfs per LDS row of the activation tile (16-byte pad)

template <int RT, int GSUB, bool ASYM>
struct GStage {
  uint4 w[RT];
  uint2 sc[RT][GSUB];    // float16 scales of the lane's accumulator rows (C layout) per group
  uint32_t z[RT][GSUB];  // zero point of the lane's A-operand row per group (asymmetric)
};

template <int RT, int CT, int GSUB, bool ASYM, int PW>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(const uint16_t* __restrict__ x, int B,
                                                        const uint4* __restrict__ packed,
                                                        const uint16_t* __restrict__ scales,
                                                        const uint8_t* __restrict__ zeros, int N, int K, int T,
                                                        int S, int Gp, int J, uint16_t* __restrict__ y) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int MPG = 4 / GSUB;
  constexpr int XROWS = CT * 16;
  constexpr int XCH = XROWS * 16 / 256;  // 16-byte chunks of one activation tile per thread
  uint16_t* xbuf = reinterpret_cast<uint16_t*>(smem);  // [2][XROWS][kXRow]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4, arow = lane & 15, crow = 4 * (lane >> 4);
  const int tile0 = blockIdx.x * 4 * RT + wave * RT;
  const int b0 = blockIdx.y * XROWS;

  int tiles[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) tiles[r] = min(tile0 + r, T - 1);

  auto load_w = [&](GStage<RT, GSUB, ASYM>& st, int s) {
    s = min(s, S - 1);  // trailing prefetches re-read the last block: no branch around loads
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const uint4* wp = packed + ((size_t)tiles[r] * S + s) * kWave + lane;
      st.w[r] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wp)));
#pragma unroll
      for (int gs = 0; gs < GSUB; ++gs) {
        const int j = (GSUB == 1) ? s / J : s * GSUB + gs;
        const size_t g0 = ((size_t)tiles[r] * Gp + j) * 16;
        st.sc[r][gs] = *reinterpret_cast<const uint2*>(scales + g0 + crow);
        if (ASYM) st.z[r][gs] = zeros[g0 + arow];
      }
    }
  };
  // this thread's chunks of an activation tile: chunk c = threadIdx.x + 256 * i -> row c / 16, 8 halfs at 8 * (c % 16)
  auto load_x = [&](uint4 (&v)[XCH], int s) {
    s = min(s, S - 1);
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int b = min(b0 + (c >> 4), B - 1);
      const int k = min(s * kSuperK + 8 * (c & 15), K - 8);
      v[i] = *reinterpret_cast<const uint4*>(x + (size_t)b * K + k);
    }
  };
  auto store_x = [&](const uint4 (&v)[XCH], int s, int buf) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int row = c >> 4, col = 8 * (c & 15);
      const bool valid = (b0 + row < B) && (s * kSuperK + col < K);
      *reinterpret_cast<uint4*>(xbuf + (buf * XROWS + row) * kXRow + col) = valid ? v[i] : make_uint4(0u, 0u, 0u, 0u);
    }
  };

  float4_t acc[RT][CT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[r][c] = float4_t{0.f, 0.f, 0.f, 0.f};

  uint4 xv[XCH];
  load_x(xv, 0);
  GStage<RT, GSUB, ASYM> ring[PW];
#pragma unroll
  for (int p = 0; p < PW; ++p) load_w(ring[p], p);
  store_x(xv, 0, 0);
  lds_barrier();

  const DequantRegs dq = DequantRegs::make();

  auto step = [&](GStage<RT, GSUB, ASYM>& st, int s) {
    const int buf = s & 1;
    load_x(xv, s + 1);  // next activation tile: issued before the next codes (in-order completion)
    // this block's codes as float16 integers in MFMA A-operand order, and the scales
    half8_t a[RT][4];
    float4_t sc[RT][GSUB];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
#pragma unroll
      for (int gs = 0; gs < GSUB; ++gs) {
        const _Float16 z = ASYM ? (_Float16)(float)st.z[r][gs] : (_Float16)8.0f;
        const half2_t blo = {(_Float16)-1024.0f - z, (_Float16)-1024.0f - z};
        const half2_t bhi = {(_Float16)-64.0f - z, (_Float16)-64.0f - z};
#pragma unroll
        for (int mm = 0; mm < MPG; ++mm)
          a[r][gs * MPG + mm] = dequant8r(lane_dword(st.w[r], gs * MPG + mm), dq, blo, bhi);
        const half4_t sh = __builtin_bit_cast(half4_t, st.sc[r][gs]);
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[r][gs][i] = (float)sh[i];
      }
    }
    load_w(st, s + PW);  // codes for PW steps ahead into the slot just consumed
    const uint16_t* xb = xbuf + (buf * XROWS + (lane & 15)) * kXRow + 8 * kq;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      half8_t bop[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) bop[m] = *reinterpret_cast<const half8_t*>(xb + c * 16 * kXRow + m * kBlockK);
#pragma unroll
      for (int r = 0; r < RT; ++r) {
#pragma unroll
        for (int gs = 0; gs < GSUB; ++gs) {
          float4_t part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int mm = 0; mm < MPG; ++mm) part = mfma16x16x32(a[r][gs * MPG + mm], bop[gs * MPG + mm], part);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[r][c][i] = __builtin_fmaf(sc[r][gs][i], part[i], acc[r][c][i]);
        }
      }
    }
    store_x(xv, s + 1, buf ^ 1);  // the other buffer was last read in step s-1, before the barrier
    lds_barrier();
  };

  for (int s = 0; s < S; s += PW) {
#pragma unroll
    for (int p = 0; p < PW; ++p)
      if (s + p < S) step(ring[p], s + p);
  }

  // accumulator element i of lane l in tile (r, c): row 16*tile + crow + i, batch row b0 + 16c + l%16
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    if (tile0 + r >= T) continue;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int b = b0 + c * 16 + (lane & 15);
      if (b >= B) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = (tile0 + r) * 16 + crow + i;
        if (n < N) y[(size_t)b * N + n] = __builtin_bit_cast(uint16_t, (_Float16)acc[r][c][i]);
      }
    }
  }
}

template <int RT, int CT, int GSUB, bool ASYM>
hipError_t launch_mfma_t(const GemmArgs& a, hipStream_t stream) {
  constexpr int PW = 3;
  const int T = a.Np / kTileRows;
  const int S = a.Kp / kSuperK;
  const int J = a.group >= kSuperK ? a.group / kSuperK : 1;
  const int col_tiles = (a.B + 15) / 16;
  dim3 grid((T + 4 * RT - 1) / (4 * RT), (col_tiles + CT - 1) / CT);
  const size_t lds = (size_t)2 * CT * 16 * kXRow * 2;
  hipLaunchKernelGGL((gemm_mfma_kernel<RT, CT, GSUB, ASYM, PW>), grid, dim3(256), lds, stream,
                     static_cast<const uint16_t*>(a.x), a.B, static_cast<const uint4*>(a.packed),
                     static_cast<const uint16_t*>(a.scales), static_cast<const uint8_t*>(a.zeros), a.N, a.K, T, S,
                     a.Gp, J, static_cast<uint16_t*>(a.y));
  return hipGetLastError();
}

// Only shapes whose accumulators and per-group partial tiles fit the register file
// (RT * CT * GSUB <= 16) are built; the host never selects the others.
template <int RT, int CT, int GSUB, bool ASYM>
hipError_t launch_mfma_fit(const GemmArgs& a, hipStream_t stream) {
  if constexpr (RT * CT * GSUB <= 16) return launch_mfma_t<RT, CT, GSUB, ASYM>(a, stream);
  return hipErrorInvalidConfiguration;
}

template <int RT, int CT, bool ASYM>
hipError_t launch_mfma_g(const GemmArgs& a, hipStream_t stream) {
  if (a.group == 32) return launch_mfma_fit<RT, CT, 4, ASYM>(a, stream);
  if (a.group == 64) return launch_mfma_fit<RT, CT, 2, ASYM>(a, stream);
  return launch_mfma_fit<RT, CT, 1, ASYM>(a, stream);
}

template <int RT, int CT>
hipError_t launch_mfma_a(const GemmArgs& a, hipStream_t stream) {
  return a.asym ? launch_mfma_g<RT, CT, true>(a, stream) : launch_mfma_g<RT, CT, false>(a, stream);
}

template <int CT>
hipError_t launch_mfma_r(const GemmArgs& a, hipStream_t stream) {
  if (a.rows_per_wave == 1) return launch_mfma_a<1, CT>(a, stream);
  if (a.rows_per_wave == 2) return launch_mfma_a<2, CT>(a, stream);
  return launch_mfma_a<4, CT>(a, stream);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.B <= 16) return launch_gemv(a, stream);
  switch (a.col_tiles) {
    case 2: return launch_mfma_r<2>(a, stream);
    case 4: return launch_mfma_r<4>(a, stream);
    default: return launch_mfma_r<8>(a, stream);
  }
}

}  // namespace q4
