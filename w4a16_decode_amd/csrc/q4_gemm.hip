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
//    take units of (row tiles x a chunk of the channel range, usually 1024
//    channels) and their partial sums are
//    reduced through LDS in a fixed order (deterministic). Larger B runs the skinny
//    GEMM: 2 to 8 column tiles of 16 batch rows per workgroup, staged through LDS
//    and shared by its 8 (or 4) wavefronts, each owning whole row tiles.
#include <algorithm>

#include <map>
#include <mutex>

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
// The grid is sized to what the GPU holds at once (normally one workgroup of 16
// wavefronts per CU). Workgroup g owns k-split ks = g % KS of the channel range and
// the row blocks (R tiles of 16 rows) g/KS, g/KS + G/KS, ... Its work is cut into
// units: one row block times one of CH chunks of the k-split's 128-channel blocks,
// chunk c holding blocks c, c + CH, c + 2 CH, ... of the split, so the wavefronts on
// the chunks of a row block read neighbouring kilobytes at the same time (contiguous
// chunks, which put them 8 KiB apart, measured 0.3-1.2 us slower per launch).
// Wavefronts take units from a counter in LDS as they go, so a wavefront that the
// SIMD serves faster simply takes more units and all of them finish together (the
// sequencer favours older wavefronts; a static split leaves the youngest ones
// streaming alone at the end). Each wavefront streams the blocks of codes and
// scales of its units through a ring of P stages (vector loads retire in order, so
// only weights ride that pipeline): INT4 codes with one row tile per wavefront fill
// the ring in bursts of P/2 blocks of the unit, one half loading while the other
// is computed (back-to-back loads stream faster than the same loads spread out),
// the other kinds keep a rolling window of P-1 blocks in flight. Activation operands are read from LDS: the
// workgroup copies its slice of x (all B rows) into LDS once. The units a
// wavefront starts with are fixed (wave, wave + W, ...: as many as its first loads
// can reach, normally one) and only later ones come from the counter, so every
// wavefront starts streaming as soon as it runs instead of waiting at a barrier for
// the workgroup's last wavefront to start; the counter is initialised before the
// barrier that publishes x and used only after it. A finished unit's partial sums
// (the B real columns only) are parked
// in LDS under the unit's index; after one barrier at the end they are added over
// the chunks in chunk order, so the result does not depend on which wavefront ran
// which unit. With KS > 1 the workgroups write float32 partials to the workspace
// and reduce_splits_kernel adds them in a fixed order.
template <int R, int GSUB, bool ASYM, int NW = 1>
struct WStage {
  uint4 w[R][NW];  // NW 16-byte pieces of codes per lane and block (1: INT4, 2: INT8)
  uint2 sc[R][GSUB];
  uint32_t z[R][GSUB];
  int s;     // block index (uniform)
  int unit;  // unit index, or -1 once the wavefront has no more work (uniform)
  bool last; // last block of its unit (uniform)
};


// LDS layout of one GEMV workgroup, in bytes (shared with the host-side sizing).
struct GemvLds {
  size_t x, beta, part, total;
  __host__ __device__ GemvLds(int B, int nsb, int GSUB, bool bias, int R, int units) {
    x = ((((size_t)B * (nsb * kSuperK + kGemmRowPad) + kSuperK) * 2) + 15) & ~(size_t)15;  // x rows + zero row
    beta = bias ? (((size_t)B * nsb * GSUB + 1 + 3) / 4 * 4) * 4 : 0;            // per-unit biases + a zero
    part = (size_t)units * R * 16 * B * 4;  // partial sums of every unit
    total = x + beta + part + 16;           // + the unit counter
  }
};

// Wavefronts per workgroup the kernel is built for: 16 (one workgroup per CU,
// 128 VGPRs) for one group per block and R <= 2 (R = 1 for INT8 codes), else 8
// (256 VGPRs) so that the extra scales, row tiles or code pieces stay in registers.
template <int R, int GSUB, bool Q8 = false>
constexpr int gemv_max_waves() { return (GSUB > 1 || R > 2 || (Q8 && R > 1)) ? 8 : 16; }

// Eight INT8 codes of the W8A16 layout (two dwords, four offset-binary bytes
// b = q + 128 each, channel order) -> the float16 operand 1024 + b = 1152 + q:
// v_perm_b32 interleaves the code bytes with the exponent byte 0x64 (1024.0h),
// one instruction per pair. The GEMV subtracts 1152 * sum(x) per block.
__device__ __forceinline__ half8_t magic8_i8(uint32_t d0, uint32_t d1) {
  constexpr uint32_t kExp = 0x64646464u;
  const uint32_t p0 = __builtin_amdgcn_perm(kExp, d0, 0x04010400u);
  const uint32_t p1 = __builtin_amdgcn_perm(kExp, d0, 0x04030402u);
  const uint32_t p2 = __builtin_amdgcn_perm(kExp, d1, 0x04010400u);
  const uint32_t p3 = __builtin_amdgcn_perm(kExp, d1, 0x04030402u);
  return __builtin_bit_cast(half8_t, make_uint4(p0, p1, p2, p3));
}

// Step 1 of the staged GEMVs: the workgroup's x slice (all B rows of the k-split's
// channels from block wsb0 on) -> registers, XCH chunks of 16 bytes per thread, the
// fewest that cover it (indices clamped into x, so every thread issues the same
// number of loads and the later wait is exact).
template <int XCH>
__device__ __forceinline__ void gemv_load_x(uint4 (&xr)[XCH], const uint16_t* __restrict__ x, int B, int K, int wsb0,
                                            int row_chunks) {
  const int xchunks = B * row_chunks;
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int idx = min((int)threadIdx.x + i * (int)blockDim.x, xchunks - 1);
    const int b = idx / row_chunks;
    const int k = min(wsb0 * kSuperK + (idx - b * row_chunks) * 8, K - 8);
    xr[i] = *reinterpret_cast<const uint4*>(x + (size_t)b * K + k);
  }
}

// Step 3 of the staged GEMVs: the x slice -> LDS (x rows of xstride = row_chunks * 8
// + kGemmRowPad halfs; elements 2, 3, 6, 7 of every 8 divided by 16 when BIAS and
// the codes are INT4: exact powers of two; channels past K are zero), plus the zero
// row. With BIAS the per-unit bias 1032 * (sum of plain elements) + 1152 * (sum of
// scaled elements) (INT8 codes: 1152 * sum(x)) is reduced on the way into beta: the
// UNIT / 8 chunks of a bias unit sit in consecutive lanes (row_chunks is a multiple
// of 16 and the block a multiple of 64 threads).
template <int XCH, bool BIAS, bool Q8, int UNIT>
__device__ __forceinline__ void gemv_store_x(const uint4 (&xr)[XCH], uint16_t* xl, uint16_t* xzero, float* beta, int B,
                                             int K, int wsb0, int row_chunks, int nunits) {
  constexpr int CPU = UNIT / 8;  // chunks per bias unit
  const int xchunks = B * row_chunks;
  const int xstride = row_chunks * 8 + kGemmRowPad;
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int idx = threadIdx.x + i * blockDim.x;
    if (i * (int)blockDim.x >= xchunks) break;  // uniform: no chunk of this round is real
    const bool real = idx < xchunks;
    const int b = idx / row_chunks;
    const int c8 = idx - b * row_chunks;
    uint4 v = (real && wsb0 * kSuperK + c8 * 8 < K) ? xr[i] : make_uint4(0u, 0u, 0u, 0u);
    if (BIAS) {
      // INT8 codes keep x as it is: bias 1152 * sum(x) (magic8_i8)
      half8_t h = as_half8(v);
      if (!Q8) {
        h[2] *= (_Float16)0.0625f;
        h[3] *= (_Float16)0.0625f;
        h[6] *= (_Float16)0.0625f;
        h[7] *= (_Float16)0.0625f;
        v = __builtin_bit_cast(uint4, h);
      }
      float plain = ((float)h[0] + (float)h[1]) + ((float)h[4] + (float)h[5]);
      float scaled = ((float)h[2] + (float)h[3]) + ((float)h[6] + (float)h[7]);
#pragma unroll
      for (int m = 1; m < CPU; m <<= 1) {
        plain += __shfl_xor(plain, m);
        scaled += __shfl_xor(scaled, m);
      }
      // one explicit fma: the same rounding in every kernel this is inlined into
      if (real && c8 % CPU == 0)
        beta[b * nunits + c8 / CPU] = Q8 ? 1152.f * (plain + scaled) : __builtin_fmaf(1032.f, plain, 1152.f * scaled);
    }
    if (real) *reinterpret_cast<uint4*>(xl + b * xstride + c8 * 8) = v;
  }
  if (threadIdx.x < kSuperK / 8) *reinterpret_cast<uint4*>(xzero + threadIdx.x * 8) = make_uint4(0u, 0u, 0u, 0u);
  if (BIAS && threadIdx.x == 0) beta[B * nunits] = 0.f;
}

// Step 4 of the staged GEMVs (after the barrier that ends the streaming): the units'
// partial sums, parked in LDS as [unit = i * CH + c][r][b][16 rows], added in chunk
// order for every row block i of the workgroup -> y, or with KS > 1 -> the k-split's
// float32 slice of the workspace; e = ((i * R + r) * B + b) * 16 + row.
template <int R>
__device__ __forceinline__ void gemv_write_units(const float* part0, int n_rb, int CH, int B, int N, int rb_first,
                                                 int rb_stride, int KS, int ks, uint16_t* __restrict__ y,
                                                 float* __restrict__ ws) {
  const int nout = n_rb * R * 16 * B;
  for (int e = threadIdx.x; e < nout; e += blockDim.x) {
    const int row = e & 15;
    const int t = e >> 4;
    const int b = t % B;
    const int ir = t / B;  // i * R + r
    const int i = ir / R, r = ir - i * R;
    const float* pp = part0 + ((size_t)i * CH * R + r) * 16 * B + b * 16 + row;
    float sum = 0.f;
    for (int c = 0; c < CH; ++c) sum += pp[(size_t)c * R * 16 * B];
    const int n = ((rb_first + i * rb_stride) * R + r) * 16 + row;
    if (n < N) {
      if (KS == 1) y[(size_t)b * N + n] = __builtin_bit_cast(uint16_t, (_Float16)sum);
      else ws[((size_t)ks * B + b) * N + n] = sum;
    }
  }
}

// Q8: W8A16 codes (per-row INT8 scale passed as one group spanning the row, J = S,
// Gp = 1): a 16-row x 128-channel block is 2 KiB, two 1 KiB halves of 64 channels;
// lane l's 16 bytes of half h hold row l%16, channels 64h + 32j + 8(l/16) + e at
// byte 8j + e (j = 0, 1; e = 0..7), so each half feeds two MFMA steps.
template <int R, int GSUB, bool ASYM, int P, int XCH, bool Q8 = false>
__global__ __launch_bounds__((gemv_max_waves<R, GSUB, Q8>() * 64))
void gemv_kernel(const uint16_t* __restrict__ x, int B, const uint4* __restrict__ packed,
                 const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int N, int K, int T,
                 int S, int Gp, int J, int KS, int nRB, int CH, uint16_t* __restrict__ y,
                 float* __restrict__ ws) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int MPG = 4 / GSUB;
  // Symmetric codes skip the per-pair bias removal (magic8r) and subtract a
  // per-unit bias from the float32 partial instead; a bias unit is the channel run
  // one partial covers (128 / GSUB).
  constexpr bool BIAS = !ASYM;
  constexpr int UNIT = kSuperK / GSUB;
  constexpr int NW = Q8 ? 2 : 1;        // 16-byte code pieces per lane and block
  constexpr size_t BLK = 1024 * NW;     // bytes of one 16 x 128 block
  static_assert(!Q8 || (GSUB == 1 && !ASYM), "INT8 codes are symmetric with one scale per row");
  const int W = blockDim.x >> 6;
  // readfirstlane: the wavefront index is uniform, and saying so keeps every value
  // derived from it in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ks = blockIdx.x % KS;
  const int rb_first = blockIdx.x / KS;
  const int rb_stride = gridDim.x / KS;
  const int wsb0 = (int)(((int64_t)S * ks) / KS);
  const int wsb1 = (int)(((int64_t)S * (ks + 1)) / KS);
  const int nsb = wsb1 - wsb0;  // >= CH: the host keeps every chunk at least one block long
  const int n_rb = rb_first < nRB ? (nRB - 1 - rb_first) / rb_stride + 1 : 0;
  const int n_units = n_rb * CH;
  const int KR = nsb * kSuperK;
  const int xstride = KR + kGemmRowPad;  // halfs per x row in LDS (32-byte pad: conflict-free operand reads)
  const int nunits = nsb * GSUB;
  const GemvLds lay(B, nsb, GSUB, BIAS, R, n_units);
  uint16_t* xl = reinterpret_cast<uint16_t*>(smem);      // x (x/16 at the scaled elements when BIAS)
  uint16_t* xzero = xl + B * xstride;                     // 128 zero halfs for absent batch rows
  float* beta = reinterpret_cast<float*>(smem + lay.x);
  float* part0 = reinterpret_cast<float*>(smem + lay.x + lay.beta);  // [unit][r][b][16 rows]
  int* counter = reinterpret_cast<int*>(smem + lay.x + lay.beta + lay.part);
  const int crow = 4 * (lane >> 4);
  const int arow = lane & 15;
  const int bcol = lane & 15;

  // 1. the workgroup's x slice -> registers
  const int row_chunks = KR >> 3;
  uint4 xr[XCH];
  gemv_load_x(xr, x, B, K, wsb0, row_chunks);
  // 2. the first L blocks of codes / scales (P/2 in the burst ring, else P-1).
  //    Those loads end at most L / (shortest unit) units, so the first KST grabs of
  //    each wavefront, which cover them, take units wave + j * W (j < KST) without
  //    the counter; the counter serves the rest (units from KST * W on) and is used
  //    only after the barrier that follows the x staging. Block addresses are
  //    wave-uniform (tile base + 1 KiB per block); only the lane offsets live in
  //    VGPRs. Loads are unconditional: once the units run out the last block is
  //    loaded again, which keeps the loop free of branches around loads.
  constexpr bool BURST = R == 1 && !Q8;  // ring filled in two halves of H blocks
  constexpr int H = P / 2;
  static_assert(!BURST || P % 2 == 0, "the burst ring has two equal halves");
  constexpr int L = BURST ? H : P - 1;
  const int KST = 1 + L / (nsb / CH);  // nsb >= CH: every chunk is at least one block
  if (threadIdx.x == 0) *counter = KST * W * 64;
  const unsigned char* pk = reinterpret_cast<const unsigned char*>(packed);
  const uint32_t w_lane = (uint32_t)lane * 16u;
  const uint32_t s_lane = (uint32_t)crow * 2u;
  int l_unit = 0, l_s = 0, l_j = 0;
  const unsigned char* l_wt[R];
  const unsigned char* l_st[R];
  int grabs = 0;  // grabs made by this wavefront (uniform)
  auto grab = [&]() __attribute__((always_inline)) {
    // the first KST grabs take units wave + j * W; later ones the counter, where
    // every lane adds 1 (called with all lanes active), so a grab moves it by 64 and
    // each lane sees a value in [64u, 64u + 63]
    const int u = grabs < KST ? wave + grabs * W : __builtin_amdgcn_readfirstlane(atomicAdd(counter, 1)) >> 6;
    ++grabs;
    if (u >= n_units) {
      l_unit = -1;  // the address registers keep the last unit (loads clamp the block)
      return;
    }
    l_unit = u;
    const int i = u / CH, c = u - i * CH;
    l_s = wsb0 + c;  // blocks wsb0 + c, + CH, + 2 CH, ... below wsb1 (CH <= nsb)
    l_j = (GSUB == 1) ? l_s / J : l_s * GSUB;
    const int rb = rb_first + i * rb_stride;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const size_t tile = (size_t)min(rb * R + r, T - 1);
      l_wt[r] = pk + tile * S * BLK;
      l_st[r] = reinterpret_cast<const unsigned char*>(scales) + tile * Gp * 32;
    }
  };
  grab();
  if (l_unit < 0) {  // no work for this wavefront: point the (unused) loads at tile 0
    l_s = wsb0;
    l_j = (GSUB == 1) ? wsb0 / J : wsb0 * GSUB;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      l_wt[r] = pk;
      l_st[r] = reinterpret_cast<const unsigned char*>(scales);
    }
  }
  auto load = [&](WStage<R, GSUB, ASYM, NW>& st) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const unsigned char* wp = l_wt[r] + (size_t)min(l_s, S - 1) * BLK + w_lane;
#pragma unroll
      for (int h = 0; h < NW; ++h)
        st.w[r][h] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wp + 1024 * h)));
#pragma unroll
      for (int gs = 0; gs < GSUB; ++gs) {
        const size_t goff = (size_t)(l_j + gs) * 32;
        st.sc[r][gs] = *reinterpret_cast<const uint2*>(l_st[r] + goff + s_lane);
        if (ASYM) st.z[r][gs] = zeros[(size_t)((l_st[r] - reinterpret_cast<const unsigned char*>(scales)) >> 1) +
                                      (goff >> 1) + arow];
      }
    }
    st.s = min(l_s, wsb1 - 1);
    st.unit = l_unit;
    st.last = l_s + CH >= wsb1;
    if (l_unit < 0) return;
    l_s += CH;
    if (l_s >= wsb1) {
      grab();
      return;
    }
    l_j = (GSUB == 1) ? (J == 1 ? l_s : l_s / J) : l_s * GSUB;
  };
  WStage<R, GSUB, ASYM, NW> buf[P];
#pragma unroll
  for (int p = 0; p < L; ++p) load(buf[p]);

  // 3. x slice -> LDS, plus the zero row (and, with BIAS, the per-unit biases)
  gemv_store_x<XCH, BIAS, Q8, UNIT>(xr, xl, xzero, beta, B, K, wsb0, row_chunks, nunits);
  lds_barrier();

  float4_t acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = float4_t{0.f, 0.f, 0.f, 0.f};
  const DequantRegs dq = DequantRegs::make();
  // LDS read pointers of this lane's activation operand and bias; lanes of absent
  // batch rows stay on the zero row / zero bias
  const bool real_col = bcol < B;
  const uint16_t* xlane0 = real_col ? xl + bcol * xstride + 8 * (lane >> 4) : xzero + 8 * (lane >> 4);
  const int xstep = real_col ? kSuperK : 0;
  const float* blane0 = real_col ? beta + bcol * nunits : beta + B * nunits;
  const int bstep = real_col ? GSUB : 0;

  // activation operands (and biases) of the next block to compute, read from LDS
  // one block ahead so the LDS latency hides behind the current block's work
  half8_t xb[4];
  float bu[GSUB];
  auto read_x = [&](int s) __attribute__((always_inline)) {
    const uint16_t* xp = xlane0 + (s - wsb0) * xstep;
#pragma unroll
    for (int m = 0; m < 4; ++m) xb[m] = *reinterpret_cast<const half8_t*>(xp + m * kBlockK);
    if (BIAS) {
      const float* bp = blane0 + (s - wsb0) * bstep;
#pragma unroll
      for (int gs = 0; gs < GSUB; ++gs) bu[gs] = bp[gs];
    }
  };
  read_x(buf[0].s);

  auto compute = [&](const WStage<R, GSUB, ASYM, NW>& st, int s_next) __attribute__((always_inline)) {
    half8_t xc[4];
    float bc[GSUB];
#pragma unroll
    for (int m = 0; m < 4; ++m) xc[m] = xb[m];
#pragma unroll
    for (int gs = 0; gs < GSUB; ++gs) bc[gs] = BIAS ? bu[gs] : 0.f;
    read_x(s_next);
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int gs = 0; gs < GSUB; ++gs) {
        const half4_t sh = __builtin_bit_cast(half4_t, st.sc[r][gs]);
        float4_t part = {0.f, 0.f, 0.f, 0.f};
        if (Q8) {
#pragma unroll
          for (int mm = 0; mm < 4; ++mm) {
            const uint4& v = st.w[r][mm >> 1];
            part = mfma16x16x32(magic8_i8(lane_dword(v, 2 * (mm & 1)), lane_dword(v, 2 * (mm & 1) + 1)), xc[mm], part);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[r][i] = __builtin_fmaf((float)sh[i], part[i] - bc[gs], acc[r][i]);
        } else if (BIAS) {
#pragma unroll
          for (int mm = 0; mm < MPG; ++mm)
            part = mfma16x16x32(magic8r(lane_dword(st.w[r][0], gs * MPG + mm), dq), xc[gs * MPG + mm], part);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[r][i] = __builtin_fmaf((float)sh[i], part[i] - bc[gs], acc[r][i]);
        } else {
          const _Float16 z = (_Float16)(float)st.z[r][gs];
          const half2_t blo = {(_Float16)-1024.0f - z, (_Float16)-1024.0f - z};
          const half2_t bhi = {(_Float16)-64.0f - z, (_Float16)-64.0f - z};
#pragma unroll
          for (int mm = 0; mm < MPG; ++mm)
            part = mfma16x16x32(dequant8r(lane_dword(st.w[r][0], gs * MPG + mm), dq, blo, bhi), xc[gs * MPG + mm], part);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[r][i] = __builtin_fmaf((float)sh[i], part[i], acc[r][i]);
        }
      }
    }
    if (!st.last) return;
    // unit finished: park the partial sums of the real batch columns (the lane
    // holds rows crow..crow+3 of column bcol) and start the next unit from zero
    if (real_col) {
      float* pp = part0 + (size_t)st.unit * R * 16 * B + bcol * 16 + crow;
#pragma unroll
      for (int r = 0; r < R; ++r) *reinterpret_cast<float4_t*>(pp + r * 16 * B) = acc[r];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = float4_t{0.f, 0.f, 0.f, 0.f};
  };

  // once a stage has no unit, every later one has none either
  if constexpr (BURST) {
    while (buf[0].unit >= 0) {
#pragma unroll
      for (int p = H; p < P; ++p) load(buf[p]);
#pragma unroll
      for (int p = 0; p < H; ++p)
        if (buf[p].unit >= 0) compute(buf[p], buf[p + 1].s);
#pragma unroll
      for (int p = 0; p < H; ++p) load(buf[p]);
#pragma unroll
      for (int p = H; p < P; ++p)
        if (buf[p].unit >= 0) compute(buf[p], buf[(p + 1) % P].s);
    }
  } else {
    while (buf[0].unit >= 0) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        load(buf[(p + P - 1) % P]);
        if (buf[p].unit >= 0) compute(buf[p], buf[(p + 1) % P].s);
      }
    }
  }

  // 4. results of all row blocks -> y (or the k-split workspace)
  lds_barrier();
  gemv_write_units<R>(part0, n_rb, CH, B, N, rb_first, rb_stride, KS, ks, y, ws);
}

// ---------------------------------------------------------------------------------
// GEMV for the common case of the staged kernel: symmetric INT4 codes with one scale
// per 1 KiB block (groups of 128 channels), one row tile per wavefront, and chunks of
// a whole number of NB-block bursts (the host checks S % KS == 0 and
// (S / KS) % (NB CH) == 0). It runs gemv_kernel<1, 1, false, 8, XCH>'s grid, units,
// x staging, arithmetic and final reduction (its burst ring has two halves of NB
// blocks: 4 as gemv_kernel's, or 2, which the host takes for rows of >= 8192
// channels), so for the same CH the two give identical bits whatever NB (the blocks of
// a unit are summed in the same order); what differs is the instruction stream
// around the loads. gemv_kernel re-derives every block's code and scale addresses from a block
// index, with clamps, a group division and a unit test per block (~40 scalar
// instructions and several branches per 1 KiB block). Here a unit's code and scale
// bases are formed once when the unit is taken, a burst is NB loads from one scalar
// base plus per-lane offsets held in registers (block q of a burst sits q * CH KiB
// further), and the unit counter is read once per unit.
template <int XCH, int NB, bool Q8 = false>  // NB: blocks per burst (2 or 4); Q8: INT8 codes
__global__ __launch_bounds__(16 * 64)
void gemv_burst_kernel(const uint16_t* __restrict__ x, int B, const uint4* __restrict__ packed,
                       const uint16_t* __restrict__ scales, int N, int K, int S, int Gp, int KS, int nRB, int CH,
                       uint16_t* __restrict__ y, float* __restrict__ ws) {
  static_assert(NB == 2 || NB == 4, "bursts of 2 or 4 blocks");
  extern __shared__ __align__(16) unsigned char smem[];
  // INT8 codes (W8A16): 2 KiB blocks of two 16-byte pieces per lane, one scale per row
  constexpr int NW = Q8 ? 2 : 1;
  constexpr uint32_t BLKB = 1024u * NW;
  const int W = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ks = blockIdx.x % KS;
  const int rb_first = blockIdx.x / KS;
  const int rb_stride = gridDim.x / KS;
  const int nsb = S / KS;  // blocks per split: a multiple of NB * CH
  const int wsb0 = nsb * ks;
  const int bursts = nsb / (NB * CH);  // bursts per unit
  const int n_rb = rb_first < nRB ? (nRB - 1 - rb_first) / rb_stride + 1 : 0;
  const int n_units = n_rb * CH;
  const int KR = nsb * kSuperK;
  const int xstride = KR + kGemmRowPad;
  const GemvLds lay(B, nsb, 1, true, 1, n_units);
  uint16_t* xl = reinterpret_cast<uint16_t*>(smem);
  uint16_t* xzero = xl + B * xstride;
  float* beta = reinterpret_cast<float*>(smem + lay.x);
  float* part0 = reinterpret_cast<float*>(smem + lay.x + lay.beta);  // [unit][b][16 rows]
  int* counter = reinterpret_cast<int*>(smem + lay.x + lay.beta + lay.part);
  const int crow = 4 * (lane >> 4);
  const int bcol = lane & 15;

  // 1. the workgroup's x slice -> registers
  const int row_chunks = KR >> 3;
  uint4 xr[XCH];
  gemv_load_x(xr, x, B, K, wsb0, row_chunks);

  // The wavefront's cursor (all uniform): the unit it streams (-1 once the units
  // have run out), that unit's chunk, its code and scale bases (block wsb0 + c of
  // its tile) and the next burst to load. Block q of burst j of a unit sits
  // (j * NB + q) * CH blocks past the unit's base: the lane offsets of the NB blocks
  // of a burst are fixed registers, the burst's scalar base moves by NB * CH blocks.
  const unsigned char* pk = reinterpret_cast<const unsigned char*>(packed);
  const unsigned char* sk = reinterpret_cast<const unsigned char*>(scales);
  const uint32_t cstride = (uint32_t)CH * BLKB;        // bytes between a unit's blocks (codes)
  const uint32_t sstride = Q8 ? 0u : (uint32_t)CH * 32u;  // ... (scales: 16 float16 per block; per row for INT8)
  uint32_t woff[NB], soff[NB], lw[NB], ls[NB];  // lw, ls: the offsets loads use now
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    woff[q] = (uint32_t)lane * 16u + q * cstride;
    soff[q] = (uint32_t)crow * 2u + q * sstride;
    lw[q] = woff[q];
    ls[q] = soff[q];
  }
  int c_unit = -1, c_chunk = 0, c_burst = 0;
  const unsigned char* c_w = pk;
  const unsigned char* c_s = sk;
  // Units: the first KST of each wavefront are fixed (wave, wave + W): they cover
  // the burst issued before the barrier that publishes x (with one-burst units that
  // burst ends the first unit and takes the second). Later units come from the
  // counter (every lane adds 1, so a grab moves it by 64), which thread 0 sets
  // before that barrier and nobody touches until after it.
  const int KST = bursts == 1 ? 2 : 1;
  int grabs = 0;
  auto take = [&]() __attribute__((always_inline)) {
    const int u = grabs < KST ? wave + grabs * W : __builtin_amdgcn_readfirstlane(atomicAdd(counter, 1)) >> 6;
    ++grabs;
    c_burst = 0;
    if ((unsigned)u >= (unsigned)n_units) {
      // no more units: the loads that still follow (unconditional, so the compiler
      // keeps exact vmcnt counts) all re-read the block this wavefront loaded last,
      // which the L2 still holds or is fetching. Re-reading the last unit's first
      // burst, loaded long before, fetched 4 KiB more per wavefront from HBM (+6%
      // bytes on gate/up); its last whole burst still +4% (+17% on q/k/v); one burst
      // shared by all such wavefronts cost ~0.8 us on the small matrices.
      c_unit = -1;
      c_burst = bursts - 1;
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        lw[q] = woff[NB - 1];
        ls[q] = soff[NB - 1];
      }
      return;
    }
    c_unit = u;
    const int i = u / CH;
    c_chunk = u - i * CH;
    const size_t tile = (size_t)(rb_first + i * rb_stride);
    c_w = pk + (tile * S + wsb0 + c_chunk) * BLKB;
    c_s = sk + (tile * Gp + (Q8 ? 0 : wsb0 + c_chunk)) * 32;
  };
  if (threadIdx.x == 0) *counter = KST * W * 64;
  take();

  // one burst in flight: codes and scales of NB blocks, the unit and chunk they
  // belong to, the index of the burst's first block in the unit and whether it ends it
  struct Burst {
    uint4 w[NB][NW];
    uint2 sc[NB];
    int unit, chunk, j0;
    bool last;
  };
  auto issue = [&](Burst& b) __attribute__((always_inline)) {
    const size_t boff = (size_t)c_burst * NB * CH;
    const unsigned char* wb = c_w + boff * BLKB;
    const unsigned char* sb = c_s + (Q8 ? 0 : boff * 32);
    // codes and scale of one block after the other: loads complete in order, so
    // block q waits for the first 2 (q + 1) loads of the burst only
#pragma unroll
    for (int q = 0; q < NB; ++q) {
#pragma unroll
      for (int h = 0; h < NW; ++h)
        b.w[q][h] = __builtin_bit_cast(
            uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wb + lw[q] + 1024u * h)));
      b.sc[q] = *reinterpret_cast<const uint2*>(sb + ls[q]);
    }
    b.unit = c_unit;
    b.chunk = c_chunk;
    b.j0 = c_burst * NB;
    b.last = c_burst + 1 == bursts;
    if (c_unit < 0) return;
    if (++c_burst == bursts) take();
  };
  Burst ring[2];
  issue(ring[0]);

  // 3. x slice -> LDS, plus the zero row and the per-unit biases
  const int nunits = nsb;
  gemv_store_x<XCH, true, Q8, kSuperK>(xr, xl, xzero, beta, B, K, wsb0, row_chunks, nunits);
  lds_barrier();

  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  const DequantRegs dq = DequantRegs::make();
  // LDS read pointers of this lane's activation operand and bias; lanes of absent
  // batch rows stay on the zero row / zero bias (steps of 0)
  const bool real_col = bcol < B;
  const uint16_t* xlane0 = real_col ? xl + bcol * xstride + 8 * (lane >> 4) : xzero + 8 * (lane >> 4);
  const float* blane0 = real_col ? beta + bcol * nunits : beta + B * nunits;
  // activation operands and bias of the next block to compute, read from LDS one
  // block ahead; block index sb = s - wsb0 = chunk + j * CH (uniform: the lane's
  // offset is a select, not a multiply)
  half8_t xb[4];
  float bu;
  auto read_x = [&](int sb) __attribute__((always_inline)) {
    const uint16_t* xp = xlane0 + (real_col ? sb * kSuperK : 0);
#pragma unroll
    for (int m = 0; m < 4; ++m) xb[m] = *reinterpret_cast<const half8_t*>(xp + m * kBlockK);
    bu = blane0[real_col ? sb : 0];
  };
  auto block_of = [&](const Burst& b, int q) __attribute__((always_inline)) {
    return b.unit < 0 ? 0 : b.chunk + (b.j0 + q) * CH;
  };
  read_x(block_of(ring[0], 0));

  // the NB blocks of burst b, each: 4 MFMA steps over the raw magic-number operands,
  // bias removed and the group's scale applied in float32; nx is the burst after it
  // (whose first block's x is read ahead during b's last block)
  auto compute = [&](const Burst& b, const Burst& nx) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      half8_t xc[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) xc[m] = xb[m];
      const float bc = bu;
      read_x(q + 1 < NB ? block_of(b, q + 1) : block_of(nx, 0));
      const half4_t sh = __builtin_bit_cast(half4_t, b.sc[q]);
      float4_t part = {0.f, 0.f, 0.f, 0.f};
      if constexpr (Q8) {
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          const uint4& v = b.w[q][mm >> 1];
          part = mfma16x16x32(magic8_i8(lane_dword(v, 2 * (mm & 1)), lane_dword(v, 2 * (mm & 1) + 1)), xc[mm], part);
        }
      } else {
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) part = mfma16x16x32(magic8r(lane_dword(b.w[q][0], mm), dq), xc[mm], part);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf((float)sh[i], part[i] - bc, acc[i]);
    }
    if (!b.last) return;
    // unit finished: park the partial sums of the real batch columns (the lane
    // holds rows crow..crow+3 of column bcol) and start the next unit from zero
    if (real_col) *reinterpret_cast<float4_t*>(part0 + (size_t)b.unit * 16 * B + bcol * 16 + crow) = acc;
    acc = float4_t{0.f, 0.f, 0.f, 0.f};
  };

  // once a burst has no unit, every later one has none either
  while (ring[0].unit >= 0) {
    issue(ring[1]);
    compute(ring[0], ring[1]);
    issue(ring[0]);
    if (ring[1].unit < 0) break;
    compute(ring[1], ring[0]);
  }

  // 4. results of all row blocks -> y (or the k-split workspace)
  lds_barrier();
  gemv_write_units<1>(part0, n_rb, CH, B, N, rb_first, rb_stride, KS, ks, y, ws);
}

__global__ void reduce_splits_kernel(const float* __restrict__ ws, int KS, int64_t BN, uint16_t* __restrict__ y) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < BN; i += (int64_t)gridDim.x * blockDim.x) {
    float sum = 0.f;
    for (int k = 0; k < KS; ++k) sum += ws[(size_t)k * BN + i];
    y[i] = __builtin_bit_cast(uint16_t, (_Float16)sum);
  }
}

// The same sums, 8 outputs per thread: two 16-byte loads per split and one 16-byte
// store, so each thread keeps 32 bytes per split in flight instead of 4. Needs
// BN % 8 == 0 (every split then starts 32-byte aligned in the 16-byte aligned
// workspace) and a 16-byte aligned y; each output adds its splits in the same
// order as reduce_splits_kernel, so the two give identical bits.
__global__ void reduce_splits8_kernel(const float* __restrict__ ws, int KS, int64_t BN, uint16_t* __restrict__ y) {
  const int64_t n8 = BN >> 3;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    float4_t lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int k = 0; k < KS; ++k) {
      const float4_t* p = reinterpret_cast<const float4_t*>(ws + (size_t)k * BN) + 2 * i;
      const float4_t a = p[0], b = p[1];
      lo += a;
      hi += b;
    }
    half8_t h;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = (_Float16)lo[e];
      h[4 + e] = (_Float16)hi[e];
    }
    *reinterpret_cast<uint4*>(y + 8 * i) = __builtin_bit_cast(uint4, h);
  }
}

// Adds the KS float32 partial products in the workspace, split by split, into y.
void launch_reduce_splits(const float* ws, int KS, int64_t BN, uint16_t* y, hipStream_t stream) {
  const bool vec = BN % 8 == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0;
  const int64_t work = vec ? BN / 8 : BN;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (vec)
    hipLaunchKernelGGL(reduce_splits8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ws, KS, BN, y);
  else
    hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ws, KS, BN, y);
}

// ---------------------------------------------------------------------------------
// GEMV for B <= 3 with the activation streamed per unit (at B = 4 the per-unit
// activation loads, half the bytes of the unit's codes, cost more than staging).
//
// Same units, counter, partial sums and final reduction as gemv_kernel, but no
// workgroup-wide copy of x: a unit is always 8 blocks (1024 channels: blocks c,
// c + CH, ..., c + 7 CH of the row, strided like the staged GEMV's chunks, which
// measured 0.3-0.7 us faster per launch on down and o than 8 consecutive blocks), and
// the wavefront that takes a unit loads that unit's 1024 activations itself, in
// the same in-order stream as the unit's codes (2 loads of 16 bytes per lane,
// issued right before the unit's first codes). When it finishes its
// previous unit it writes them (and the per-block biases of symmetric codes) into
// its own slice of LDS, from which the MFMA operands are read as in gemv_kernel.
// The kernel therefore starts streaming codes at once instead of first staging the
// whole activation slice, and x is read from L2 in small pieces spread over the
// kernel. Units are at least P - 1 blocks long, so a wavefront never has the x of
// more than one unit waiting in registers.
constexpr int kUnitBlocks = kStreamUnitBlocks;
constexpr int kUnitXStride = kUnitBlocks * kSuperK + kGemmRowPad;  // halfs per batch row of a unit's x in LDS

// LDS of one streaming workgroup, in bytes (shared with the host-side sizing).
struct GemvStreamLds {
  size_t xw, bw, zero, part, total;
  __host__ __device__ GemvStreamLds(int BMAX, int GSUB, bool bias, int W, int R, int B, int units) {
    xw = (size_t)W * BMAX * kUnitXStride * 2;                   // per-wavefront x of its unit
    bw = bias ? (size_t)W * BMAX * kUnitBlocks * GSUB * 4 : 0;  // per-wavefront biases of its unit
    zero = kSuperK * 2 + 16;                                    // zero row + zero bias
    part = (size_t)units * R * 16 * B * 4;
    total = xw + bw + zero + part + 16;  // + the unit counter
  }
};

// Stage of the streaming GEMV: codes, scales and one packed word of metadata,
// unit << 4 | block-in-unit << 1 | last-block-of-unit, or -1 once the wavefront
// has no more work (uniform, so it lives in one scalar register).
template <int R, int GSUB, bool ASYM>
struct SStage {
  uint4 w[R];
  uint2 sc[R][GSUB];
  uint32_t z[R][GSUB];
  int meta;
};

// Register budget: 128 VGPRs (two 8-wavefront workgroups per CU) for one batch row
// and one group per block; smaller groups (more scales in flight) and 2-3 batch
// rows (BMAX = 2 or 4: the x registers of a unit grow with them) run with 256 -- the shapes
// that take this kernel have at most one row block per CU anyway.
template <int R, int GSUB, bool ASYM, int P, int BMAX = 1>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(BMAX == 1 && GSUB == 1 ? 4 : 1, 8)))
void gemv_stream_kernel(const uint16_t* __restrict__ x, int B, const uint4* __restrict__ packed,
                        const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int N, int K,
                        int T, int S, int Gp, int J, int nRB, uint16_t* __restrict__ y) {
  static_assert(P - 1 <= kUnitBlocks, "a unit must outlast the blocks in flight");
  // BMAX: batch rows the unit's x registers and LDS slice are sized for (B <= BMAX)
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int MPG = 4 / GSUB;
  constexpr bool BIAS = !ASYM;
  constexpr int CPU = kSuperK / GSUB / 8;  // 16-byte chunks per bias unit
  const int W = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int rb_first = blockIdx.x;
  const int rb_stride = gridDim.x;
  const int CH = S / kUnitBlocks;  // the host keeps S a multiple of 8
  const int n_rb = rb_first < nRB ? (nRB - 1 - rb_first) / rb_stride + 1 : 0;
  const int n_units = n_rb * CH;
  const GemvStreamLds lay(BMAX, GSUB, BIAS, W, R, B, n_units);
  uint16_t* xw = reinterpret_cast<uint16_t*>(smem) + (size_t)wave * BMAX * kUnitXStride;
  float* bw = reinterpret_cast<float*>(smem + lay.xw) + (size_t)wave * BMAX * kUnitBlocks * GSUB;
  uint16_t* xzero = reinterpret_cast<uint16_t*>(smem + lay.xw + lay.bw);
  float* bzero = reinterpret_cast<float*>(smem + lay.xw + lay.bw + kSuperK * 2);
  float* part0 = reinterpret_cast<float*>(smem + lay.xw + lay.bw + lay.zero);  // [unit][r][b][16 rows]
  int* counter = reinterpret_cast<int*>(smem + lay.xw + lay.bw + lay.zero + lay.part);
  const int crow = 4 * (lane >> 4);
  const int arow = lane & 15;
  const int bcol = lane & 15;
  const int kq = lane >> 4;

  // the zero row and the counter are published by the barrier after the first
  // unit's loads; a wavefront's first unit is fixed (unit `wave`; units are 8
  // blocks, longer than the P - 1 loads issued before that barrier), later ones come
  // from the counter
  if (threadIdx.x < kSuperK / 8) *reinterpret_cast<uint4*>(xzero + threadIdx.x * 8) = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x == 0) {
    *bzero = 0.f;
    *counter = W * 64;
  }

  // load side: the unit being streamed, its next block and scale group
  const unsigned char* pk = reinterpret_cast<const unsigned char*>(packed);
  const uint32_t w_lane = (uint32_t)lane * 16u;
  const uint32_t s_lane = (uint32_t)crow * 2u;
  int l_unit = -1, l_s = 0, l_s0 = 0, l_j = 0, l_jj = 0;
  const unsigned char* l_wt[R];
  const unsigned char* l_st[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    l_wt[r] = pk;
    l_st[r] = reinterpret_cast<const unsigned char*>(scales);
  }
  uint4 xn[BMAX][2];  // x of the unit taken last: channels 8 * (lane + 64 i) of its 1024, per batch row
  bool first = true;
  auto grab = [&]() __attribute__((always_inline)) {
    // the first unit is `wave`; then the counter, to which all lanes add: +64 per grab
    const int u = first ? wave : __builtin_amdgcn_readfirstlane(atomicAdd(counter, 1)) >> 6;
    first = false;
    if (u < n_units) {
      l_unit = u;
      const int i = u / CH, c = u - i * CH;
      l_s0 = l_s = c;  // blocks c, c + CH, ..., c + 7 CH (strided, as in the staged GEMV)
      l_jj = 0;
      l_j = (GSUB == 1) ? l_s / J : l_s * GSUB;
      const int rb = rb_first + i * rb_stride;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const size_t tile = (size_t)min(rb * R + r, T - 1);
        l_wt[r] = pk + tile * S * 1024;
        l_st[r] = reinterpret_cast<const unsigned char*>(scales) + tile * Gp * 32;
      }
    } else {
      l_unit = -1;  // addresses keep the last unit; the loads below repeat its x
    }
    // the unit's activations, ahead of its codes (issued on every grab, so the
    // number of loads in flight does not depend on the outcome)
#pragma unroll
    for (int b = 0; b < BMAX; ++b)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int pc = lane + 64 * i;  // 16-byte piece pc of the unit: block pc / 16
        const int k = min((l_s0 + (pc >> 4) * CH) * kSuperK + 8 * (pc & 15), K - 8);
        xn[b][i] = *reinterpret_cast<const uint4*>(x + (size_t)min(b, B - 1) * K + k);
      }
  };
  auto load = [&](SStage<R, GSUB, ASYM>& st) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const unsigned char* wp = l_wt[r] + (size_t)min(l_s, S - 1) * 1024 + w_lane;
      st.w[r] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wp)));
#pragma unroll
      for (int gs = 0; gs < GSUB; ++gs) {
        const size_t goff = (size_t)(l_j + gs) * 32;
        st.sc[r][gs] = *reinterpret_cast<const uint2*>(l_st[r] + goff + s_lane);
        if (ASYM) st.z[r][gs] = zeros[(size_t)((l_st[r] - reinterpret_cast<const unsigned char*>(scales)) >> 1) +
                                      (goff >> 1) + arow];
      }
    }
    st.meta = l_unit < 0 ? -1 : (l_unit << 4) | (l_jj << 1) | (l_jj + 1 == kUnitBlocks ? 1 : 0);
    if (l_unit < 0) return;
    l_s += CH;
    if (++l_jj == kUnitBlocks) {
      grab();
      return;
    }
    l_j = (GSUB == 1) ? (J == 1 ? l_s : l_s / J) : l_s * GSUB;
  };

  // the unit's x (x/16 at elements 2, 3, 6, 7 when BIAS; channels past K are zero)
  // -> this wavefront's LDS, with the per-block biases 1032 * sum(plain) +
  // 1152 * sum(scaled) reduced over the CPU lanes of each bias unit
  auto write_x = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
      if (b >= B) break;  // uniform
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c8 = lane + 64 * i;  // 16-byte chunk of the unit's 1024 channels
        uint4 v = ((l_s0 + (c8 >> 4) * CH) * kSuperK + 8 * (c8 & 15) < K) ? xn[b][i] : make_uint4(0u, 0u, 0u, 0u);
        if (BIAS) {
          half8_t h = as_half8(v);
          h[2] *= (_Float16)0.0625f;
          h[3] *= (_Float16)0.0625f;
          h[6] *= (_Float16)0.0625f;
          h[7] *= (_Float16)0.0625f;
          v = __builtin_bit_cast(uint4, h);
          float plain = ((float)h[0] + (float)h[1]) + ((float)h[4] + (float)h[5]);
          float scaled = ((float)h[2] + (float)h[3]) + ((float)h[6] + (float)h[7]);
#pragma unroll
          for (int m = 1; m < CPU; m <<= 1) {
            plain += __shfl_xor(plain, m);
            scaled += __shfl_xor(scaled, m);
          }
          // one explicit fma, as in every GEMV: the same rounding wherever it is inlined
          if (c8 % CPU == 0) bw[b * kUnitBlocks * GSUB + c8 / CPU] = __builtin_fmaf(1032.f, plain, 1152.f * scaled);
        }
        *reinterpret_cast<uint4*>(xw + b * kUnitXStride + 8 * c8) = v;
      }
    }
  };

  grab();
  SStage<R, GSUB, ASYM> buf[P];
#pragma unroll
  for (int p = 0; p < P - 1; ++p) load(buf[p]);
  lds_barrier();  // the zero row and the counter (written above) are set

  float4_t acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = float4_t{0.f, 0.f, 0.f, 0.f};
  const DequantRegs dq = DequantRegs::make();
  const bool real_col = bcol < B;
  const uint16_t* xlane0 = real_col ? xw + bcol * kUnitXStride + 8 * kq : xzero + 8 * kq;
  const int xstep = real_col ? kSuperK : 0;
  const float* blane0 = real_col ? bw + bcol * kUnitBlocks * GSUB : bzero;
  const int bstep = real_col ? GSUB : 0;
  half8_t xb[4];
  float bu[GSUB];
  auto read_x = [&](int j) __attribute__((always_inline)) {
    const uint16_t* xp = xlane0 + j * xstep;
#pragma unroll
    for (int m = 0; m < 4; ++m) xb[m] = *reinterpret_cast<const half8_t*>(xp + m * kBlockK);
    if (BIAS) {
      const float* bp = blane0 + j * bstep;
#pragma unroll
      for (int gs = 0; gs < GSUB; ++gs) bu[gs] = bp[gs];
    }
  };
  if (buf[0].meta >= 0) write_x();  // the first unit's x (its loads are the oldest in flight)
  read_x(0);

  auto compute = [&](const SStage<R, GSUB, ASYM>& st, const SStage<R, GSUB, ASYM>& nx) __attribute__((always_inline)) {
    half8_t xc[4];
    float bc[GSUB];
#pragma unroll
    for (int m = 0; m < 4; ++m) xc[m] = xb[m];
#pragma unroll
    for (int gs = 0; gs < GSUB; ++gs) bc[gs] = BIAS ? bu[gs] : 0.f;
    const bool last = st.meta & 1;
    if (!last) read_x((nx.meta >> 1) & 7);  // same unit: its x is in LDS already
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
    if (!last) return;
    if (real_col) {
      float* pp = part0 + (size_t)(st.meta >> 4) * R * 16 * B + bcol * 16 + crow;
#pragma unroll
      for (int r = 0; r < R; ++r) *reinterpret_cast<float4_t*>(pp + r * 16 * B) = acc[r];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = float4_t{0.f, 0.f, 0.f, 0.f};
    // the next unit: its x replaces this one's in LDS (this unit's reads of it were
    // issued earlier by this wavefront, and LDS serves them in order)
    if (nx.meta >= 0) write_x();
    read_x(0);
  };

  while (buf[0].meta >= 0) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      load(buf[(p + P - 1) % P]);
      if (buf[p].meta >= 0) compute(buf[p], buf[(p + 1) % P]);
    }
  }

  // results: the units' partials added in chunk order -> y
  lds_barrier();
  gemv_write_units<R>(part0, n_rb, CH, B, N, rb_first, rb_stride, 1, 0, y, nullptr);
}

// ---------------------------------------------------------------------------------
// The streaming GEMV for its common case: symmetric INT4 codes with one scale per
// block (groups of 128 channels), two row tiles per wavefront. Same grid, units
// (8 strided blocks), per-unit activation loads and LDS slices, arithmetic and final
// reduction as gemv_stream_kernel<2, 1, false, 4, BMAX>, so the two give identical
// bits; the instruction stream around the loads is that of gemv_burst_kernel. The
// weights of a unit go in 4 bursts of 2 blocks (each block: both row tiles' codes
// and scales), two bursts in flight: a unit's 2 x 2 tile bases are formed once
// when it is taken, the 2 blocks of a burst (CH KiB apart) are loads from those
// scalar bases plus lane offsets held in registers, and the counter is read once
// per unit. The unit's x loads go out when it is taken, right before its first
// codes; the x of the next unit replaces this one's in the wavefront's LDS slice when
// this unit's last block is computed (4 bursts per unit, 2 in flight: the next unit
// is taken only after that). It holds more registers than 128 (one 8-wavefront
// workgroup per CU), so the host runs it where the grid needs no more than that.
template <int BMAX>
__global__ __launch_bounds__(512)
void gemv_stream_burst_kernel(const uint16_t* __restrict__ x, int B, const uint4* __restrict__ packed,
                              const uint16_t* __restrict__ scales, int N, int K, int T, int S, int Gp, int nRB,
                              uint16_t* __restrict__ y) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int R = 2;                        // row tiles per wavefront
  constexpr int NB = 2;                       // blocks per burst
  constexpr int BURSTS = kUnitBlocks / NB;    // bursts per unit
  constexpr int CPU = kSuperK / 8;            // 16-byte chunks per bias unit (one block)
  static_assert(BURSTS >= 2, "the next unit is taken only after this one's last block is computed");
  const int W = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int rb_first = blockIdx.x;
  const int rb_stride = gridDim.x;
  const int CH = S / kUnitBlocks;  // the host keeps S a multiple of 8
  const int n_rb = rb_first < nRB ? (nRB - 1 - rb_first) / rb_stride + 1 : 0;
  const int n_units = n_rb * CH;
  const GemvStreamLds lay(BMAX, 1, true, W, R, B, n_units);
  uint16_t* xw = reinterpret_cast<uint16_t*>(smem) + (size_t)wave * BMAX * kUnitXStride;
  float* bw = reinterpret_cast<float*>(smem + lay.xw) + (size_t)wave * BMAX * kUnitBlocks;
  uint16_t* xzero = reinterpret_cast<uint16_t*>(smem + lay.xw + lay.bw);
  float* bzero = reinterpret_cast<float*>(smem + lay.xw + lay.bw + kSuperK * 2);
  float* part0 = reinterpret_cast<float*>(smem + lay.xw + lay.bw + lay.zero);  // [unit][r][b][16 rows]
  int* counter = reinterpret_cast<int*>(smem + lay.xw + lay.bw + lay.zero + lay.part);
  const int crow = 4 * (lane >> 4);
  const int bcol = lane & 15;
  const int kq = lane >> 4;

  // the zero row and the counter are published by the barrier after the first
  // burst; each wavefront's first unit is fixed (unit `wave`: a unit is 4 bursts, so
  // the one burst issued before that barrier never ends it), later ones come from the
  // counter, read only after the barrier
  if (threadIdx.x < kSuperK / 8) *reinterpret_cast<uint4*>(xzero + threadIdx.x * 8) = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x == 0) {
    *bzero = 0.f;
    *counter = W * 64;
  }

  const unsigned char* pk = reinterpret_cast<const unsigned char*>(packed);
  const unsigned char* sk = reinterpret_cast<const unsigned char*>(scales);
  const uint32_t cstride = (uint32_t)CH * 1024u;  // bytes between a unit's blocks (codes)
  const uint32_t sstride = (uint32_t)CH * 32u;    // ... (scales)
  uint32_t woff[NB], soff[NB], lw[NB], ls[NB];  // lane offsets of a burst's blocks; lw, ls: those loads use now
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    woff[q] = (uint32_t)lane * 16u + q * cstride;
    soff[q] = (uint32_t)crow * 2u + q * sstride;
    lw[q] = woff[q];
    ls[q] = soff[q];
  }
  // cursor (uniform): unit being streamed (-1 once they have run out), its chunk,
  // the code and scale bases of its two tiles (block c of each), the next burst
  int c_unit = -1, c_chunk = 0, c_burst = 0;
  const unsigned char* c_w[R] = {pk, pk};
  const unsigned char* c_s[R] = {sk, sk};
  uint4 xn[BMAX][2];  // x of the unit taken last: channels 8 * (lane + 64 i) of its 1024, per batch row
  bool first = true;
  auto take = [&]() __attribute__((always_inline)) {
    const int u = first ? wave : __builtin_amdgcn_readfirstlane(atomicAdd(counter, 1)) >> 6;
    first = false;
    c_burst = 0;
    if ((unsigned)u < (unsigned)n_units) {
      c_unit = u;
      const int i = u / CH;
      c_chunk = u - i * CH;
      const int rb = rb_first + i * rb_stride;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const size_t tile = (size_t)min(rb * R + r, T - 1);
        c_w[r] = pk + (tile * S + c_chunk) * 1024;
        c_s[r] = sk + (tile * Gp + c_chunk) * 32;
      }
    } else {
      // no more units: the loads that still follow (unconditional, for exact vmcnt
      // counts) all re-read the block loaded last (still in the L2 or on its way; the
      // last whole burst cost 4-5% more HBM bytes on down and o), and the x loads
      // repeat the last unit's
      c_unit = -1;
      c_burst = BURSTS - 1;
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        lw[q] = woff[NB - 1];
        ls[q] = soff[NB - 1];
      }
    }
    // the unit's activations, ahead of its codes (issued on every take, so the
    // number of loads in flight does not depend on the outcome)
#pragma unroll
    for (int b = 0; b < BMAX; ++b)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int pc = lane + 64 * i;  // 16-byte piece pc of the unit: block pc / 16
        const int k = min((c_chunk + (pc >> 4) * CH) * kSuperK + 8 * (pc & 15), K - 8);
        xn[b][i] = *reinterpret_cast<const uint4*>(x + (size_t)min(b, B - 1) * K + k);
      }
  };

  struct Burst {
    uint4 w[NB][R];
    uint2 sc[NB][R];
    int unit, j0;
    bool last;
  };
  auto issue = [&](Burst& bt) __attribute__((always_inline)) {
    const size_t boff = (size_t)c_burst * NB * CH;
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        bt.w[q][r] = __builtin_bit_cast(
            uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(c_w[r] + boff * 1024 + lw[q])));
        bt.sc[q][r] = *reinterpret_cast<const uint2*>(c_s[r] + boff * 32 + ls[q]);
      }
    bt.unit = c_unit;
    bt.j0 = c_burst * NB;
    bt.last = c_burst + 1 == BURSTS;
    if (c_unit < 0) return;
    if (++c_burst == BURSTS) take();
  };

  // the unit's x (x/16 at elements 2, 3, 6, 7; channels past K are zero) -> this
  // wavefront's LDS, with the per-block biases 1032 * sum(plain) + 1152 * sum(scaled)
  // reduced over the 16 lanes of each block
  int xn_chunk = 0;  // chunk of the unit whose x is in xn
  auto write_x = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
      if (b >= B) break;  // uniform
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c8 = lane + 64 * i;  // 16-byte chunk of the unit's 1024 channels
        uint4 v = ((xn_chunk + (c8 >> 4) * CH) * kSuperK + 8 * (c8 & 15) < K) ? xn[b][i] : make_uint4(0u, 0u, 0u, 0u);
        half8_t h = as_half8(v);
        h[2] *= (_Float16)0.0625f;
        h[3] *= (_Float16)0.0625f;
        h[6] *= (_Float16)0.0625f;
        h[7] *= (_Float16)0.0625f;
        v = __builtin_bit_cast(uint4, h);
        float plain = ((float)h[0] + (float)h[1]) + ((float)h[4] + (float)h[5]);
        float scaled = ((float)h[2] + (float)h[3]) + ((float)h[6] + (float)h[7]);
#pragma unroll
        for (int m = 1; m < CPU; m <<= 1) {
          plain += __shfl_xor(plain, m);
          scaled += __shfl_xor(scaled, m);
        }
        if (c8 % CPU == 0) bw[b * kUnitBlocks + c8 / CPU] = __builtin_fmaf(1032.f, plain, 1152.f * scaled);
        *reinterpret_cast<uint4*>(xw + b * kUnitXStride + 8 * c8) = v;
      }
    }
  };

  take();
  xn_chunk = c_chunk;
  Burst ring[2];
  issue(ring[0]);
  lds_barrier();  // the zero row and the counter (written above) are set

  float4_t acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = float4_t{0.f, 0.f, 0.f, 0.f};
  const DequantRegs dq = DequantRegs::make();
  const bool real_col = bcol < B;
  const uint16_t* xlane0 = real_col ? xw + bcol * kUnitXStride + 8 * kq : xzero + 8 * kq;
  const float* blane0 = real_col ? bw + bcol * kUnitBlocks : bzero;
  half8_t xb[4];
  float bu;
  auto read_x = [&](int j) __attribute__((always_inline)) {  // block j of the unit in LDS
    const uint16_t* xp = xlane0 + (real_col ? j * kSuperK : 0);
#pragma unroll
    for (int m = 0; m < 4; ++m) xb[m] = *reinterpret_cast<const half8_t*>(xp + m * kBlockK);
    bu = blane0[real_col ? j : 0];
  };
  if (ring[0].unit >= 0) write_x();  // the first unit's x (its loads are the oldest in flight)
  read_x(0);

  auto compute = [&](const Burst& bt, const Burst& nx) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      half8_t xc[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) xc[m] = xb[m];
      const float bc = bu;
      const bool last = bt.last && q + 1 == NB;
      if (!last) read_x(bt.j0 + q + 1);  // same unit: its x is in LDS already
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const half4_t sh = __builtin_bit_cast(half4_t, bt.sc[q][r]);
        float4_t part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) part = mfma16x16x32(magic8r(lane_dword(bt.w[q][r], mm), dq), xc[mm], part);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[r][i] = __builtin_fmaf((float)sh[i], part[i] - bc, acc[r][i]);
      }
      if (!last) continue;
      if (real_col) {
        float* pp = part0 + (size_t)bt.unit * R * 16 * B + bcol * 16 + crow;
#pragma unroll
        for (int r = 0; r < R; ++r) *reinterpret_cast<float4_t*>(pp + r * 16 * B) = acc[r];
      }
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = float4_t{0.f, 0.f, 0.f, 0.f};
      // the next unit: its x replaces this one's in LDS (this unit's reads of it were
      // issued earlier by this wavefront, and LDS serves them in order)
      if (nx.unit >= 0) {
        xn_chunk = nx.unit - (nx.unit / CH) * CH;
        write_x();
      }
      read_x(0);
    }
  };

  // once a burst has no unit, every later one has none either
  while (ring[0].unit >= 0) {
    issue(ring[1]);
    compute(ring[0], ring[1]);
    issue(ring[0]);
    if (ring[1].unit < 0) break;
    compute(ring[1], ring[0]);
  }

  // results: the units' partials added in chunk order -> y
  lds_barrier();
  gemv_write_units<R>(part0, n_rb, CH, B, N, rb_first, rb_stride, 1, 0, y, nullptr);
}

template <int R, int GSUB, bool ASYM, int XCH, bool Q8 = false>
hipError_t launch_gemv_t(const GemmArgs& a, hipStream_t stream) {
  // ring stages per row-tile count: INT4 with one row tile, two bursts of 4
  // blocks; otherwise blocks in flight + 1 (INT8 blocks are twice as large)
  constexpr int P = Q8 ? (R == 1 ? 4 : 3) : (R == 1 ? 8 : 4);
  const int T = a.Np / kTileRows;
  const int S = a.Kp / kSuperK;
  const int J = a.group >= kSuperK ? a.group / kSuperK : 1;
  const int W = std::min(a.waves_per_group, gemv_max_waves<R, GSUB, Q8>());
  const int KS = a.k_splits;
  const int nRB = (T + R - 1) / R;
  const int max_nsb = (S + KS - 1) / KS;
  const int min_nsb = S / KS;  // >= 1: the host keeps KS <= S
  // the burst kernel where its conditions hold (same grid, units and result bits)
  constexpr bool kBurstKind = R == 1 && GSUB == 1 && !ASYM;
  const bool burst = kBurstKind && (Q8 || J == 1) && S % KS == 0;  // CH is checked below (INT8: one group per row)
  // bursts of 2 blocks on rows of >= 8192 channels and from B = 4 up (ABBA against 4: q/k/v
  // of the 70B layer -0.7 to -0.9 us at B = 1-16, gate/up and 28672x8192 -0.2 to -0.7 us;
  // 4096-channel rows of the 8B layer -0.3 to -1.0 us at B = 4-8), of 4 on shorter rows at
  // B <= 3 (4096x4096, 6144x4096 and 28672x4096 at B = 1: 0.2-0.4 us faster with 4)
  // (INT8 blocks are 2 KiB: bursts of 2 blocks always)
  const int NBB = (Q8 || S >= 64 || a.B >= 4) ? 2 : 4;
  const void* fn = !burst ? reinterpret_cast<const void*>(&gemv_kernel<R, GSUB, ASYM, P, XCH, Q8>)
                   : NBB == 2 ? reinterpret_cast<const void*>(&gemv_burst_kernel<XCH, 2, Q8>)
                              : reinterpret_cast<const void*>(&gemv_burst_kernel<XCH, 4, Q8>);
  const size_t lim = a.lds_limit;
  const size_t unit_bytes = (size_t)R * 16 * a.B * 4;
  const size_t base = GemvLds(a.B, max_nsb, GSUB, !ASYM, R, 0).total;
  // Persistent grid: as many workgroups as stay resident, the row blocks spread
  // evenly over them; more workgroups only if one row block per chunk would not
  // fit the LDS limit.
  const int64_t resident = (int64_t)resident_per_cu(fn, W * kWave, base + unit_bytes) * device_cu_count_cached();
  int64_t per_split = std::max<int64_t>(1, std::min<int64_t>(nRB, resident / KS));
  if (a.grid_limit > 0) per_split = std::min<int64_t>(per_split, std::max(1, a.grid_limit / KS));
  int n_rb = (int)((nRB + per_split - 1) / per_split);
  const int64_t max_rb = std::max<int64_t>(1, (int64_t)((lim - std::min(lim, base)) / unit_bytes));
  if (n_rb > max_rb) {
    n_rb = (int)max_rb;
    per_split = (nRB + n_rb - 1) / n_rb;
  }
  n_rb = (int)((nRB + per_split - 1) / per_split);
  // chunks per row block: 8 blocks (8 KiB of codes per tile) each, which streams
  // best; shorter ones if that leaves fewer than two units per wavefront; at most
  // 64 and as many as the LDS holds
  int CH = std::max(1, min_nsb / 8);
  if ((int64_t)CH * n_rb < 2 * W) CH = (int)std::min<int64_t>(min_nsb, (2 * W + n_rb - 1) / n_rb);
  CH = std::min(CH, 64);
  CH = (int)std::min<int64_t>(CH, std::max<int64_t>(1, (int64_t)((lim - std::min(lim, base)) / (unit_bytes * n_rb))));
  CH = std::max(CH, 1);
  if (burst && min_nsb % NBB == 0 && min_nsb % (NBB * CH) != 0) {
    // the burst kernel needs units of whole bursts: the next larger CH that divides
    // the split's bursts (shorter units) where its partials fit the LDS
    const int bursts = min_nsb / NBB;
    const int64_t ch_max = std::min<int64_t>(
        64, std::max<int64_t>(1, (int64_t)((lim - std::min(lim, base)) / (unit_bytes * n_rb))));
    for (int d = CH + 1; d <= bursts && d <= ch_max; ++d)
      if (bursts % d == 0) {
        CH = d;
        break;
      }
  }
  const size_t lds = GemvLds(a.B, max_nsb, GSUB, !ASYM, R, n_rb * CH).total;
  const int grid = (int)(per_split * KS);
  if constexpr (kBurstKind) {
    if (burst && (S / KS) % (NBB * CH) == 0) {
      if (NBB == 2)
        hipLaunchKernelGGL((gemv_burst_kernel<XCH, 2, Q8>), dim3(grid), dim3(W * kWave), lds, stream,
                           static_cast<const uint16_t*>(a.x), a.B, static_cast<const uint4*>(a.packed),
                           static_cast<const uint16_t*>(a.scales), a.N, a.K, S, a.Gp, KS, nRB, CH,
                           static_cast<uint16_t*>(a.y), static_cast<float*>(a.workspace));
      else
        hipLaunchKernelGGL((gemv_burst_kernel<XCH, 4, Q8>), dim3(grid), dim3(W * kWave), lds, stream,
                           static_cast<const uint16_t*>(a.x), a.B, static_cast<const uint4*>(a.packed),
                           static_cast<const uint16_t*>(a.scales), a.N, a.K, S, a.Gp, KS, nRB, CH,
                           static_cast<uint16_t*>(a.y), static_cast<float*>(a.workspace));
      if (KS > 1)
        launch_reduce_splits(static_cast<const float*>(a.workspace), KS, (int64_t)a.B * a.N,
                             static_cast<uint16_t*>(a.y), stream);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemv_kernel<R, GSUB, ASYM, P, XCH, Q8>), dim3(grid), dim3(W * kWave), lds, stream,
                     static_cast<const uint16_t*>(a.x), a.B, static_cast<const uint4*>(a.packed),
                     static_cast<const uint16_t*>(a.scales), static_cast<const uint8_t*>(a.zeros), a.N, a.K, T, S,
                     a.Gp, J, KS, nRB, CH, static_cast<uint16_t*>(a.y), static_cast<float*>(a.workspace));
  if (KS > 1)
    launch_reduce_splits(static_cast<const float*>(a.workspace), KS, (int64_t)a.B * a.N, static_cast<uint16_t*>(a.y),
                         stream);
  return hipGetLastError();
}

// x chunks of 16 bytes each thread copies: the fewest of 2, 4, 8 that cover the
// activation slice of the largest split
template <int R, int GSUB, bool ASYM, bool Q8 = false>
hipError_t launch_gemv_x(const GemmArgs& a, hipStream_t stream) {
  const int W = std::min(a.waves_per_group, gemv_max_waves<R, GSUB, Q8>());
  const int64_t max_nsb = (a.Kp / kSuperK + a.k_splits - 1) / a.k_splits;
  const int64_t per_thread = ((int64_t)a.B * max_nsb * 16 + W * kWave - 1) / (W * kWave);
  if (per_thread <= 2) return launch_gemv_t<R, GSUB, ASYM, 2, Q8>(a, stream);
  if (per_thread <= 4) return launch_gemv_t<R, GSUB, ASYM, 4, Q8>(a, stream);
  return launch_gemv_t<R, GSUB, ASYM, 8, Q8>(a, stream);
}

template <int R, bool ASYM>
hipError_t launch_gemv_g(const GemmArgs& a, hipStream_t stream) {
  if (a.group == 32) return launch_gemv_x<R, 4, ASYM>(a, stream);
  if (a.group == 64) return launch_gemv_x<R, 2, ASYM>(a, stream);
  return launch_gemv_x<R, 1, ASYM>(a, stream);
}

template <int R>
hipError_t launch_gemv_a(const GemmArgs& a, hipStream_t stream) {
  return a.asym ? launch_gemv_g<R, true>(a, stream) : launch_gemv_g<R, false>(a, stream);
}

template <int R, int GSUB, bool ASYM, int BMAX>
hipError_t launch_gemv_stream_t(const GemmArgs& a, hipStream_t stream) {
  constexpr int P = R == 1 ? 8 : 4;
  const int T = a.Np / kTileRows;
  const int S = a.Kp / kSuperK;
  const int J = a.group >= kSuperK ? a.group / kSuperK : 1;
  const int W = std::min(a.waves_per_group, 8);
  const int nRB = (T + R - 1) / R;
  const int CH = S / kUnitBlocks;
  // the burst form where its conditions hold (same grid, units and result bits)
  constexpr bool kBurstKind = R == 2 && GSUB == 1 && !ASYM;
  const bool burst = kBurstKind && gemv_stream_burst_ok(a.Np, a.group, a.asym, a.q8, device_cu_count_cached());
  const void* fn = burst ? reinterpret_cast<const void*>(&gemv_stream_burst_kernel<BMAX>)
                         : reinterpret_cast<const void*>(&gemv_stream_kernel<R, GSUB, ASYM, P, BMAX>);
  const size_t unit_bytes = (size_t)R * 16 * a.B * 4;
  const size_t base = GemvStreamLds(BMAX, GSUB, !ASYM, W, R, a.B, 0).total;
  const size_t lim = std::max(a.lds_limit, base + unit_bytes * CH);
  const int64_t resident = (int64_t)resident_per_cu(fn, W * kWave, base + unit_bytes * CH) * device_cu_count_cached();
  int64_t grid = std::max<int64_t>(1, std::min<int64_t>(nRB, resident));
  if (a.grid_limit > 0) grid = std::min<int64_t>(grid, a.grid_limit);
  int n_rb = (int)((nRB + grid - 1) / grid);
  const int64_t max_rb = std::max<int64_t>(1, (int64_t)((lim - base) / (unit_bytes * CH)));
  if (n_rb > max_rb) grid = (nRB + max_rb - 1) / max_rb;
  n_rb = (int)((nRB + grid - 1) / grid);
  const size_t lds = GemvStreamLds(BMAX, GSUB, !ASYM, W, R, a.B, n_rb * CH).total;
  if constexpr (kBurstKind) {
    if (burst) {
      hipLaunchKernelGGL((gemv_stream_burst_kernel<BMAX>), dim3((unsigned)grid), dim3(W * kWave), lds, stream,
                         static_cast<const uint16_t*>(a.x), a.B, static_cast<const uint4*>(a.packed),
                         static_cast<const uint16_t*>(a.scales), a.N, a.K, T, S, a.Gp, nRB,
                         static_cast<uint16_t*>(a.y));
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemv_stream_kernel<R, GSUB, ASYM, P, BMAX>), dim3((unsigned)grid), dim3(W * kWave), lds,
                     stream, static_cast<const uint16_t*>(a.x), a.B, static_cast<const uint4*>(a.packed),
                     static_cast<const uint16_t*>(a.scales), static_cast<const uint8_t*>(a.zeros), a.N, a.K, T, S,
                     a.Gp, J, nRB, static_cast<uint16_t*>(a.y));
  return hipGetLastError();
}

template <int R, bool ASYM, int BMAX>
hipError_t launch_gemv_stream_b(const GemmArgs& a, hipStream_t stream) {
  if (a.group == 32) return launch_gemv_stream_t<R, 4, ASYM, BMAX>(a, stream);
  if (a.group == 64) return launch_gemv_stream_t<R, 2, ASYM, BMAX>(a, stream);
  return launch_gemv_stream_t<R, 1, ASYM, BMAX>(a, stream);
}

template <int R, bool ASYM>
hipError_t launch_gemv_stream_g(const GemmArgs& a, hipStream_t stream) {
  if (a.B == 1) return launch_gemv_stream_b<R, ASYM, 1>(a, stream);
  if (a.B == 2) return launch_gemv_stream_b<R, ASYM, 2>(a, stream);
  return launch_gemv_stream_b<R, ASYM, 4>(a, stream);
}

template <int R>
hipError_t launch_gemv_stream_a(const GemmArgs& a, hipStream_t stream) {
  return a.asym ? launch_gemv_stream_g<R, true>(a, stream) : launch_gemv_stream_g<R, false>(a, stream);
}

hipError_t launch_gemv(const GemmArgs& a, hipStream_t stream) {
  if (a.q8) {
    switch (a.rows_per_wave) {
      case 1: return launch_gemv_x<1, 1, false, true>(a, stream);
      case 2: return launch_gemv_x<2, 1, false, true>(a, stream);
      default: return launch_gemv_x<4, 1, false, true>(a, stream);
    }
  }
  if (gemv_streams_x(a.B, a.Kp, a.rows_per_wave, a.k_splits,
                     gemv_stream_burst_ok(a.Np, a.group, a.asym, a.q8, device_cu_count_cached())))
    return launch_gemv_stream_a<2>(a, stream);
  switch (a.rows_per_wave) {
    case 1: return launch_gemv_a<1>(a, stream);
    case 2: return launch_gemv_a<2>(a, stream);
    default: return launch_gemv_a<4>(a, stream);
  }
}

// ---------------------------------------------------------------------------------
// Skinny GEMM for B > 16 (MFMA-bound from a few dozen rows of x upward).
//
// Workgroup = WV (4 or 8) wavefronts; wavefront w owns row tiles WV*RT*blockIdx.x + RT*w + r,
// the workgroup owns column tiles CT*blockIdx.y .. + CT - 1 (16 batch rows each).
// Codes are dequantized exactly to float16 integers (q, or q - z) in registers, as
// in the GEMV; each group's MFMA partial sum is scaled in float32 and added to the
// accumulator tile. The channel range is walked in chunks of NB blocks (NB * 128
// channels): the chunk's activation tile (CT*16 rows) sits in one of two padded
// LDS buffers and is read by all wavefronts as B operands, each read feeding
// RT row tiles. The next chunk's tile is loaded into registers a whole chunk ahead
// and written to the other buffer at the chunk's end, so there is one barrier per
// chunk; codes and scales stream through a ring of NB stages (NB - 1 blocks in
// flight) that runs on across chunk boundaries.
template <int RT, int GSUB, bool ASYM, int NW = 1>
struct GStage {
  uint4 w[RT][NW];       // NW 16-byte pieces of codes per lane and block (1: INT4, 2: INT8)
  uint2 sc[RT][GSUB];    // float16 scales of the lane's accumulator rows (C layout) per group
  uint32_t z[RT][GSUB];  // zero point of the lane's A-operand row per group (asymmetric)
};

// Q8: per-channel INT8 codes (the GEMV's 2 KiB block layout, one scale per row
// passed as a single group spanning the row): each code pair becomes 1024 + q + 128
// through v_perm_b32 (magic8_i8) and one packed add of -1152 leaves q exactly.
template <int RT, int CT, int GSUB, bool ASYM, int NB, int WV, bool Q8 = false>
__global__ __launch_bounds__(WV * 64) void gemm_mfma_kernel(const uint16_t* __restrict__ x, int B,
                                                        const uint4* __restrict__ packed,
                                                        const uint16_t* __restrict__ scales,
                                                        const uint8_t* __restrict__ zeros, int N, int K, int T,
                                                        int S, int Gp, int J, uint16_t* __restrict__ y,
                                                        float* __restrict__ ws) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int MPG = 4 / GSUB;
  constexpr int XROWS = CT * 16;
  constexpr int KC = NB * kSuperK;           // channels per chunk
  constexpr int XSTR = KC + kGemmRowPad;     // halfs per LDS row (32-byte pad: conflict-free B reads)
  constexpr int C8 = KC / 8;                 // 16-byte pieces per row of a chunk
  constexpr int NT = WV * 64;                // threads
  constexpr int XCH = XROWS * C8 / NT;       // pieces of one chunk's tile per thread
  constexpr int NW = Q8 ? 2 : 1;             // 16-byte code pieces per lane and block
  static_assert(!Q8 || (GSUB == 1 && !ASYM), "INT8 codes are symmetric with one scale per row");
  uint16_t* xbuf = reinterpret_cast<uint16_t*>(smem);  // [2][XROWS][XSTR]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4, arow = lane & 15, crow = 4 * (lane >> 4);
  const int tile0 = blockIdx.x * WV * RT + wave * RT;
  const int b0 = blockIdx.y * XROWS;
  // k-split blockIdx.z of gridDim.z: whole chunks [c0, c0 + nchunks) of the channel range
  const int all_chunks = (S + NB - 1) / NB;
  const int KS = gridDim.z, ks = blockIdx.z;
  const int c0 = (int)(((int64_t)all_chunks * ks) / KS);
  const int nchunks = (int)(((int64_t)all_chunks * (ks + 1)) / KS) - c0;  // >= 1: the host keeps KS <= chunks
  const int S1 = min(S, (c0 + nchunks) * NB);  // end of this split's blocks

  int tiles[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) tiles[r] = min(tile0 + r, T - 1);

  auto load_w = [&](GStage<RT, GSUB, ASYM, NW>& st, int s) __attribute__((always_inline)) {
    s = min(c0 * NB + s, S1 - 1);  // trailing prefetches re-read the last block: no branch around loads
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const uint4* wp = packed + ((size_t)tiles[r] * S + s) * kWave * NW + lane;
#pragma unroll
      for (int h = 0; h < NW; ++h)
        st.w[r][h] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wp + kWave * h)));
#pragma unroll
      for (int gs = 0; gs < GSUB; ++gs) {
        const int j = (GSUB == 1) ? s / J : s * GSUB + gs;
        const size_t g0 = ((size_t)tiles[r] * Gp + j) * 16;
        st.sc[r][gs] = *reinterpret_cast<const uint2*>(scales + g0 + crow);
        if (ASYM) st.z[r][gs] = zeros[g0 + arow];
      }
    }
  };
  // this thread's pieces of a chunk's activation tile: piece i = threadIdx.x + NT * i
  // -> row i / C8, 8 halfs at 8 * (i % C8) of the chunk
  auto load_x = [&](uint4 (&v)[XCH], int c) __attribute__((always_inline)) {
    c = c0 + min(c, nchunks - 1);
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int pc = threadIdx.x + NT * i;
      const int b = min(b0 + pc / C8, B - 1);
      const int k = min(c * KC + 8 * (pc % C8), K - 8);
      v[i] = *reinterpret_cast<const uint4*>(x + (size_t)b * K + k);
    }
  };
  auto store_x = [&](const uint4 (&v)[XCH], int c, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int pc = threadIdx.x + NT * i;
      const int row = pc / C8, col = 8 * (pc % C8);
      const bool valid = (b0 + row < B) && ((c0 + c) * KC + col < K);
      *reinterpret_cast<uint4*>(xbuf + (buf * XROWS + row) * XSTR + col) = valid ? v[i] : make_uint4(0u, 0u, 0u, 0u);
    }
  };

  float4_t acc[RT][CT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[r][c] = float4_t{0.f, 0.f, 0.f, 0.f};

  uint4 xv[XCH];
  load_x(xv, 0);
  GStage<RT, GSUB, ASYM, NW> ring[NB];
#pragma unroll
  for (int p = 0; p < NB - 1; ++p) load_w(ring[p], p);
  store_x(xv, 0, 0);
  lds_barrier();
  load_x(xv, 1);  // a whole chunk ahead

  const DequantRegs dq = DequantRegs::make();

  // block p of the chunk in buffer buf, codes from stage st
  auto step = [&](const GStage<RT, GSUB, ASYM, NW>& st, int buf, int p) __attribute__((always_inline)) {
    half8_t a[RT][4];
    float4_t sc[RT][GSUB];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
#pragma unroll
      for (int gs = 0; gs < GSUB; ++gs) {
        const _Float16 z = ASYM ? (_Float16)(float)st.z[r][gs] : (_Float16)8.0f;
        const half2_t blo = {(_Float16)-1024.0f - z, (_Float16)-1024.0f - z};
        const half2_t bhi = {(_Float16)-64.0f - z, (_Float16)-64.0f - z};
        if constexpr (Q8) {
          const half8_t bias8 = {(_Float16)-1152.0f, (_Float16)-1152.0f, (_Float16)-1152.0f, (_Float16)-1152.0f,
                                 (_Float16)-1152.0f, (_Float16)-1152.0f, (_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
          for (int mm = 0; mm < 4; ++mm) {
            const uint4& v = st.w[r][mm >> 1];
            a[r][mm] = magic8_i8(lane_dword(v, 2 * (mm & 1)), lane_dword(v, 2 * (mm & 1) + 1)) + bias8;
          }
        } else {
#pragma unroll
          for (int mm = 0; mm < MPG; ++mm)
            a[r][gs * MPG + mm] = dequant8r(lane_dword(st.w[r][0], gs * MPG + mm), dq, blo, bhi);
        }
        const half4_t sh = __builtin_bit_cast(half4_t, st.sc[r][gs]);
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[r][gs][i] = (float)sh[i];
      }
    }
    const uint16_t* xb = xbuf + (buf * XROWS + (lane & 15)) * XSTR + p * kSuperK + 8 * kq;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      half8_t bop[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) bop[m] = *reinterpret_cast<const half8_t*>(xb + c * 16 * XSTR + m * kBlockK);
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
  };

  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      const int s = c * NB + p;  // block of this split
      load_w(ring[(p + NB - 1) % NB], s + NB - 1);  // into the slot of block s - 1
      if (c0 * NB + s < S1) step(ring[p], buf, p);
    }
    // the next chunk's tile into the other buffer (last read in chunk c - 1, before
    // the previous barrier), then the one after that into registers
    store_x(xv, c + 1, buf ^ 1);
    lds_barrier();
    load_x(xv, c + 2);
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
        if (n >= N) continue;
        if (KS == 1) y[(size_t)b * N + n] = __builtin_bit_cast(uint16_t, (_Float16)acc[r][c][i]);
        else ws[((size_t)ks * B + b) * N + n] = acc[r][c][i];
      }
    }
  }
}

template <int RT, int CT, int GSUB, bool ASYM, int WV, bool Q8 = false>
hipError_t launch_mfma_t(const GemmArgs& a, hipStream_t stream) {
  constexpr int NB = mfma_chunk_blocks(CT);
  const int T = a.Np / kTileRows;
  const int S = a.Kp / kSuperK;
  const int J = a.group >= kSuperK ? a.group / kSuperK : 1;
  const int col_tiles = (a.B + 15) / 16;
  const int KS = a.k_splits;
  dim3 grid((T + WV * RT - 1) / (WV * RT), (col_tiles + CT - 1) / CT, KS);
  const size_t lds = mfma_lds_bytes(CT);
  hipLaunchKernelGGL((gemm_mfma_kernel<RT, CT, GSUB, ASYM, NB, WV, Q8>), grid, dim3(WV * 64), lds, stream,
                     static_cast<const uint16_t*>(a.x), a.B, static_cast<const uint4*>(a.packed),
                     static_cast<const uint16_t*>(a.scales), static_cast<const uint8_t*>(a.zeros), a.N, a.K, T, S,
                     a.Gp, J, static_cast<uint16_t*>(a.y), static_cast<float*>(a.workspace));
  if (KS > 1)
    launch_reduce_splits(static_cast<const float*>(a.workspace), KS, (int64_t)a.B * a.N, static_cast<uint16_t*>(a.y),
                         stream);
  return hipGetLastError();
}

// Only shapes whose accumulators and per-group partial tiles fit the register file
// (RT * CT * GSUB <= 16, and RT <= 2 with 8 wavefronts) are built; the host never
// selects the others.
template <int RT, int CT, int GSUB, bool ASYM, bool Q8 = false>
hipError_t launch_mfma_fit(const GemmArgs& a, hipStream_t stream) {
  if constexpr (RT * CT * GSUB <= 16) {
    if constexpr (RT <= 2) {  // 8 wavefronts: at most 256 VGPRs each
      if (a.waves_per_group == 8) return launch_mfma_t<RT, CT, GSUB, ASYM, 8, Q8>(a, stream);
    }
    return launch_mfma_t<RT, CT, GSUB, ASYM, 4, Q8>(a, stream);
  }
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
  if (a.q8) return launch_mfma_fit<RT, CT, 1, false, true>(a, stream);
  return a.asym ? launch_mfma_g<RT, CT, true>(a, stream) : launch_mfma_g<RT, CT, false>(a, stream);
}

template <int RT, int CT>
int mfma_resident_t() {
  const void* fn =
      reinterpret_cast<const void*>(&gemm_mfma_kernel<RT, CT, 1, false, mfma_chunk_blocks(CT), 8, false>);
  return resident_per_cu(fn, 8 * kWave, mfma_lds_bytes(CT));
}

template <int CT>
int mfma_resident_r(int rows_per_wave) {
  return rows_per_wave == 1 ? mfma_resident_t<1, CT>() : mfma_resident_t<2, CT>();
}

template <int CT>
hipError_t launch_mfma_r(const GemmArgs& a, hipStream_t stream) {
  if (a.rows_per_wave == 1) return launch_mfma_a<1, CT>(a, stream);
  if (a.rows_per_wave == 2) return launch_mfma_a<2, CT>(a, stream);
  return launch_mfma_a<4, CT>(a, stream);
}

}  // namespace

// x_perm[b][k] = x[b][perm[k]] (indices clamped into the row): the act-order
// reorder of the activations ("Post-training quantization: GPTQ, AWQ and rotation",
// arganzheng.life, section 十一.2: a gather), written to the workspace ahead of the
// GEMV / skinny GEMM, which then run unchanged on the permuted codes. Gathering
// inside the GEMV's activation staging instead was measured slower at every batch
// size (2-byte gathers repeated by every workgroup; +3 to +33 us on the 70B
// shapes against ~2.2 us for this kernel and its boundary).
// Eight outputs per thread (K is a multiple of 32): two 16-byte loads of perm,
// eight 2-byte gathers, one 16-byte store.
__global__ void gather_cols_kernel(const uint16_t* __restrict__ x, int B, int K, const int32_t* __restrict__ perm,
                                   uint16_t* __restrict__ xp) {
  const int K8 = K / 8;
  const int64_t total = (int64_t)B * K8;
  const unsigned km = (unsigned)(K - 1);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = i / K8;
    const int k = (int)(i - b * K8) * 8;
    const int4 p0 = *reinterpret_cast<const int4*>(perm + k);
    const int4 p1 = *reinterpret_cast<const int4*>(perm + k + 4);
    const uint16_t* xrow = x + b * K;
    auto at = [&](int j) __attribute__((always_inline)) { return (uint32_t)xrow[min((unsigned)j, km)]; };
    *reinterpret_cast<uint4*>(xp + b * K + k) =
        make_uint4(at(p0.x) | at(p0.y) << 16, at(p0.z) | at(p0.w) << 16, at(p1.x) | at(p1.y) << 16,
                   at(p1.z) | at(p1.w) << 16);
  }
}

// Library-owned device scratch for q4_gemm_noalloc (callers that cannot allocate):
// the split partial sums that q4_gemm keeps in the caller's workspace. Each GPU the
// library runs on holds its own copy until the process ends. In host code `scratch`
// names a host-side stand-in, so its device address is looked up once per device
// and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** out) {
  static std::mutex mu;
  static std::map<int, void*> ptrs;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  auto it = ptrs.find(dev);
  if (it == ptrs.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // on the current device
    if (e != hipSuccess) return e;
    it = ptrs.emplace(dev, p).first;
  }
  *out = it->second;
  return hipSuccess;
}

int mfma_resident_per_cu(int rows_per_wave, int col_tiles) {
  switch (col_tiles) {
    case 2: return mfma_resident_r<2>(rows_per_wave);
    case 3: return mfma_resident_r<3>(rows_per_wave);
    case 4: return mfma_resident_r<4>(rows_per_wave);
    case 6: return mfma_resident_r<6>(rows_per_wave);
    default: return mfma_resident_r<8>(rows_per_wave);
  }
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.perm) {
    // gather x into the front of the workspace, then the plain GEMV / skinny GEMM
    // (split partials, if any, follow it at a 256-byte boundary)
    uint16_t* xp = static_cast<uint16_t*>(a.workspace);
    const size_t xbytes = ((size_t)a.B * a.K * 2 + 255) / 256 * 256;
    int64_t blocks = ((int64_t)a.B * (a.K / 8) + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(gather_cols_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(a.x), a.B, a.K, a.perm, xp);
    GemmArgs b = a;
    b.x = xp;
    b.perm = nullptr;
    b.workspace = static_cast<unsigned char*>(a.workspace) + xbytes;
    return launch_gemm(b, stream);
  }
  if (a.B <= 16) return launch_gemv(a, stream);
  switch (a.col_tiles) {
    case 2: return launch_mfma_r<2>(a, stream);
    case 3: return launch_mfma_r<3>(a, stream);
    case 4: return launch_mfma_r<4>(a, stream);
    case 6: return launch_mfma_r<6>(a, stream);
    default: return launch_mfma_r<8>(a, stream);
  }
}

}  // namespace q4
