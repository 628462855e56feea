// INT4 group-wise quantization of a KV cache and its dequantization.
//
// Method: "压缩算法" (cs-knowledge-wiki), section 7.4.1.2, quantize_kv_cache_int4: the
// head_dim axis of K or V [batch, heads, seq_len, head_dim] is cut into groups;
// scale = group amax / 7, codes round(x / scale) clamped to [-8, 7], two codes per
// byte. "LLM 后训练量化深度实战…" (www.ybb.press), section 七: the scales must follow
// the tokens they belong to (here one per token, head and group), so a cache can be
// appended one decode step at a time and paged with its scales.
//
// Layout: codes [BH][max_seq][head_dim / 2] bytes, low nibble = even channel, 4-bit
// two's complement; scales [BH][max_seq][head_dim / group] float16. The kernels
// write / read positions pos .. pos + n - 1 of every (batch, head) sequence.
//
// Mapping: one lane per 8 channels of a token (16-byte load, 4-byte store); the
// GL = group / 8 lanes of a group are consecutive and aligned in the wavefront, so
// the group amax is a butterfly over GL lanes. Rounding as the weight quantizer:
// float16 scale fp16(fp32(amax) / 7), the quotient rounded half to even (the IEEE
// float32 quotient's decision, taken without a per-element divide: q4_rtn.h).
#include <algorithm>

#include "q4_device.h"
#include "q4_internal.h"
#include "q4_rtn.h"

namespace q4 {
namespace {

// A persistent grid of resident wavefronts; each walks its 64-chunk pieces with the
// next piece's 16-byte loads in flight while the current one is coded. Chunk c of the
// source is its 8 channels at element 8c (token rows are contiguous); its codes go to
// dword c + (bh * (max_seq - n) + pos) * cpr of the cache, bh = c / (n * cpr).
template <int GL>
__global__ __launch_bounds__(256) void kv_quant_kernel(const uint16_t* __restrict__ src, int n, int d, int64_t max_seq,
                                                       int64_t pos, int64_t chunks, uint32_t* __restrict__ codes,
                                                       uint16_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int cpr = d / 8;  // chunks of 8 channels per token row
  const int64_t per_bh = (int64_t)n * cpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const bool small = chunks <= 0xFFFFFFFFll;
  auto fetch = [&](int64_t base) __attribute__((always_inline)) {
    const int64_t c = base + lane;
    return c < chunks ? *reinterpret_cast<const uint4*>(src + 8 * c) : make_uint4(0u, 0u, 0u, 0u);
  };
  auto code = [&](int64_t base, uint4 raw) __attribute__((always_inline)) {
    const int64_t c = base + lane;
    const half8_t h = as_half8(raw);
    float v[8];
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = (float)h[e];
      a = fmaxf(a, fabsf(v[e]));
    }
#pragma unroll
    for (int m = 1; m < GL; m <<= 1) a = fmaxf(a, __shfl_xor(a, m, 64));
    // fp16(fp32(amax) / 7) through the constant fl(1/7): the same float16 for every
    // float16 amax (checked for all of them on the host)
    const _Float16 s16 = (_Float16)(fmaxf(a, 1e-12f) * (1.0f / 7.0f));
    const float rcp = rtn_recip((float)s16);  // 0 for a zero scale: codes 0
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int q = (int)fminf(fmaxf(rtn_quot(v[e], rcp), -8.0f), 7.0f);
      word |= (uint32_t)(q & 0xF) << (4 * e);
    }
    if (c < chunks) {
      // 32-bit division whenever the indices fit (the usual case)
      const int64_t bh = small ? (int64_t)((uint32_t)c / (uint32_t)per_bh) : c / per_bh;
      const int64_t dc = c + (bh * (max_seq - n) + pos) * cpr;  // chunk index in the cache
      codes[dc] = word;
      if (c % GL == 0) scales[dc / GL] = __builtin_bit_cast(uint16_t, s16);  // first chunk of a group (GL | cpr)
    }
  };
  // wave-uniform loop: every lane of a wavefront takes part in each butterfly
  int64_t base = (int64_t)blockIdx.x * blockDim.x + (threadIdx.x & ~63);
  uint4 cur = base < chunks ? fetch(base) : make_uint4(0u, 0u, 0u, 0u);
  for (; base < chunks; base += stride) {
    const uint4 nxt = base + stride < chunks ? fetch(base + stride) : make_uint4(0u, 0u, 0u, 0u);
    code(base, cur);
    cur = nxt;
  }
}

__global__ void kv_dequant_kernel(const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales, int n,
                                  int d, int GL, int64_t max_seq, int64_t pos, int64_t chunks,
                                  uint16_t* __restrict__ dst) {
  const int cpr = d / 8;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks; c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = c / cpr;
    const int e8 = (int)(c - r * cpr);
    const int64_t bh = r / n, t = r - bh * n;
    const int64_t drow = bh * max_seq + pos + t;
    const uint32_t word = codes[drow * cpr + e8];
    const float sf = (float)__builtin_bit_cast(_Float16, scales[drow * (cpr / GL) + e8 / GL]);
    half8_t h;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int q = (int)((word >> (4 * e)) & 0xF) - (int)((word >> (4 * e)) & 0x8) * 2;  // sign-extend the nibble
      h[e] = (_Float16)((float)q * sf);  // exact float32 product, one rounding to float16
    }
    *reinterpret_cast<uint4*>(dst + r * d + 8 * e8) = __builtin_bit_cast(uint4, h);
  }
}

inline int grid_for(int64_t work, int block) {
  int64_t g = (work + block - 1) / block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

hipError_t launch_kv_quantize(const KvArgs& a, hipStream_t stream) {
  const int64_t chunks = a.bh * a.n * (a.d / 8);
  const int block = 256;
  const void* fn = a.group == 32 ? reinterpret_cast<const void*>(&kv_quant_kernel<4>)
                   : a.group == 64 ? reinterpret_cast<const void*>(&kv_quant_kernel<8>)
                                   : reinterpret_cast<const void*>(&kv_quant_kernel<16>);
  const int grid = std::min(grid_for(chunks, block), resident_grid(fn, block));  // resident workgroups at most
  const uint16_t* src = static_cast<const uint16_t*>(a.src);
  uint32_t* codes = static_cast<uint32_t*>(a.codes);
  uint16_t* sc = static_cast<uint16_t*>(a.scales);
  switch (a.group) {
    case 32: hipLaunchKernelGGL(kv_quant_kernel<4>, dim3(grid), dim3(block), 0, stream, src, (int)a.n, a.d, a.max_seq, a.pos, chunks, codes, sc); break;
    case 64: hipLaunchKernelGGL(kv_quant_kernel<8>, dim3(grid), dim3(block), 0, stream, src, (int)a.n, a.d, a.max_seq, a.pos, chunks, codes, sc); break;
    default: hipLaunchKernelGGL(kv_quant_kernel<16>, dim3(grid), dim3(block), 0, stream, src, (int)a.n, a.d, a.max_seq, a.pos, chunks, codes, sc); break;
  }
  return hipGetLastError();
}

hipError_t launch_kv_dequant(const KvArgs& a, hipStream_t stream) {
  const int64_t chunks = a.bh * a.n * (a.d / 8);
  const int block = 256;
  hipLaunchKernelGGL(kv_dequant_kernel, dim3(grid_for(chunks, block)), dim3(block), 0, stream,
                     static_cast<const uint32_t*>(a.codes), static_cast<const uint16_t*>(a.scales), (int)a.n, a.d,
                     a.group / 8, a.max_seq, a.pos, chunks, static_cast<uint16_t*>(a.dst));
  return hipGetLastError();
}

}  // namespace q4
