// Device-side definitions shared by the libq4 kernels (gfx950, wave64).
//
// Packed-code device layout, restated from include/q4.h: a 16-row x 128-channel
// tile is one 1 KiB block; lane l = r + 16*c of a wavefront owns its 16 bytes
// at offset 16*l: four dwords, dword m holding the 8 codes of row r, channels
// 32*m + 8*c + e (e = 0..7). Inside a dword the even e sit in the low 16 bits and
// the odd e in the high 16 bits (nibble e/2, resp. 4 + (e-1)/2), so that
// (dword >> 8*i) & 0x000F000F, i in {0, 1}, and (dword >> 8*i) & 0x00F000F0 are
// half2 pairs (e, e+1) ready for the float16 magic-number conversion below.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTileRows = 16;      // rows per tile (MFMA M)
constexpr int kSuperK = 128;       // input channels per 1 KiB block
constexpr int kBlockK = 32;        // channels per MFMA step (K of 16x16x32)
constexpr int kWave = 64;

// Nibble index inside a dword of the 8-code element e (0..7).
__host__ __device__ constexpr int nibble_of(int e) { return (e & 1) ? 4 + (e >> 1) : (e >> 1); }

__device__ __forceinline__ half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }
__device__ __forceinline__ uint32_t as_u32(half2_t v) { return __builtin_bit_cast(uint32_t, v); }

// Eight 4-bit codes of one dword -> eight float16 values (n - z), exact.
// Each nibble n is OR-ed into the mantissa of 1024.0h (0x6400): the half then
// equals 1024 + n, or 1024 + 16 n for a nibble in bits 4..7 of a half-word.
// One packed add (resp. fma with 1/16) removes the bias and the zero point:
// every intermediate is an integer below 2048, so nothing rounds.
// bias_lo = -(1024 + z), bias_hi = -(64 + z) as half2 pairs (z = 8 for
// symmetric offset-binary codes).
__device__ __forceinline__ half8_t dequant8(uint32_t w, half2_t bias_lo, half2_t bias_hi) {
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t t = w >> 8;
  half2_t p0 = as_half2((w & 0x000F000Fu) | 0x64006400u) + bias_lo;
  half2_t p1 = __builtin_elementwise_fma(as_half2((w & 0x00F000F0u) | 0x64006400u), sixteenth, bias_hi);
  half2_t p2 = as_half2((t & 0x000F000Fu) | 0x64006400u) + bias_lo;
  half2_t p3 = __builtin_elementwise_fma(as_half2((t & 0x00F000F0u) | 0x64006400u), sixteenth, bias_hi);
  half4_t lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  half4_t hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ half8_t as_half8(uint4 v) { return __builtin_bit_cast(half8_t, v); }

// A 32-bit constant held in a VGPR. gfx9 VOP3 encodings take no literal operand,
// so (w & mask) | magic only becomes one v_and_or_b32 when mask and magic are
// registers; the asm is a plain register move the compiler cannot fold back.
__device__ __forceinline__ uint32_t vreg_const(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

// Workgroup barrier for LDS-only communication: waits for this wavefront's LDS
// operations, not for its outstanding global loads. __syncthreads() also waits for
// every vector-memory load in flight (vmcnt(0)), which would drain the prefetched
// weight pipeline at each barrier. The "memory" clobber keeps the compiler from
// moving memory operations across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The magic-number masks of dequant8 as VGPR operands.
struct DequantRegs {
  uint32_t lo, hi, magic;
  __device__ __forceinline__ static DequantRegs make() {
    return DequantRegs{vreg_const(0x000F000Fu), vreg_const(0x00F000F0u), vreg_const(0x64006400u)};
  }
};

// dequant8 with register masks: 1 shift + 4 v_and_or_b32 + 4 packed f16 ops per 8 codes.
__device__ __forceinline__ half8_t dequant8r(uint32_t w, const DequantRegs& k, half2_t bias_lo, half2_t bias_hi) {
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t t = w >> 8;
  half2_t p0 = as_half2((w & k.lo) | k.magic) + bias_lo;
  half2_t p1 = __builtin_elementwise_fma(as_half2((w & k.hi) | k.magic), sixteenth, bias_hi);
  half2_t p2 = as_half2((t & k.lo) | k.magic) + bias_lo;
  half2_t p3 = __builtin_elementwise_fma(as_half2((t & k.hi) | k.magic), sixteenth, bias_hi);
  half4_t lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  half4_t hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Raw magic-number halves of 8 codes for the symmetric GEMV: the MFMA operand
// holds 1024 + n (elements 0, 1, 4, 5) and 1024 + 16 n (elements 2, 3, 6, 7), with
// n = q + 8. The kernel pairs them with x (resp. x/16) and subtracts the bias
// 1032 * sum(x at plain elements) + 1152 * sum(x/16 at scaled elements) from the
// float32 partial sum, which leaves exactly sum(q * x): 1 shift + 4 v_and_or_b32.
__device__ __forceinline__ half8_t magic8r(uint32_t w, const DequantRegs& k) {
  const uint32_t t = w >> 8;
  const half2_t p0 = as_half2((w & k.lo) | k.magic);
  const half2_t p1 = as_half2((w & k.hi) | k.magic);
  const half2_t p2 = as_half2((t & k.lo) | k.magic);
  const half2_t p3 = as_half2((t & k.hi) | k.magic);
  half4_t lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  half4_t hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace q4
