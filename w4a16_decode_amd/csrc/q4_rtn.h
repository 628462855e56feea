// Round-to-nearest code decision without a per-element divide.
//
// The quantizers round the quotient of a float16 weight w by a float16 scale s half
// to even ("LLM 后训练量化深度实战…", www.ybb.press, section 二: q = round(w / scale);
// for w8: "量化：PTQ、GPTQ、AWQ 与 SmoothQuant", charles2530.github.io, the closing
// quick code example). Taking the IEEE float32 quotient and rounding it gives the same
// code as rounding the exact rational w / s, and that is what these helpers compute,
// with one hardware reciprocal per scale and a multiply per element:
//
//  * Gap. w and s are integer multiples of 2^-24 with 11-bit significands. For a
//    half-integer h, w / s - h = (2w - (2k+1)s) / (2s); if the numerator is not 0
//    it is at least ulp(s) in magnitude when w's exponent is at least s's minus 1,
//    which gives |w / s - h| >= 1 / (2 m_s) >= 1/4094 (m_s < 2048 the significand
//    of s); and when w's exponent is smaller, |w / s| <= 1/2 - 2^-12. So a quotient
//    that is not exactly a half-integer stays at least 2^-12 away from every one.
//  * Error. r = v_rcp_f32(s) is within one ulp of 1 / s (relative 2^-23; s is a
//    normal float32, 1 / s too), and t = fl(w * r) adds a rounding of relative size
//    2^-24, so t differs from w / s by at most |w / s| * 1.5 * 2^-23 (plus a term of
//    order 2^-47), i.e. below 2^-14 for |w / s| < 341.
//  * Decision. If t lies within 2^-14 of the half-integer h = floor(t) + 1/2, the
//    exact quotient is within 2^-13 < 2^-12 of h, hence equal to h, and rint(h)
//    rounds the tie to even. Otherwise t and w / s lie strictly on the same side of
//    every half-integer, and rint(t) is the code. Both branches are exact for
//    |w / s| < 341, which covers every clamp range used (|q| <= 127); beyond it the
//    result is still at least 340 in magnitude and clamps the same way. The test
//    |t - h| < 2^-14 holds whether the compiler rounds t first or fuses w * r - h
//    into one FMA (the fused form only has the smaller error).
//  * s == 0 gives r = 0 and hence the code 0 that the quantizers assign to a zero
//    scale, without a per-element branch.
#pragma once

#include <hip/hip_runtime.h>

namespace q4 {

// Reciprocal of a scale (float16 value held in a float): v_rcp_f32, within one ulp
// of 1 / s, or 0 for s == 0.
__device__ __forceinline__ float rtn_recip(float s) { return s == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(s); }

// rint(w / s) half to even, exactly, for float16-valued w and s with r = rtn_recip(s).
__device__ __forceinline__ float rtn_quot(float w, float r) {
  const float t = w * r;
  const float h = floorf(t) + 0.5f;
  return rintf(fabsf(t - h) < 0x1p-14f ? h : t);
}

}  // namespace q4
