// E4M3 / E8M0 encoding of one MXFP8 block on the device (shared by the quantisers and by
// the GEMM epilogues that write an MXFP8 copy of their output).
//
// Scale: the smallest 2^s with amax * 2^-s <= 448 (E4M3's largest finite value), s clamped
// to [-127, 127]; blocks whose amax is zero or an fp32 subnormal get -127.  Elements:
// v * 2^-s (exact in fp32) rounded to nearest-even onto the E4M3 grid by gfx950's packed
// fp8 conversion, two elements per instruction.
#pragma once
#include "common.h"

namespace moe {

__device__ __forceinline__ int mx_scale_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int eb = (int)((u >> 23) & 0xff);
  if (eb == 0) return -127;
  int s = eb - 127 - 8 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);  // mantissa above 1.75 -> next power
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// Four values of magnitude <= 448 -> four E4M3 codes (bytes 0..3), round to nearest even.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

__device__ __forceinline__ float exp2i(int s) { return __uint_as_float((uint32_t)(s + 127) << 23); }  // 2^s, s in [-126,127]

// 2^-s as one fp32 factor.  Finite bf16 input has amax < 2^128, so s <= 120 and the factor
// is a normal number; v * 2^-s is exact unless it falls below 2^-126, where its code is
// zero either way.
__device__ __forceinline__ float mx_inv_scale(int s) { return exp2i(-s); }

}  // namespace moe
