// MXFP8 block encoding on the device (internal): the E8M0 scale of a block
// and its E4M3FN codes.  The rule (OCP MX format, as applied by the group-aware
// MXFP8 quantisation of the TE dropless-MoE page, "03 Specialised
// optimisations"): X = the smallest integer with amax <= 448 * 2^X, clamped to
// [-127, 127] (-127 for an all-zero block), scale byte X + 127; code = v / 2^X
// rounded to the nearest E4M3FN value, ties to even, sign of zero kept.
#pragma once

#include "moe_internal.h"

namespace moe {

// X from the bits of amax (finite, >= 0): amax = (1 + f) 2^(eb-127) and
// 448 = 1.75 * 2^8, so X = eb - 135 when f <= 0.75, else eb - 134; adding
// 0x1FFFFF to the bits carries into the exponent exactly when f > 0.75.  A
// zero or subnormal amax is first scaled by 2^64 (exact), which makes it
// normal; zero then lands below -127 and clamps there.  Branch-free.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const bool sub = b < 0x800000u;
  const uint32_t u = sub ? __float_as_uint(amax * 18446744073709551616.f) : b;   // amax * 2^64
  const int X = (int)((u + 0x1FFFFFu) >> 23) - (sub ? 135 + 64 : 135);
  return min(max(X, -127), 127);
}

// 32 values -> 32 codes packed into 8 words (element i in byte i%4 of word
// i/4), returns the E8M0 byte.  v / 2^X is exact (ldexp); the hardware
// conversion rounds to the nearest E4M3FN value, ties to even, and keeps the
// sign of zero; |v / 2^X| <= 448 by the choice of X, so nothing overflows.
__device__ __forceinline__ uint32_t mx_quant_block(const float (&v)[32], uint32_t (&packed)[8]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int X = mx_scale_exp(amax);
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * w], -X), ldexpf(v[4 * w + 1], -X), 0, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * w + 2], -X), ldexpf(v[4 * w + 3], -X), word, true);
    packed[w] = (uint32_t)word;
  }
  return (uint32_t)(X + 127);
}

// Four values of one block -> four codes in one word (value i in byte i).
__device__ __forceinline__ uint32_t mx_pack4(float a, float b, float c, float d, int X) {
  int word = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(a, -X), ldexpf(b, -X), 0, false);
  word = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(c, -X), ldexpf(d, -X), word, true);
  return (uint32_t)word;
}

}  // namespace moe
