// FP8 (OCP e4m3) encoder shared by the FP8 cache write and the decode
// kernel's one-call append over FP8 pools, so both store the same codes.
// Rounds a float32 to the nearest e4m3 value, ties to the even code,
// saturating at +-448 (infinities too); NaN stays NaN (S.1111.111).
// Normal codes cover |x| >= 2^-6 (exponent bias 7); below that the step is
// 2^-9 (subnormals m/8 * 2^-6). The pages fix no FP8 format; this is the one
// gfx950 decodes natively.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace pkv {

__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t mag = b & 0x7fffffffu;
  if (mag > 0x7f800000u) return sign | 0x7fu;   // NaN
  if (mag >= 0x43e00000u) return sign | 0x7eu;  // |x| >= 448 (infinity too): saturate
  const int e = (int)(mag >> 23);               // biased float32 exponent
  const uint32_t m = mag & 0x7fffffu;
  if (e >= 121) {                               // |x| >= 2^-6: normal e4m3
    uint32_t r = m >> 20;
    const uint32_t rem = m & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
    const uint32_t code = ((uint32_t)(e - 120) << 3) + r;  // r == 8 carries into the exponent
    return sign | (code > 0x7eu ? 0x7eu : code);
  }
  // below 2^-6: a multiple of the subnormal step 2^-9, |x| / 2^-9 = sig * 2^(e - 141)
  const int sh = 141 - e;                       // >= 21
  if (e == 0 || sh > 25) return sign;           // below half a step: zero
  const uint32_t sig = (1u << 23) | m;
  uint32_t q = sig >> sh;
  const uint32_t rem = sig & ((1u << sh) - 1u), half = 1u << (sh - 1);
  if (rem > half || (rem == half && (q & 1u))) ++q;
  return sign | q;                              // 0 .. 8 (8 is the smallest normal, 0x08)
}

}  // namespace pkv
