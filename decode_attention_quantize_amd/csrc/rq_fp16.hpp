// binary64 -> binary16 rounding of librq's append kernels (the fp16 offsets,
// scales and LS coefficients of the cache: paper "KV Cache Quantization for
// Looped Transformers with 2-Bit Residuals", §2.1 and §3.2), in the hardware
// conversions plus one correction per step, with no branches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rq {

enum : int { kRoundNearest = 0, kRoundDown = 1, kRoundUp = 2 };  // to nearest-even, toward -inf, toward +inf

// Two conversions, binary64 -> binary32 -> binary16, each at nearest-even in
// hardware (IEEE subnormals in both formats) and then corrected:
//  - toward -inf / +inf: a result on the wrong side of its input moves one step
//    (an integer step of the bit pattern) back past it. Directed roundings
//    compose, RD16(RD32(x)) = RD16(x), so the two steps give the one rounding;
//    overflow gives infinity, or 65504 when rounding toward zero.
//  - nearest: the first step rounds to odd (toward zero, then the last bit set
//    if inexact). binary32 carries 13 more bits than binary16, enough for the
//    second rounding to nearest-even to equal the direct one (no double
//    rounding).
// Inputs are finite. Equal, bit for bit, to a direct rounding of x (checked
// against an integer-only encoder over every binary16 value, its neighbours
// and midpoints, and tens of millions of random binary64 values).
template <int MODE>
__host__ __device__ __forceinline__ uint16_t f64_to_f16(double x) {
  float f = (float)x;
  const double fd = (double)f;
  uint32_t fb = __builtin_bit_cast(uint32_t, f);
  const bool neg = (fb >> 31) != 0;  // x's sign (f keeps it, zeros included)
  if constexpr (MODE == kRoundDown) {
    fb = fd > x ? (neg ? fb + 1u : fb - 1u) : fb;
  } else if constexpr (MODE == kRoundUp) {
    fb = fd < x ? (neg ? fb - 1u : fb + 1u) : fb;
  } else {
    fb = __builtin_fabs(fd) > __builtin_fabs(x) ? fb - 1u : fb;
    fb |= ((double)__builtin_bit_cast(float, fb) != x) ? 1u : 0u;
  }
  f = __builtin_bit_cast(float, fb);
  const _Float16 hh = (_Float16)f;
  uint16_t h = __builtin_bit_cast(uint16_t, hh);
  if constexpr (MODE == kRoundDown) {
    h = (float)hh > f ? (uint16_t)((h & 0x8000) ? h + 1 : h - 1) : h;
  } else if constexpr (MODE == kRoundUp) {
    h = (float)hh < f ? (uint16_t)((h & 0x8000) ? h - 1 : h + 1) : h;
  }
  return h;
}

}  // namespace rq
