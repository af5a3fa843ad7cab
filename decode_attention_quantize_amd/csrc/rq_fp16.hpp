// binary64 -> binary16 rounding of librq's append kernels (the fp16 offsets,
// scales and LS coefficients of the cache: paper "KV Cache Quantization for
// Looped Transformers with 2-Bit Residuals", §2.1 and §3.2), branch-free so
// that a wave executes one path whatever its lanes hold.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rq {

enum : int { kRoundNearest = 0, kRoundDown = 1, kRoundUp = 2 };  // to nearest-even, toward -inf, toward +inf

// The magnitude M 2^(E - 52) is cut at the fp16 spacing 2^q of its binade
// (q = E - 10, or -24 below the normal range); the bits cut off decide the
// rounding. A magnitude below half the smallest spacing has a shift of 64 or
// more: clamping it to 63 leaves n = 0 and the whole mantissa as remainder,
// which is still below half a spacing. Overflow gives infinity, or 65504
// when rounding toward zero.
template <int MODE>
__host__ __device__ __forceinline__ uint16_t f64_to_f16(double x) {
  const uint64_t bits = __builtin_bit_cast(uint64_t, x);
  const bool neg = (bits >> 63) != 0;
  const uint32_t sign = neg ? 0x8000u : 0u;
  const int e = (int)((bits >> 52) & 0x7ff);
  const uint64_t frac = bits & 0xFFFFFFFFFFFFFull;
  const int E = (e == 0 ? 1 : e) - 1023;
  const uint64_t M = e == 0 ? frac : (frac | (1ull << 52));
  const bool sub = E < -14;                      // fp16 subnormal range
  const int q = sub ? -24 : E - 10;
  int shift = q - (E - 52);                      // >= 42
  shift = shift > 63 ? 63 : shift;
  uint64_t n = M >> shift;
  const uint64_t rem = M & ((1ull << shift) - 1ull);
  const uint64_t half = 1ull << (shift - 1);
  bool up;
  if constexpr (MODE == kRoundNearest) up = rem > half || (rem == half && (n & 1ull));
  else if constexpr (MODE == kRoundDown) up = neg && rem != 0;
  else up = !neg && rem != 0;
  n += up ? 1ull : 0ull;
  const bool carry = !sub && n == 2048;          // rounded up into the next binade
  const int EE = E + (carry ? 1 : 0);
  const uint32_t nn = carry ? 1024u : (uint32_t)n;
  const bool toward_zero = (MODE == kRoundDown && !neg) || (MODE == kRoundUp && neg);
  uint32_t mag = sub ? nn : ((uint32_t)(EE + 15) << 10) | (nn - 1024u);   // sub: n <= 1024 (1024 = 2^-14)
  mag = (!sub && EE > 15) ? (toward_zero ? 0x7bffu : 0x7c00u) : mag;
  mag = e == 0x7ff ? (frac ? 0x7e00u : 0x7c00u) : mag;
  return (uint16_t)(sign | mag);
}

}  // namespace rq
