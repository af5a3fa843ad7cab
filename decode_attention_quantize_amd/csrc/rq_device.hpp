// Small device helpers shared by the decode kernels of librq (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rq {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

// v_dot2c_f32_f16: c + a.lo * b.lo + a.hi * b.hi (fp16 inputs, fp32 accumulate).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b), c, false);
}
__device__ __forceinline__ float f16lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
__device__ __forceinline__ float f16u(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  h2_t v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Sum over the G consecutive lanes G*i .. G*i+G-1 (every lane gets the sum).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (G == 1) {
    return x;
  } else if constexpr ((G & (G - 1)) == 0) {
#pragma unroll
    for (int m = 1; m < G; m <<= 1) x += __shfl_xor(x, m, 64);
    return x;
  } else {
    const int lane = threadIdx.x & 63;
    const int base = lane - lane % G;
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < G; ++j) s += __shfl(x, base + j, 64);
    return s;
  }
}

// Work item of this workgroup in a 1-D grid of nsplit * B * H workgroups.
// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs, each
// with its own L2; the ids are remapped so that every XCD receives one
// contiguous, head-major range of items (h, b, split), and a head's rotation
// is fetched into few L2s.
constexpr int kXcds = 8;
__device__ __forceinline__ void split_item(int nsplit, int B, int H, int& split, int& b, int& h) {
  const int i = (int)blockIdx.x, total = nsplit * B * H;
  const int k = (total % kXcds == 0) ? (i % kXcds) * (total / kXcds) + i / kXcds : i;
  split = k % nsplit;
  const int rest = k / nsplit;
  b = rest % B;
  h = rest / B;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

}  // namespace rq
