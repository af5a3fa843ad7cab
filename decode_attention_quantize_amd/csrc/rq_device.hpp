// Small device helpers shared by the decode kernels of librq (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rq {

__device__ __forceinline__ float f16lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
__device__ __forceinline__ float f16u(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// DPP lane moves (gfx9 data-parallel primitives) on float values.
enum : int {
  kQuadSwap1 = 0xB1,      // quad_perm [1,0,3,2]: lane ^ 1
  kQuadSwap2 = 0x4E,      // quad_perm [2,3,0,1]: lane ^ 2
  kRowHalfMirror = 0x141, // lane i <- 7 - i within each 8 lanes
  kRowMirror = 0x140,     // lane i <- 15 - i within each 16-lane row
  kRowBcast15 = 0x142,    // lane 15 of row r -> every lane of row r + 1
  kRowBcast31 = 0x143,    // lane 31 -> every lane of rows 2 and 3
};
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float x) {
  const int v = __builtin_bit_cast(int, x);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xF, false));
}

// Sum over the G consecutive lanes G*i .. G*i+G-1 (every lane gets the sum).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (G == 1) {
    return x;
  } else if constexpr (G == 2) {
    return x + dpp<kQuadSwap1>(x);
  } else if constexpr (G == 4) {
    x += dpp<kQuadSwap1>(x);
    return x + dpp<kQuadSwap2>(x);
  } else if constexpr (G == 8) {
    x += dpp<kQuadSwap1>(x);
    x += dpp<kQuadSwap2>(x);
    return x + dpp<kRowHalfMirror>(x);
  } else if constexpr (G == 16) {
    x += dpp<kQuadSwap1>(x);
    x += dpp<kQuadSwap2>(x);
    x += dpp<kRowHalfMirror>(x);
    return x + dpp<kRowMirror>(x);
  } else {
    const int lane = threadIdx.x & 63;
    const int base = lane - lane % G;
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < G; ++j) s += __shfl(x, base + j, 64);
    return s;
  }
}

// Maximum over the wave, returned wave-uniform (from lane 63).
__device__ __forceinline__ float wave_max_uniform(float x) {
  x = fmaxf(x, dpp<kQuadSwap1>(x));
  x = fmaxf(x, dpp<kQuadSwap2>(x));
  x = fmaxf(x, dpp<kRowHalfMirror>(x));
  x = fmaxf(x, dpp<kRowMirror>(x));
  x = fmaxf(x, dpp<kRowBcast15, 0xA>(x));
  x = fmaxf(x, dpp<kRowBcast31, 0xC>(x));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
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

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

}  // namespace rq
