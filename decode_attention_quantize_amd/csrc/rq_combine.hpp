// Split partials and the cross-split combine shared by the decode kernels
// (paper "KV Cache Quantization for Looped Transformers with 2-Bit Residuals",
// §4.2 "Decode": past and current token merged through their softmax
// statistics; App. G.2: one inverse value rotation per (b, h)).
//
// A decode workgroup merges its waves into one partial (m, l, acc[D]) of its
// token range and stores it; a second kernel launch (rq_combine) merges the
// partials of each (b, h) with the current token. The kernel boundary makes
// the partials visible across the chip's L2 slices without device-scope
// fences inside the streaming kernel.
#pragma once

#include "rq_device.hpp"
#include "rq_internal.hpp"

namespace rq {

struct PartialLds {
  float wm[kWaves];
  float wl[kWaves];
};

// val: this lane's E values of column block `cb` for token slot `slot` (lanes
// i*CPR + cb hold slot i); lane_l: the lane's probability sum, counted in one
// lane per slot; m_wave: the wave's running max (log2 domain).
template <int D, int E, int CPR, int SLOTS>
__device__ __forceinline__ void write_partial(const float (&val)[E], float lane_l, float m_wave, bool lane_on,
                                              float (*red)[64][E + 1], PartialLds& S, float* dst) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, tid = threadIdx.x;
#pragma unroll
  for (int e = 0; e < E; ++e) red[wave][lane][e] = lane_on ? val[e] : 0.0f;
  const float lw = wave_sum(lane_l);
  if (lane == 0) {
    S.wm[wave] = m_wave;
    S.wl[wave] = lw;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, S.wm[w]);
  if (tid < D) {
    const int c = tid / E, e = tid % E;
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = (S.wm[w] == -INFINITY) ? 0.0f : exp2f(S.wm[w] - M);
      float sw = 0.0f;
      for (int i = 0; i < SLOTS; ++i) sw += red[w][i * CPR + c][e];
      s = fmaf(f, sw, s);
    }
    dst[4 + tid] = s;
  }
  if (tid == 0) {
    float l = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) l += (S.wm[w] == -INFINITY) ? 0.0f : S.wl[w] * exp2f(S.wm[w] - M);
    dst[0] = M;
    dst[1] = l;
  }
}

}  // namespace rq
