// BF16 decode-attention baseline: split-K flash decoding over an uncompressed
// bf16 K/V cache, the comparison point of the paper "KV Cache Quantization for
// Looped Transformers with 2-Bit Residuals" (§5.3 Throughput Improvement). It
// writes the same per-split partials as the compressed kernel and shares its
// combine (with no inverse rotation).
//
// A lane owns 8 channels (16 bytes) of one token row; CPT = D/8 lanes cover a
// row and a wave covers 64/CPT tokens per step, UNR steps per iteration so that
// every lane has 2*UNR independent 16-byte loads in flight.
#include <hip/hip_runtime.h>

#include "rq_device.hpp"
#include "rq_internal.hpp"

namespace rq {
namespace {

template <int D>
__global__ __launch_bounds__(kThreads) void bf16_main(Bf16Params p) {
  constexpr int CPT = D / 8;
  constexpr int TPW = 64 / CPT;
  constexpr int UNR = 4;
  constexpr int TILE = TPW * UNR;
  __shared__ float red[kWaves][64][9];
  __shared__ float wm[kWaves], wl[kWaves];

  const int split = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.H;
  int len = p.past_len[b];
  len = len < 0 ? 0 : (len > p.T_max ? p.T_max : len);
  const int start = split * p.chunk;
  const int end = min(start + p.chunk, len);
  if (start >= end) return;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ts = lane / CPT, ch = lane % CPT;
  const bool lane_on = ts < TPW;
  const int chs = lane_on ? ch : 0;

  float q[8];
  {
    const uint4 qv = *reinterpret_cast<const uint4*>(p.q + (size_t)bh * D + 8 * chs);
    const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[2 * i] = bf16lo(w[i]) * p.scale_log2;
      q[2 * i + 1] = bf16hi(w[i]) * p.scale_log2;
    }
  }
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  float lsum = 0.0f, m = -INFINITY;
  const size_t rowbase = (size_t)bh * p.T_max;

  for (int base = start + wave * TILE; base < end; base += kWaves * TILE) {
    uint4 kr[UNR], vr[UNR];
    bool ok[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int t = base + u * TPW + ts;
      ok[u] = lane_on && t < end;
      const size_t row = rowbase + min(t, p.T_max - 1);
      kr[u] = *reinterpret_cast<const uint4*>(p.k + row * D + 8 * chs);
      vr[u] = *reinterpret_cast<const uint4*>(p.v + row * D + 8 * chs);
    }
    float s[UNR];
    float tmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const uint32_t w[4] = {kr[u].x, kr[u].y, kr[u].z, kr[u].w};
      float d = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d = fmaf(q[2 * i], bf16lo(w[i]), d);
        d = fmaf(q[2 * i + 1], bf16hi(w[i]), d);
      }
      d = group_sum<CPT>(d);
      s[u] = ok[u] ? d : -INFINITY;
      tmax = fmaxf(tmax, s[u]);
    }
    tmax = wave_max(tmax);
    if (tmax == -INFINITY) continue;
    if (tmax > m) {
      const float f = exp2f(m - tmax);
      m = tmax;
      lsum *= f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= f;
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const float pu = ok[u] ? exp2f(s[u] - m) : 0.0f;
      lsum += pu;
      const uint32_t w[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(pu, bf16lo(w[i]), acc[2 * i]);
        acc[2 * i + 1] = fmaf(pu, bf16hi(w[i]), acc[2 * i + 1]);
      }
    }
  }

#pragma unroll
  for (int e = 0; e < 8; ++e) red[wave][lane][e] = lane_on ? acc[e] : 0.0f;
  const float lw = wave_sum((lane_on && ch == 0) ? lsum : 0.0f);
  if (lane == 0) {
    wm[wave] = m;
    wl[wave] = lw;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wm[w]);
  float f[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) f[w] = (wm[w] == -INFINITY) ? 0.0f : exp2f(wm[w] - M);
  float* dst = p.part + ((size_t)bh * p.nsplit + split) * part_floats(D);
  const int d = threadIdx.x;
  if (d < D) {
    const int c = d / 8, e = d % 8;
    float sacc = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      float sw = 0.0f;
      for (int i = 0; i < TPW; ++i) sw += red[w][i * CPT + c][e];
      sacc = fmaf(f[w], sw, sacc);
    }
    dst[4 + d] = sacc;
  }
  if (d == 0) {
    float l = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) l = fmaf(f[w], wl[w], l);
    dst[0] = M;
    dst[1] = l;
  }
}

}  // namespace

int launch_bf16_main(const Bf16Params& p, int D, void* stream) {
  const dim3 grid((unsigned)p.nsplit, (unsigned)(p.B * p.H));
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (D) {
    case 64: hipLaunchKernelGGL(bf16_main<64>, grid, dim3(kThreads), 0, s, p); break;
    case 96: hipLaunchKernelGGL(bf16_main<96>, grid, dim3(kThreads), 0, s, p); break;
    case 128: hipLaunchKernelGGL(bf16_main<128>, grid, dim3(kThreads), 0, s, p); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

}  // namespace rq
