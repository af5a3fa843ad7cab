// BF16 decode-attention baseline: split-K flash decoding over an uncompressed
// bf16 K/V cache, the comparison point of the paper "KV Cache Quantization for
// Looped Transformers with 2-Bit Residuals" (§5.3 Throughput Improvement). It
// writes the same split partials as the compressed kernel and shares its
// combine (without a value rotation).
//
// A lane owns 8 channels (16 bytes) of one token row; CPT = D/8 lanes cover a
// row and a wave covers 64/CPT tokens per step, UNR steps per iteration, and
// the next iteration's rows are loaded while the current ones are processed.
#include <hip/hip_runtime.h>

#include "rq_combine.hpp"
#include "rq_device.hpp"
#include "rq_internal.hpp"

namespace rq {
namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// 16-byte streaming load of cache rows, non-temporal: each row is read once
// per call (as in the compressed kernel).
__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int D>
__global__ __launch_bounds__(kThreads) void bf16_fused(Bf16Params p) {
  constexpr int CPT = D / 8;
  constexpr int TPW = 64 / CPT;
  constexpr int UNR = 4;
  constexpr int TILE = TPW * UNR;
  __shared__ float red[kWaves][64][9];
  __shared__ PartialLds S;

  int split, b, h;
  split_item(p.nsplit, p.B, p.H, split, b, h);
  const int bh = b * p.H + h;
  int len = p.past_len[b];
  len = len < 0 ? 0 : (len > p.T_max ? p.T_max : len);
  if (split >= slots_used(len, p.nsplit, p.unit)) return;  // whole block, before any barrier
  const int chunk = slot_len(len, p.nsplit, p.unit);
  const int start = split * chunk;
  const int end = min(start + chunk, len);

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

  const int last = end > 0 ? end - 1 : 0;
  auto load = [&](int base, uint4 (&kr)[UNR], uint4 (&vr)[UNR]) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const size_t row = rowbase + min(base + u * TPW + ts, last);  // clamped rows are masked
      kr[u] = ld16(p.k + row * D + 8 * chs);
      vr[u] = ld16(p.v + row * D + 8 * chs);
    }
  };

  int base = start + wave * TILE;
  uint4 kr[UNR], vr[UNR];
  if (base < end) load(base, kr, vr);
  while (base < end) {
    const int nb = base + kWaves * TILE;
    uint4 kn[UNR], vn[UNR];
    load(nb, kn, vn);  // unconditional prefetch (clamped rows on the last pass)
    float s[UNR];
    bool ok[UNR];
    float tmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      ok[u] = lane_on && base + u * TPW + ts < end;
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
    tmax = wave_max_uniform(tmax);
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
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      kr[u] = kn[u];
      vr[u] = vn[u];
    }
    base = nb;
  }
  write_partial<D, 8, CPT, TPW>(acc, (lane_on && ch == 0) ? lsum : 0.0f, m, lane_on, red, S,
                                p.part + ((size_t)bh * p.nsplit + split) * part_floats(D));
}

}  // namespace

int launch_bf16(const Bf16Params& p, int D, int nsplit, void* stream) {
  const dim3 grid((unsigned)(nsplit * p.B * p.H));
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (D) {
    case 64: hipLaunchKernelGGL(bf16_fused<64>, grid, dim3(kThreads), 0, s, p); break;
    case 96: hipLaunchKernelGGL(bf16_fused<96>, grid, dim3(kThreads), 0, s, p); break;
    case 128: hipLaunchKernelGGL(bf16_fused<128>, grid, dim3(kThreads), 0, s, p); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

}  // namespace rq
