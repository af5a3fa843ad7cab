// Read-rate calibration, used by the benchmark only (librq_calib.so, not part of
// librq's interface). One launch streams the byte ranges that one decode call of
// the compressed cache reads (paper "KV Cache Quantization for Looped
// Transformers with 2-Bit Residuals", §4.1: the kernel reads the compressed KV in
// tiles), split into the same per-(b, h) slots with the same workgroup count,
// with plain non-temporal 16-byte loads and no arithmetic on the data. Its rate
// is the practical ceiling of that traffic pattern on the device: what a decode
// kernel with free arithmetic would reach.
//
//   int rqc_read_slots(const void* const* bufs, const int* bpt, int nbuf, int B,
//                      int H, int T_max, int len, int nsplit, int unit,
//                      unsigned* sink, void* stream)
//
// bufs[k]: device buffer k, token-major [B][H][T_max][bpt[k] bytes] (the layout
// of every codes, metadata and alpha buffer of a contiguous cache), bpt[k] * T_max
// below 2^31; len: cached tokens per sequence (the same for every sequence);
// nsplit, unit: the decode's split plan. Every workgroup streams the rows
// [s c, min((s + 1) c, len)) of its (b, h) in every buffer, c the decode's slot
// length. sink: device memory of at least nsplit*B*H words; nothing is written
// there unless the XOR of a workgroup's data equals a fixed constant (it keeps
// the loads alive). Returns 0, -1 for arguments outside those limits (nothing
// launched), or the launch error.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 16;         // 16-byte loads in flight per lane
constexpr int kMaxBuffers = 24;
constexpr int kAux = 2;             // non-temporal, as the decode's streaming loads

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct CalibParams {
  const uint8_t* buf[kMaxBuffers];
  int bpt[kMaxBuffers];
  int nbuf, B, H, T_max, len, nsplit, unit;
  unsigned* sink;
};

// Each workgroup streams its slot's byte range of every buffer in turn, 64 KB
// per round (16 loads of 16 bytes per lane, all issued before the first is
// used), through a descriptor that covers exactly that range: loads past its
// end return zero without touching memory.
__global__ __launch_bounds__(kThreads) void read_slots(CalibParams p) {
  const int split = blockIdx.x % p.nsplit, bh = blockIdx.x / p.nsplit;
  int c = (p.len + p.nsplit - 1) / p.nsplit;
  c = (c + p.unit - 1) / p.unit * p.unit;
  if (c < p.unit) c = p.unit;
  const int start = min(split * c, p.len), end = min(start + c, p.len);
  const int n = end - start;
  unsigned x = 0;
  for (int k = 0; k < p.nbuf; ++k) {
    const uint32_t bytes = (uint32_t)n * (uint32_t)p.bpt[k];
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p.buf[k] + ((size_t)bh * p.T_max + start) * p.bpt[k]), (short)0, (int)bytes, 0x00020000);
    for (uint32_t base = 0; base < bytes; base += kThreads * 16u * kUnroll) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, base + (threadIdx.x + u * kThreads) * 16u, 0, kAux);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  if (x == 0x9e3779b9u) p.sink[blockIdx.x] = x;
}

}  // namespace

extern "C" int rqc_read_slots(const void* const* bufs, const int* bpt, int nbuf, int B, int H, int T_max, int len,
                              int nsplit, int unit, unsigned* sink, void* stream) {
  if (!bufs || !bpt || !sink || nbuf < 1 || nbuf > kMaxBuffers || B < 1 || H < 1 || T_max < 1 || len < 1 ||
      len > T_max || nsplit < 1 || unit < 1)
    return -1;
  CalibParams p{};
  for (int k = 0; k < nbuf; ++k) {
    if (!bufs[k] || bpt[k] < 1 || (long long)bpt[k] * T_max > 0x7fffffffLL) return -1;
    p.buf[k] = static_cast<const uint8_t*>(bufs[k]);
    p.bpt[k] = bpt[k];
  }
  p.nbuf = nbuf;
  p.B = B;
  p.H = H;
  p.T_max = T_max;
  p.len = len;
  p.nsplit = nsplit;
  p.unit = unit;
  p.sink = sink;
  const long long grid = (long long)nsplit * B * H;
  if (grid > 0x7fffffffLL) return -1;
  hipLaunchKernelGGL(read_slots, dim3((unsigned)grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}
