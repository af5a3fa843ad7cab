// Fused dequantize + split-K decode attention over the ResidualQuant cache
// (paper "KV Cache Quantization for Looped Transformers with 2-Bit Residuals":
// §4.1 kernel, §4.2 "Decode" past/current merge, App. G.2 "Reconstruction and
// attention"), plus the query preparation and the cross-split combine that the
// BF16 baseline shares.
//
// Per (b, h) the attended keys are zhat_t = sum_c beta_{c,t} D(c_{c,t}) in the
// rotated domain, with components c = anchor, residual (Last-loop) or the
// chain anchor, residual 2, .., residual r (Previous-loop), and
// beta_{c,t} = prod_{j>c} alpha_{j,t} (so the last component has weight 1).
// With the rotation folded into the query (q' = H_K q) the score is
//   s_t = sum_c beta_{c,t} sum_groups [ s_{c,g} (q'_g . code_{c,g}) + o_{c,g} sum(q'_g) ],
// and values accumulate sum_t p_t zhat_V,t in the rotated domain with the same
// per-group split into a code part (weight p beta s) and an offset part
// (p beta o); H_V^T is applied once in the combine.
//
// Code unpacking: a masked code field read as an fp16 bit pattern is the
// subnormal number code * 2^(shift - 24), exactly, and v_dot2c_f32_f16 keeps
// fp16 subnormals, so one AND yields two codes ready for the dot product.
// The packed layout places group elements e and e+16 at the same bit offset of
// the low and high halves of a word, which is what makes one mask yield a pair.
#include <hip/hip_runtime.h>

#include "rq_device.hpp"
#include "rq_internal.hpp"

namespace rq {
namespace {

constexpr float kTwo24 = 16777216.0f;
constexpr float kWScale = 64.0f;              // value weights are stored as fp16(2^6 p beta s)
constexpr float kMinNormal = 6.103515625e-05f;  // smallest normal fp16, 2^-14

// ---------------------------------------------------------------- query prep
template <int D>
__global__ __launch_bounds__(D) void qprep_kernel(QPrepParams p) {
  constexpr int G = D / 32;
  __shared__ float qs[D];
  __shared__ float qr[D];
  const int bh = blockIdx.x, h = bh % p.H, i = threadIdx.x;
  qs[i] = bf16f(p.q[(size_t)bh * D + i]);
  __syncthreads();
  const float* row = p.rotk + ((size_t)h * D + i) * D;
  float acc = 0.0f;
  for (int j = 0; j < D; ++j) acc = fmaf(row[j], qs[j], acc);
  qr[i] = acc * p.scale_log2;
  __syncthreads();
  uint32_t* out = p.qprep + (size_t)bh * qprep_words(D);
  if (i < D / 2) {
    const int gi = i / 16, k = i % 16;
    const float a = qr[32 * gi + k], c = qr[32 * gi + 16 + k];
    const _Float16 ah = (_Float16)a, ch = (_Float16)c;
    out[gi * 33 + k] = pack_h2((float)ah, (float)ch);
    out[gi * 33 + 16 + k] = pack_h2(a - (float)ah, c - (float)ch);
  }
  if (i < G) {
    float s = 0.0f;
    for (int e = 0; e < 32; ++e) s += qr[32 * i + e];
    out[i * 33 + 32] = __float_as_uint(s);
  }
}

// ---------------------------------------------------------------- main kernel
template <int BITS>
struct Words {
  uint32_t w[BITS];  // one group of 32 codes = BITS 32-bit words
};

template <int BITS>
__device__ __forceinline__ Words<BITS> load_group(const uint8_t* base) {
  Words<BITS> r;
  if constexpr (BITS == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(base);
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(base);
    r.w[0] = v.x; r.w[1] = v.y;
  }
  return r;
}

// sum_e q'_e code_e over one group (q' as hi [+ lo] fp16 pairs (e, e+16)).
template <int BITS, bool HILO>
__device__ __forceinline__ float kdot(const Words<BITS>& c, const uint32_t (&QH)[16], const uint32_t (&QL)[16]) {
  if constexpr (BITS == 4) {
    float a1 = 0.0f, a16 = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x = c.w[j], y = x >> 8;
      const uint32_t m0 = x & 0x000F000Fu, m1 = x & 0x00F000F0u, m2 = y & 0x000F000Fu, m3 = y & 0x00F000F0u;
      a1 = dot2(m0, QH[4 * j], a1);
      a16 = dot2(m1, QH[4 * j + 1], a16);
      a1 = dot2(m2, QH[4 * j + 2], a1);
      a16 = dot2(m3, QH[4 * j + 3], a16);
      if constexpr (HILO) {
        a1 = dot2(m0, QL[4 * j], a1);
        a16 = dot2(m1, QL[4 * j + 1], a16);
        a1 = dot2(m2, QL[4 * j + 2], a1);
        a16 = dot2(m3, QL[4 * j + 3], a16);
      }
    }
    return fmaf(a16, 1.0f / 16.0f, a1);
  } else {
    float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t x = c.w[j], y = x >> 8;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t mx = x & (0x00030003u << (2 * q)), my = y & (0x00030003u << (2 * q));
        a[q] = dot2(mx, QH[8 * j + q], a[q]);
        a[q] = dot2(my, QH[8 * j + 4 + q], a[q]);
        if constexpr (HILO) {
          a[q] = dot2(mx, QL[8 * j + q], a[q]);
          a[q] = dot2(my, QL[8 * j + 4 + q], a[q]);
        }
      }
    }
    return a[0] + a[1] * 0.25f + a[2] * (1.0f / 16.0f) + a[3] * (1.0f / 64.0f);
  }
}

// acc[e] += w_t0 code_{t0,e} + w_t1 code_{t1,e} for the 32 elements of a group.
// Element e of the group lands in accumulator e with an extra factor 2^shift(e)
// (its field offset inside the selected byte), removed at the end.
template <int BITS>
__device__ __forceinline__ void vacc(const Words<BITS>& c0, const Words<BITS>& c1, uint32_t W, float (&acc)[32]) {
#pragma unroll
  for (int j = 0; j < BITS; ++j) {
#pragma unroll
    for (int by = 0; by < 4; ++by) {
      // [t0 byte `by`, 0, t1 byte `by`, 0]
      const uint32_t sel = 0x0c000c00u | ((uint32_t)(4 + by) << 16) | (uint32_t)by;
      const uint32_t x = __builtin_amdgcn_perm(c1.w[j], c0.w[j], sel);
      const int half = by >> 1, hb = by & 1;
      if constexpr (BITS == 4) {
        const int e = 16 * half + 4 * j + 2 * hb;
        acc[e] = dot2(x & 0x000F000Fu, W, acc[e]);
        acc[e + 1] = dot2(x & 0x00F000F0u, W, acc[e + 1]);
      } else {
        const int e = 16 * half + 8 * j + 4 * hb;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[e + q] = dot2(x & (0x00030003u << (2 * q)), W, acc[e + q]);
      }
    }
  }
}

// 2^shift of element e's field in the byte vacc() selected.
template <int BITS>
__device__ __forceinline__ float vclass(int e) {
  const int k = e & 15;
  if constexpr (BITS == 4) return (k & 1) ? 16.0f : 1.0f;
  else return (float)(1 << (2 * (k & 3)));
}

template <uint32_t CB, int c>
constexpr int cbits() {
  return (int)((CB >> (4 * c)) & 0xF);
}

// Per-component tile data of one lane: codes of tokens t0, t1 for K and V, metadata, alpha.
template <int BITS>
struct CompTile {
  Words<BITS> k0, k1, v0, v1;
  uint32_t km0, km1, vm0, vm1;
  uint16_t ka0, ka1, va0, va1;
};

template <int D, int BITS>
__device__ __forceinline__ void load_comp(CompTile<BITS>& T, const DecodeParams& p, int c, size_t row0, size_t row1,
                                          int gi) {
  constexpr int G = D / 32;
  constexpr int RB = D * BITS / 8, GB = 4 * BITS;
  T.k0 = load_group<BITS>(p.kcodes[c] + row0 * RB + gi * GB);
  T.k1 = load_group<BITS>(p.kcodes[c] + row1 * RB + gi * GB);
  T.v0 = load_group<BITS>(p.vcodes[c] + row0 * RB + gi * GB);
  T.v1 = load_group<BITS>(p.vcodes[c] + row1 * RB + gi * GB);
  T.km0 = p.kmeta[c][row0 * G + gi];
  T.km1 = p.kmeta[c][row1 * G + gi];
  T.vm0 = p.vmeta[c][row0 * G + gi];
  T.vm1 = p.vmeta[c][row1 * G + gi];
  if (c > 0) {
    T.ka0 = p.kalpha[c][row0];
    T.ka1 = p.kalpha[c][row1];
    T.va0 = p.valpha[c][row0];
    T.va1 = p.valpha[c][row1];
  } else {
    T.ka0 = T.ka1 = T.va0 = T.va1 = 0x3c00;  // 1.0, unused
  }
}

template <int D, int NC, uint32_t CB>
struct Tile {
  CompTile<cbits<CB, 0>()> c0;
  CompTile<cbits<CB, (NC > 1 ? 1 : 0)>()> c1;
  CompTile<cbits<CB, (NC > 2 ? 2 : 0)>()> c2;
  CompTile<cbits<CB, (NC > 3 ? 3 : 0)>()> c3;
};

template <int D, int NC, uint32_t CB>
__device__ __forceinline__ void load_tile(Tile<D, NC, CB>& T, const DecodeParams& p, size_t row0, size_t row1, int gi) {
  load_comp<D, cbits<CB, 0>()>(T.c0, p, 0, row0, row1, gi);
  if constexpr (NC > 1) load_comp<D, cbits<CB, 1>()>(T.c1, p, 1, row0, row1, gi);
  if constexpr (NC > 2) load_comp<D, cbits<CB, 2>()>(T.c2, p, 2, row0, row1, gi);
  if constexpr (NC > 3) load_comp<D, cbits<CB, 3>()>(T.c3, p, 3, row0, row1, gi);
}

template <int D, int NC, uint32_t CB, bool HILO>
__global__ __launch_bounds__(kThreads) void decode_main(DecodeParams p) {
  constexpr int G = D / 32;
  constexpr int TPW = 64 / G;
  constexpr int TILE = 2 * TPW;
  __shared__ float red[kWaves][64][33];
  __shared__ float wm[kWaves], wl[kWaves];

  const int split = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.H;
  int len = p.past_len[b];
  len = len < 0 ? 0 : (len > p.T_max ? p.T_max : len);
  const int start = split * p.chunk;
  const int end = min(start + p.chunk, len);
  if (start >= end) return;  // whole block, before any barrier

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int pi = lane / G, gi = lane % G;
  const bool lane_on = pi < TPW;
  const int gsel = lane_on ? gi : 0;

  uint32_t QH[16], QL[16];
  const uint32_t* qp = p.qprep + (size_t)bh * qprep_words(D) + gsel * 33;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    QH[k] = qp[k];
    QL[k] = qp[16 + k];
  }
  const float qsum = __uint_as_float(qp[32]);

  float acc[NC][32];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 32; ++e) acc[c][e] = 0.0f;
  float bias = 0.0f, lsum = 0.0f, m = -INFINITY;
  const size_t rowbase = (size_t)bh * p.T_max;

  for (int base = start + wave * TILE; base < end; base += kWaves * TILE) {
    const int t0 = base + pi, t1 = t0 + TPW;
    const bool ok0 = lane_on && t0 < end, ok1 = lane_on && t1 < end;
    const size_t row0 = rowbase + min(t0, p.T_max - 1), row1 = rowbase + min(t1, p.T_max - 1);
    Tile<D, NC, CB> T;
    load_tile<D, NC, CB>(T, p, row0, row1, gsel);

    // ---- keys: per-component partial scores of this lane's group
    float kp0[NC], kp1[NC];
    float kb0[NC], kb1[NC], vb0[NC], vb1[NC];  // beta weights, K and V
    auto kpart = [&](auto& C, int c, auto bits_tag) {
      constexpr int BB = decltype(bits_tag)::value;
      const float d0 = kdot<BB, HILO>(C.k0, QH, QL), d1 = kdot<BB, HILO>(C.k1, QH, QL);
      kp0[c] = fmaf(f16hi(C.km0) * kTwo24, d0, f16lo(C.km0) * qsum);
      kp1[c] = fmaf(f16hi(C.km1) * kTwo24, d1, f16lo(C.km1) * qsum);
    };
    kpart(T.c0, 0, std::integral_constant<int, cbits<CB, 0>()>{});
    if constexpr (NC > 1) kpart(T.c1, 1, std::integral_constant<int, cbits<CB, 1>()>{});
    if constexpr (NC > 2) kpart(T.c2, 2, std::integral_constant<int, cbits<CB, 2>()>{});
    if constexpr (NC > 3) kpart(T.c3, 3, std::integral_constant<int, cbits<CB, 3>()>{});
    // beta_{NC-1} = 1, beta_c = beta_{c+1} * alpha_{c+1}
    kb0[NC - 1] = kb1[NC - 1] = vb0[NC - 1] = vb1[NC - 1] = 1.0f;
    if constexpr (NC > 3) {
      kb0[2] = f16u(T.c3.ka0); kb1[2] = f16u(T.c3.ka1); vb0[2] = f16u(T.c3.va0); vb1[2] = f16u(T.c3.va1);
    }
    if constexpr (NC > 2) {
      kb0[1] = kb0[2] * f16u(T.c2.ka0); kb1[1] = kb1[2] * f16u(T.c2.ka1);
      vb0[1] = vb0[2] * f16u(T.c2.va0); vb1[1] = vb1[2] * f16u(T.c2.va1);
    }
    if constexpr (NC > 1) {
      kb0[0] = kb0[1] * f16u(T.c1.ka0); kb1[0] = kb1[1] * f16u(T.c1.ka1);
      vb0[0] = vb0[1] * f16u(T.c1.va0); vb1[0] = vb1[1] * f16u(T.c1.va1);
    }
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      s0 = fmaf(kb0[c], kp0[c], s0);
      s1 = fmaf(kb1[c], kp1[c], s1);
    }
    s0 = group_sum<G>(s0);
    s1 = group_sum<G>(s1);
    s0 = ok0 ? s0 : -INFINITY;
    s1 = ok1 ? s1 : -INFINITY;

    // ---- online softmax (log2 domain, scores already scaled by log2 e)
    const float tmax = wave_max(fmaxf(s0, s1));
    if (tmax == -INFINITY) continue;
    if (tmax > m) {
      const float f = exp2f(m - tmax);
      m = tmax;
      lsum *= f;
      bias *= f;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 32; ++e) acc[c][e] *= f;
    }
    const float p0 = ok0 ? exp2f(s0 - m) : 0.0f;
    const float p1 = ok1 ? exp2f(s1 - m) : 0.0f;
    lsum += p0 + p1;

    // ---- values: code part through dot2 with fp16 weights W = 2^6 p beta s, and the
    // offset part from the same rounded W: bias += W (o/s) 2^-6 = ptilde beta o with
    // ptilde = W / (2^6 beta s). Every stored value o + s c of a token is thus weighted
    // by one ptilde (fp16-rounded p), so rounding W costs a relative 2^-11 of the value
    // rather than of its code part s c. Subnormal W (tiny contributions, or s == 0)
    // take the exact p beta o instead.
    auto vpart = [&](auto& C, int c, auto bits_tag) {
      constexpr int BB = decltype(bits_tag)::value;
      const float pb0 = ok0 ? p0 * vb0[c] : 0.0f, pb1 = ok1 ? p1 * vb1[c] : 0.0f;
      const float s0 = f16hi(C.vm0), s1 = f16hi(C.vm1), o0 = f16lo(C.vm0), o1 = f16lo(C.vm1);
      const uint32_t W = pack_h2(fminf(pb0 * s0 * kWScale, 65504.0f), fminf(pb1 * s1 * kWScale, 65504.0f));
      const float wb0 = f16lo(W), wb1 = f16hi(W);
      bias += (wb0 >= kMinNormal) ? wb0 * (o0 * __builtin_amdgcn_rcpf(s0)) * (1.0f / kWScale) : pb0 * o0;
      bias += (wb1 >= kMinNormal) ? wb1 * (o1 * __builtin_amdgcn_rcpf(s1)) * (1.0f / kWScale) : pb1 * o1;
      vacc<BB>(C.v0, C.v1, W, acc[c]);
    };
    vpart(T.c0, 0, std::integral_constant<int, cbits<CB, 0>()>{});
    if constexpr (NC > 1) vpart(T.c1, 1, std::integral_constant<int, cbits<CB, 1>()>{});
    if constexpr (NC > 2) vpart(T.c2, 2, std::integral_constant<int, cbits<CB, 2>()>{});
    if constexpr (NC > 3) vpart(T.c3, 3, std::integral_constant<int, cbits<CB, 3>()>{});
  }

  // ---- per-lane group values -> LDS, then merge lanes and waves
  float out[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    float v = bias;
    constexpr float u = kTwo24 / kWScale;
    v = fmaf(acc[0][e], u / vclass<cbits<CB, 0>()>(e), v);
    if constexpr (NC > 1) v = fmaf(acc[1][e], u / vclass<cbits<CB, (NC > 1 ? 1 : 0)>()>(e), v);
    if constexpr (NC > 2) v = fmaf(acc[2][e], u / vclass<cbits<CB, (NC > 2 ? 2 : 0)>()>(e), v);
    if constexpr (NC > 3) v = fmaf(acc[3][e], u / vclass<cbits<CB, (NC > 3 ? 3 : 0)>()>(e), v);
    out[e] = lane_on ? v : 0.0f;
  }
#pragma unroll
  for (int e = 0; e < 32; ++e) red[wave][lane][e] = out[e];
  const float lw = wave_sum((lane_on && gi == 0) ? lsum : 0.0f);
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
    const int g = d / 32, e = d % 32;
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      float sw = 0.0f;
      for (int i = 0; i < TPW; ++i) sw += red[w][i * G + g][e];
      s = fmaf(f[w], sw, s);
    }
    dst[4 + d] = s;
  }
  if (d == 0) {
    float l = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) l = fmaf(f[w], wl[w], l);
    dst[0] = M;
    dst[1] = l;
  }
}

// ---------------------------------------------------------------- combine
template <int D>
__global__ __launch_bounds__(D) void combine_kernel(CombineParams p) {
  __shared__ float acc_s[D];
  __shared__ float red[D / 32 + 1];
  const int bh = blockIdx.x, b = bh / p.H, h = bh % p.H, i = threadIdx.x;
  int len = p.past_len[b];
  if ((len < 0 || len > p.T_max) && i == 0 && h == 0 && p.dev_err) atomicOr(p.dev_err, RQ_DEVERR_LENGTH);
  len = len < 0 ? 0 : (len > p.T_max ? p.T_max : len);
  const int nvalid = (len + p.chunk - 1) / p.chunk;
  // current token score (original domain, bf16 inputs)
  float x = bf16f(p.q[(size_t)bh * D + i]) * bf16f(p.kcur[(size_t)bh * D + i]);
  for (int m = 1; m < 32; m <<= 1) x += __shfl_xor(x, m, 32);
  if ((i & 31) == 0) red[i / 32] = x;
  __syncthreads();
  float scur = 0.0f;
  for (int w = 0; w < D / 32; ++w) scur += red[w];
  scur *= p.scale_log2;
  const float* part = p.part + (size_t)bh * p.nsplit * part_floats(D);
  float M = scur;
  for (int s = 0; s < nvalid; ++s) M = fmaxf(M, part[s * part_floats(D)]);
  float l = exp2f(scur - M), a = 0.0f;
  for (int s = 0; s < nvalid; ++s) {
    const float* ps = part + s * part_floats(D);
    const float f = exp2f(ps[0] - M);
    l = fmaf(ps[1], f, l);
    a = fmaf(ps[4 + i], f, a);
  }
  float o;
  if (p.rotv) {
    acc_s[i] = a;
    __syncthreads();
    const float* H = p.rotv + (size_t)h * D * D;
    o = 0.0f;
    for (int r = 0; r < D; ++r) o = fmaf(H[(size_t)r * D + i], acc_s[r], o);  // (H^T acc)_i
  } else {
    o = a;
  }
  o = fmaf(exp2f(scur - M), bf16f(p.vcur[(size_t)bh * D + i]), o);
  p.out[(size_t)bh * D + i] = o / l;
}

// ---------------------------------------------------------------- dispatch
typedef void (*MainFn)(DecodeParams);
struct Entry {
  int D, nc;
  uint32_t cb;
  MainFn fn;
};

#define RQ_E(D, NC, CB) {D, NC, CB, decode_main<D, NC, CB, true>}
#define RQ_PLANS(D)                                                                                        \
  RQ_E(D, 1, 0x2), RQ_E(D, 1, 0x4), RQ_E(D, 2, 0x22), RQ_E(D, 2, 0x24), RQ_E(D, 2, 0x42), RQ_E(D, 2, 0x44), \
      RQ_E(D, 3, 0x244), RQ_E(D, 3, 0x224), RQ_E(D, 3, 0x222), RQ_E(D, 3, 0x444), RQ_E(D, 4, 0x2244),        \
      RQ_E(D, 4, 0x2224), RQ_E(D, 4, 0x2222), RQ_E(D, 4, 0x4444)

const Entry kTable[] = {RQ_PLANS(64), RQ_PLANS(96), RQ_PLANS(128)};

uint32_t pack_bits(int nc, const int* bits) {
  uint32_t cb = 0;
  for (int c = 0; c < nc; ++c) cb |= (uint32_t)bits[c] << (4 * c);
  return cb;
}

const Entry* find(int D, int nc, const int* bits) {
  const uint32_t cb = pack_bits(nc, bits);
  for (const Entry& e : kTable)
    if (e.D == D && e.nc == nc && e.cb == cb) return &e;
  return nullptr;
}

}  // namespace

bool have_decode_kernel(int D, int nc, const int* bits) { return find(D, nc, bits) != nullptr; }

int launch_qprep(const QPrepParams& p, int D, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(p.B * p.H));
  switch (D) {
    case 64: hipLaunchKernelGGL(qprep_kernel<64>, grid, dim3(64), 0, s, p); break;
    case 96: hipLaunchKernelGGL(qprep_kernel<96>, grid, dim3(96), 0, s, p); break;
    case 128: hipLaunchKernelGGL(qprep_kernel<128>, grid, dim3(128), 0, s, p); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

int launch_decode_main(const DecodeParams& p, int D, int nc, const int* bits, void* stream) {
  const Entry* e = find(D, nc, bits);
  if (!e) return -1;
  const dim3 grid((unsigned)p.nsplit, (unsigned)(p.B * p.H));
  hipLaunchKernelGGL(e->fn, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

int launch_combine(const CombineParams& p, int D, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(p.B * p.H));
  switch (D) {
    case 64: hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(64), 0, s, p); break;
    case 96: hipLaunchKernelGGL(combine_kernel<96>, grid, dim3(96), 0, s, p); break;
    case 128: hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(128), 0, s, p); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

}  // namespace rq
