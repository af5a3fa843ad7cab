// Quantize-and-append kernel of the ResidualQuant cache (paper "KV Cache
// Quantization for Looped Transformers with 2-Bit Residuals": §2.1 affine
// group quantization, §3.2 Last-loop / Previous-loop references and the LS
// coefficient, §3.3 shared rotation, §3.4 per-loop bit widths, §4.2 deferred
// store after the final loop, App. G.1 the quantize-anchor-then-residual order).
//
// One wave owns a tile of 16 matrix rows = floor(16/L) (sequence, token) units
// times their L loops. The rotation Z = X H^T of the tile runs on the fp64
// matrix cores (v_mfma_f64_16x16x4_f64): the products of fp32 rotation entries
// and bf16 inputs are exact in fp64, so Z agrees with any other fp64 evaluation
// to the last bit or so, and the integer code decisions that follow are taken
// in fp64 as well. This file is compiled with -ffp-contract=off: every product
// and sum below is rounded on its own.
#include <hip/hip_runtime.h>

#include "rq_device.hpp"
#include "rq_internal.hpp"

namespace rq {
namespace {

typedef double d4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double bf16_to_f64(uint16_t h) {
  return (double)__uint_as_float((uint32_t)h << 16);
}

__device__ __forceinline__ double f16_to_f64(uint16_t h) {
  return (double)(float)__builtin_bit_cast(_Float16, h);
}

// binary64 -> binary16 bits. mode 0: nearest-even, 1: toward -inf, 2: toward +inf.
// The magnitude M * 2^(E-52) is cut at the fp16 spacing of its binade
// (2^(E-10), or 2^-24 below the normal range); the dropped bits decide rounding.
__device__ uint16_t f64_to_f16(double x, int mode) {
  const uint64_t bits = (uint64_t)__double_as_longlong(x);
  const bool neg = (bits >> 63) != 0;
  const uint16_t sign = neg ? 0x8000 : 0;
  const int e = (int)((bits >> 52) & 0x7ff);
  const uint64_t frac = bits & 0xFFFFFFFFFFFFFull;
  if (e == 0x7ff) return frac ? (uint16_t)0x7e00 : (uint16_t)(sign | 0x7c00);
  if (e == 0 && frac == 0) return sign;
  const int E = (e == 0) ? -1022 : e - 1023;
  const uint64_t M = (e == 0) ? frac : (frac | (1ull << 52));
  const int qexp = (E < -14) ? -24 : E - 10;
  const int shift = qexp - (E - 52);  // >= 42
  uint64_t n = 0;
  bool up;
  if (shift >= 64) {
    up = (mode == 1 && neg) || (mode == 2 && !neg);  // nonzero remainder below half a spacing
  } else {
    n = M >> shift;
    const uint64_t rem = M & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (mode == 0) up = rem > half || (rem == half && (n & 1));
    else if (mode == 1) up = neg && rem != 0;
    else up = !neg && rem != 0;
  }
  n += up ? 1 : 0;
  if (qexp == -24) return (uint16_t)(sign | (uint16_t)n);  // n <= 1024; 1024 is 2^-14
  int EE = E;
  if (n == 2048) {
    n = 1024;
    EE += 1;
  }
  if (EE > 15) {
    const bool toward_zero = (mode == 1 && !neg) || (mode == 2 && neg);
    return (uint16_t)(sign | (toward_zero ? 0x7bff : 0x7c00));
  }
  return (uint16_t)(sign | (uint16_t)((EE + 15) << 10) | (uint16_t)(n - 1024));
}

// The cache holds offsets, scales and LS coefficients as finite fp16 numbers:
// a rounding that overflows (inputs or residuals beyond the fp16 range) is held
// at the largest finite magnitude of its sign and reported through `sat`.
__device__ __forceinline__ uint16_t f16_sat(uint16_t h, bool& sat) {
  if ((h & 0x7fff) == 0x7c00) {
    sat = true;
    return (uint16_t)((h & 0x8000) | 0x7bff);
  }
  return h;
}

// Lane exchanges of the reductions below, in the vector unit (no LDS round
// trip). Within a row of 16 lanes, DPP: the quad permutations give lane l ^ 1
// and l ^ 2; after those, every lane of a quad holds the same value, so the
// half-row mirror (lane i <- 7 - i) and the row mirror (i <- 15 - i) give the
// value of lane l ^ 4 and then l ^ 8. Across rows, the gfx950 swaps of odd and
// even 16-lane rows and of the two half-waves. A reduction therefore combines
// exactly the pairs a xor butterfly combines, and its fp64 sums are the same.
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int x) {
  return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = dpp_i32<CTRL>((int)(b & 0xffffffff)), hi = dpp_i32<CTRL>((int)(b >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
// Sum over lanes l and l ^ 16 (W = 16) or l ^ 32 (W = 32).
template <int W>
__device__ __forceinline__ double swap_add_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = (int)(b & 0xffffffff), hi = (int)(b >> 32);
  const auto l = W == 16 ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                         : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto h = W == 16 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                         : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  const double a = __longlong_as_double(((long long)h[0] << 32) | (unsigned int)l[0]);
  const double c = __longlong_as_double(((long long)h[1] << 32) | (unsigned int)l[1]);
  return a + c;                                   // own and partner value, in either order
}

// op over the 16 lanes of a row, the result in every lane of it.
template <typename Op>
__device__ __forceinline__ double row16_f64(double v, Op op) {
  v = op(v, dpp_f64<kQuadSwap1>(v));
  v = op(v, dpp_f64<kQuadSwap2>(v));
  v = op(v, dpp_f64<kRowHalfMirror>(v));
  return op(v, dpp_f64<kRowMirror>(v));
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  v = row16_f64(v, [](double a, double b) { return a + b; });
  v = swap_add_f64<16>(v);
  return swap_add_f64<32>(v);
}

// Bitwise or over the N consecutive lanes N i .. N i + N - 1 (N = 2, 4, 8, 16).
template <int N>
__device__ __forceinline__ uint32_t group_or(uint32_t x) {
  int v = (int)x;
  v |= dpp_i32<kQuadSwap1>(v);
  if constexpr (N > 2) v |= dpp_i32<kQuadSwap2>(v);
  if constexpr (N > 4) v |= dpp_i32<kRowHalfMirror>(v);
  if constexpr (N > 8) v |= dpp_i32<kRowMirror>(v);
  return (uint32_t)v;
}

// Quantize one row's pair of elements e0 = 32 gi + k, e1 = e0 + 16 (held by
// lane k of lane group gi) in one group of 32 channels, or, with g16, e0 in
// group 2 gi and e1 in group 2 gi + 1 of 16 channels each (INT2 only); store
// codes and metadata, return the dequantized pair.
// Row of token t of (b, h) in every cache buffer: contiguous [B][H][T_max], or
// through the block table of a paged cache. False for an invalid block id.
__device__ __forceinline__ bool cache_row(const int32_t* table, int maxblk, int lbs, int num_blocks, int H, int T_max,
                                          int b, int h, int t, size_t& row) {
  if (!table) {
    row = ((size_t)b * H + h) * T_max + t;
    return true;
  }
  const int32_t blk = table[(size_t)b * maxblk + (t >> lbs)];
  if ((uint32_t)blk >= (uint32_t)num_blocks) return false;
  row = (((size_t)blk * H + h) << lbs) + (size_t)(t & ((1 << lbs) - 1));
  return true;
}

template <int D>
__device__ void quantize_pair(double v0, double v1, int bits, bool g16, bool lane_on, int gi, int k,
                              uint8_t* codes, uint32_t* meta, size_t tok, double& d0, double& d1, bool& sat) {
  double mn0, mx0, mn1, mx1;
  if (g16) {
    mn0 = lane_on ? v0 : 0.0;
    mx0 = mn0;
    mn1 = lane_on ? v1 : 0.0;
    mx1 = mn1;
  } else {
    mn0 = mn1 = lane_on ? fmin(v0, v1) : 0.0;
    mx0 = mx1 = lane_on ? fmax(v0, v1) : 0.0;
  }
  {                                             // the 16 lanes of one lane group
    auto mn = [](double a, double b) { return fmin(a, b); };
    auto mx = [](double a, double b) { return fmax(a, b); };
    mn0 = row16_f64(mn0, mn);
    mx0 = row16_f64(mx0, mx);
    if (g16) {
      mn1 = row16_f64(mn1, mn);
      mx1 = row16_f64(mx1, mx);
    }
  }
  if (!g16) {
    mn1 = mn0;
    mx1 = mx0;
  }
  const double qmax = (double)((1 << bits) - 1);
  uint16_t o16[2], s16[2];
  double od[2], sd[2];
  for (int i = 0; i < (g16 ? 2 : 1); ++i) {
    o16[i] = f16_sat(f64_to_f16(i ? mn1 : mn0, 1), sat);
    od[i] = f16_to_f64(o16[i]);
    s16[i] = f16_sat(f64_to_f16(((i ? mx1 : mx0) - od[i]) / qmax, 2), sat);
    sd[i] = f16_to_f64(s16[i]);
  }
  if (!g16) {
    o16[1] = o16[0]; s16[1] = s16[0];
    od[1] = od[0]; sd[1] = sd[0];
  }
  uint32_t c0 = 0, c1 = 0;
  if (sd[0] != 0.0) c0 = (uint32_t)fmin(fmax(rint((v0 - od[0]) / sd[0]), 0.0), qmax);
  if (sd[1] != 0.0) c1 = (uint32_t)fmin(fmax(rint((v1 - od[1]) / sd[1]), 0.0), qmax);
  d0 = od[0] + sd[0] * (double)c0;
  d1 = od[1] + sd[1] * (double)c1;
  uint8_t* row = codes + tok * (size_t)(D * bits / 8);
  if (g16) {
    // one 32-bit word per group: element k at bit 16 (k / 8) + 2 (k mod 8)
    const int sh = 16 * (k >> 3) + 2 * (k & 7);
    uint32_t wa = c0 << sh, wb = c1 << sh;
    wa = group_or<16>(wa);
    wb = group_or<16>(wb);
    if (lane_on && k == 0) {
      *reinterpret_cast<uint2*>(row + gi * 8) = make_uint2(wa, wb);
      *reinterpret_cast<uint2*>(meta + tok * (D / 16) + 2 * gi) =
          make_uint2((uint32_t)o16[0] | ((uint32_t)s16[0] << 16), (uint32_t)o16[1] | ((uint32_t)s16[1] << 16));
    }
    return;
  }
  const int per = 16 / bits;                    // codes per 16-bit half-word
  const int sh = bits * (k % per);
  uint32_t word = (c0 << sh) | (c1 << (16 + sh));
  word = per == 8 ? group_or<8>(word) : group_or<4>(word);
  if (lane_on) {
    if (k % per == 0) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(row + gi * 4 * bits);
      dst[k / per] = word;
    }
    if (k == 0) meta[tok * (D / 32) + gi] = (uint32_t)o16[0] | ((uint32_t)s16[0] << 16);
  }
}

template <int D>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  constexpr int NT = D / 16;   // 16-wide output column tiles
  constexpr int NK = D / 4;    // k steps of the 16x16x4 instruction
  constexpr int HP = D + 16;   // padded row of the transposed rotation in LDS
  __shared__ float Ht[D * HP];                 // Ht[k][n] = H[n][k]
  __shared__ double Zs[kWaves][16][D + 1];
  const int kv = blockIdx.z, h = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float* Hg = p.rot[kv] + (size_t)h * D * D;
  for (int idx = threadIdx.x; idx < D * D; idx += blockDim.x) {
    const int n = idx / D, k = idx % D;
    Ht[k * HP + n] = Hg[idx];
  }
  __syncthreads();

  const int L = p.L;
  const int U = 16 / L;                        // (sequence, token) units per tile
  const int units = p.B * p.n;
  const int u0 = (blockIdx.x * kWaves + wave) * U;
  if (u0 >= units) return;                     // no block-wide barrier follows

  // ---- Z = X H^T on the matrix cores ----------------------------------------
  const int m = lane & 15;
  const int mu = m / L, mr = m % L;
  const bool row_ok = mu < U && u0 + mu < units;
  const int urow = row_ok ? u0 + mu : 0;
  const int b_row = urow / p.n, i_row = urow % p.n;
  const uint16_t* xrow =
      p.kv + (((((size_t)kv * L + mr) * p.B + b_row) * p.H + h) * p.n + i_row) * (size_t)D;
  d4 acc[NT];
  for (int ct = 0; ct < NT; ++ct) acc[ct] = d4{0.0, 0.0, 0.0, 0.0};
  for (int kk = 0; kk < NK; ++kk) {
    const int k = kk * 4 + (lane >> 4);
    const double a = row_ok ? bf16_to_f64(xrow[k]) : 0.0;
    const float* hk = &Ht[k * HP + (lane & 15)];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
      acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, (double)hk[ct * 16], acc[ct], 0, 0, 0);
  }
  // lane l, register j of column tile ct holds Z[4j + l/16][16 ct + l%16]
#pragma unroll
  for (int ct = 0; ct < NT; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) Zs[wave][4 * j + (lane >> 4)][ct * 16 + (lane & 15)] = acc[ct][j];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

  // ---- per unit: anchor, LS alpha, residuals ---------------------------------
  const int gi = lane >> 4, k = lane & 15;
  const bool lane_on = gi < D / 32;
  const int e0 = lane_on ? 32 * gi + k : 0, e1 = e0 + 16;
  for (int uu = 0; uu < U; ++uu) {
    const int u = u0 + uu;
    if (u >= units) break;
    const int b = u / p.n, i = u % p.n;
    const int t = p.pos[b] + i;
    if (t < 0 || t >= p.T_max) {
      if (lane == 0 && p.dev_err) atomicOr(p.dev_err, RQ_DEVERR_CAPACITY);
      continue;
    }
    size_t tok;
    if (!cache_row(p.table, p.maxblk, p.lbs, p.num_blocks, p.H, p.T_max, b, h, t, tok)) {
      if (lane == 0 && p.dev_err) atomicOr(p.dev_err, RQ_DEVERR_BLOCK);
      continue;
    }
    const double(*Z)[D + 1] = &Zs[wave][uu * L];
    bool sat = false;
    // each loop group independently: its anchor, then the other loops of the group
    for (int g0 = 0; g0 < L; g0 += p.G) {
      const int a = (p.policy == RQ_POLICY_LAST_LOOP) ? g0 + p.G - 1 : g0;
      double r0, r1;  // reference (reconstructed anchor, or previous loop) at e0, e1
      quantize_pair<D>(Z[a][e0], Z[a][e1], p.bits[a], (p.g16 >> a) & 1, lane_on, gi, k, p.codes[kv][a],
                       p.meta[kv][a], tok, r0, r1, sat);
      if (!lane_on) r0 = r1 = 0.0;
      double den_cur = wave_sum_f64(r0 * r0 + r1 * r1);
      for (int r = g0; r < g0 + p.G; ++r) {
        if (r == a) continue;
        const double z0 = lane_on ? Z[r][e0] : 0.0, z1 = lane_on ? Z[r][e1] : 0.0;
        const double num = wave_sum_f64(z0 * r0 + z1 * r1);
        const double alpha = den_cur > 0.0 ? num / den_cur : 0.0;
        const uint16_t a16 = f16_sat(f64_to_f16(alpha, 0), sat);
        const double at = f16_to_f64(a16);
        if (lane == 0) p.alpha[kv][r][tok] = a16;
        double q0, q1;
        quantize_pair<D>(z0 - at * r0, z1 - at * r1, p.bits[r], (p.g16 >> r) & 1, lane_on, gi, k, p.codes[kv][r],
                         p.meta[kv][r], tok, q0, q1, sat);
        if (p.policy == RQ_POLICY_PREV_LOOP) {  // zhat_r = alpha_r zhat_{r-1} + D(c_r)
          r0 = lane_on ? at * r0 + q0 : 0.0;
          r1 = lane_on ? at * r1 + q1 : 0.0;
          den_cur = wave_sum_f64(r0 * r0 + r1 * r1);
        }
      }
    }
    if (sat && p.dev_err) atomicOr(p.dev_err, RQ_DEVERR_RANGE);
  }
}

// Few-token path (decode-time store of the current token, short chunks): one
// workgroup per (sequence, token) unit, head, tensor and layer (blockIdx.z =
// 2 layer + tensor; the launch's p.nl layers find their cache pointers in
// p.slot, and layer i reads its inputs at kv + i * 2 L B H n D). The workgroup stages
// the head's rotation in LDS once; wave w computes Z_r for its loops
// r = w, w + 4, .. on the fp64 vector units (lane k of group gi holds channels
// e0 = 32 gi + k and e1 = e0 + 16, the pair quantize_pair takes), so the four
// waves rotate in parallel. Then every loop group's anchor is quantized, and
// the other loops follow in the policy's dependency order: all at once against
// the shared anchor (Last-loop, First-loop), or one chain step per barrier
// (Previous-loop, all groups together). LM bounds the loop count: the LDS
// footprint grows with it, and at most 8 loops leave room for two workgroups
// per compute unit at D = 128.
template <int D, int LM>
__global__ __launch_bounds__(256) void append_unit(UnitParams p) {
  constexpr int kLoopsPerWave = LM / kWaves;
  constexpr int HS = D + 2;                // padded LDS row: 8-byte aligned pairs, 16 rows cover all banks
  constexpr int NF = D * D / 4 / kThreads; // float4 per thread of the rotation
  static_assert(NF * 4 * kThreads == D * D, "rotation staging must tile the block");
  __shared__ float Hs[D * HS];
  __shared__ float xs[LM][D];
  __shared__ double rec[LM][D];            // per loop group: current reference (reconstruction)
  __shared__ double dens[LM];              // its squared norm
  const int u = blockIdx.x, h = blockIdx.y, kv = blockIdx.z & 1, layer = blockIdx.z >> 1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int L = p.L, G = p.G;
  // this layer's and tensor's pointers
  const void* const* sl = p.slot + (size_t)layer * unit_stride(L);
  const int32_t* table = p.maxblk ? static_cast<const int32_t*>(sl[0]) : nullptr;
  const void* const* st = sl + 1 + kv * (1 + 3 * L);
  const float* rot = static_cast<const float*>(st[0]);
  auto codes_of = [&](int r) { return static_cast<uint8_t*>(const_cast<void*>(st[1 + r])); };
  auto meta_of = [&](int r) { return static_cast<uint32_t*>(const_cast<void*>(st[1 + L + r])); };
  auto alpha_of = [&](int r) { return static_cast<uint16_t*>(const_cast<void*>(st[1 + 2 * L + r])); };
  const uint16_t* kvin = p.kv + (size_t)layer * 2 * L * p.B * p.H * p.n * D;
  const int b = u / p.n, i = u % p.n;
  const int t = p.pos[b] + i;
  if (t < 0 || t >= p.T_max) {             // whole block, before any barrier
    if (tid == 0 && p.dev_err) atomicOr(p.dev_err, RQ_DEVERR_CAPACITY);
    return;
  }
  size_t tok;
  if (!cache_row(table, p.maxblk, p.lbs, p.num_blocks, p.H, p.T_max, b, h, t, tok)) {  // likewise
    if (tid == 0 && p.dev_err) atomicOr(p.dev_err, RQ_DEVERR_BLOCK);
    return;
  }

  // ---- stage H (row-major, padded) and the L input rows
  {
    const float4* Hg = reinterpret_cast<const float4*>(rot + (size_t)h * D * D);
    float4 hv[NF];
#pragma unroll
    for (int j = 0; j < NF; ++j) hv[j] = Hg[tid + j * kThreads];
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int f = 4 * (tid + j * kThreads), n = f / D, k = f % D;
      float2* dst = reinterpret_cast<float2*>(&Hs[n * HS + k]);
      dst[0] = make_float2(hv[j].x, hv[j].y);
      dst[1] = make_float2(hv[j].z, hv[j].w);
    }
    for (int idx = tid; idx < L * (D / 8); idx += kThreads) {
      const int xr = idx / (D / 8), xc = idx % (D / 8);
      const uint16_t* row = kvin + (((((size_t)kv * L + xr) * p.B + b) * p.H + h) * p.n + i) * (size_t)D;
      const uint4 xv = reinterpret_cast<const uint4*>(row)[xc];
      const uint32_t w[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xs[xr][8 * xc + 2 * q] = __uint_as_float(w[q] << 16);
        xs[xr][8 * xc + 2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
      }
    }
  }
  __syncthreads();

  // ---- Z_r at (e0, e1) for this wave's loops; products of fp32 and bf16 are exact in fp64
  const int gi = lane >> 4, kk = lane & 15;
  const bool lane_on = gi < D / 32;
  const int e0 = lane_on ? 32 * gi + kk : 0, e1 = e0 + 16;
  double z0[kLoopsPerWave], z1[kLoopsPerWave];
#pragma unroll
  for (int j = 0; j < kLoopsPerWave; ++j) {
    const int r = wave + kWaves * j;
    double a0 = 0.0, a1 = 0.0, c0 = 0.0, c1 = 0.0;
    if (r < L) {
      const float* x = xs[r];
      const float* h0 = &Hs[e0 * HS];
      const float* h1 = &Hs[e1 * HS];
#pragma unroll 4
      for (int k = 0; k < D; k += 2) {
        const float2 xv = *reinterpret_cast<const float2*>(&x[k]);
        const float2 u0 = *reinterpret_cast<const float2*>(&h0[k]);
        const float2 u1 = *reinterpret_cast<const float2*>(&h1[k]);
        const double x0 = (double)xv.x, x1 = (double)xv.y;
        a0 = fma((double)u0.x, x0, a0);
        c0 = fma((double)u0.y, x1, c0);
        a1 = fma((double)u1.x, x0, a1);
        c1 = fma((double)u1.y, x1, c1);
      }
    }
    z0[j] = a0 + c0;
    z1[j] = a1 + c1;
  }

  const bool last = p.policy == RQ_POLICY_LAST_LOOP, chain = p.policy == RQ_POLICY_PREV_LOOP;
  auto anchor_of = [&](int r) { return last ? r / G * G + G - 1 : r / G * G; };

  bool sat = false;                        // an fp16 offset, scale or alpha was saturated
  // ---- anchors of every group (by the waves that own them)
#pragma unroll
  for (int j = 0; j < kLoopsPerWave; ++j) {
    const int r = wave + kWaves * j;
    if (r < L && r == anchor_of(r)) {
      double r0, r1;
      quantize_pair<D>(z0[j], z1[j], p.bits[r], (p.g16 >> r) & 1, lane_on, gi, kk, codes_of(r), meta_of(r), tok, r0,
                       r1, sat);
      if (!lane_on) r0 = r1 = 0.0;
      const double den = wave_sum_f64(r0 * r0 + r1 * r1);
      if (lane_on) {
        rec[r / G][e0] = r0;
        rec[r / G][e1] = r1;
      }
      if (lane == 0) dens[r / G] = den;
    }
  }
  __syncthreads();

  // ---- one residual: alpha against the group's reference, then Q(Z_r - alpha ref)
  auto residual = [&](int r, double zz0, double zz1, double& q0, double& q1, double& at, double& r0,
                      double& r1) __attribute__((always_inline)) {
    const int g = r / G;
    r0 = lane_on ? rec[g][e0] : 0.0;
    r1 = lane_on ? rec[g][e1] : 0.0;
    const double den = dens[g];
    const double num = wave_sum_f64((lane_on ? zz0 : 0.0) * r0 + (lane_on ? zz1 : 0.0) * r1);
    const double alpha = den > 0.0 ? num / den : 0.0;
    const uint16_t a16 = f16_sat(f64_to_f16(alpha, 0), sat);
    at = f16_to_f64(a16);
    if (lane == 0) alpha_of(r)[tok] = a16;
    quantize_pair<D>(zz0 - at * r0, zz1 - at * r1, p.bits[r], (p.g16 >> r) & 1, lane_on, gi, kk, codes_of(r),
                     meta_of(r), tok, q0, q1, sat);
  };

  if (!chain) {
    // shared anchor: the waves work on all their loops at once
#pragma unroll
    for (int j = 0; j < kLoopsPerWave; ++j) {
      const int r = wave + kWaves * j;
      if (r < L && r != anchor_of(r)) {
        double q0, q1, at, r0, r1;
        residual(r, z0[j], z1[j], q0, q1, at, r0, r1);
      }
    }
  } else {
    // a chain in every group: step st handles loop g G + st of each group g
    for (int st = 1; st < G; ++st) {
#pragma unroll
      for (int j = 0; j < kLoopsPerWave; ++j) {
        const int r = wave + kWaves * j;
        if (r < L && r % G == st) {
          double q0, q1, at, r0, r1;
          residual(r, z0[j], z1[j], q0, q1, at, r0, r1);
          const double n0 = lane_on ? at * r0 + q0 : 0.0, n1 = lane_on ? at * r1 + q1 : 0.0;
          const double den = wave_sum_f64(n0 * n0 + n1 * n1);
          if (lane_on) {
            rec[r / G][e0] = n0;
            rec[r / G][e1] = n1;
          }
          if (lane == 0) dens[r / G] = den;
        }
      }
      __syncthreads();
    }
  }
  if (sat && p.dev_err) atomicOr(p.dev_err, RQ_DEVERR_RANGE);
}

}  // namespace

int launch_append_unit(const UnitParams& p, int D, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(p.B * p.n), (unsigned)p.H, (unsigned)(2 * p.nl));
  const bool small = p.L <= 8;
  switch (D) {
    case 64:
      if (small) hipLaunchKernelGGL((append_unit<64, 8>), grid, dim3(kThreads), 0, s, p);
      else hipLaunchKernelGGL((append_unit<64, RQ_MAX_LOOPS>), grid, dim3(kThreads), 0, s, p);
      break;
    case 96:
      if (small) hipLaunchKernelGGL((append_unit<96, 8>), grid, dim3(kThreads), 0, s, p);
      else hipLaunchKernelGGL((append_unit<96, RQ_MAX_LOOPS>), grid, dim3(kThreads), 0, s, p);
      break;
    case 128:
      if (small) hipLaunchKernelGGL((append_unit<128, 8>), grid, dim3(kThreads), 0, s, p);
      else hipLaunchKernelGGL((append_unit<128, RQ_MAX_LOOPS>), grid, dim3(kThreads), 0, s, p);
      break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

int launch_append(const AppendParams& p, int D, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int U = 16 / p.L;
  const long long tiles = ((long long)p.B * p.n + U - 1) / U;
  const dim3 grid((unsigned)((tiles + kWaves - 1) / kWaves), (unsigned)p.H, 2);
  switch (D) {
    case 64: hipLaunchKernelGGL(append_kernel<64>, grid, dim3(kThreads), 0, s, p); break;
    case 96: hipLaunchKernelGGL(append_kernel<96>, grid, dim3(kThreads), 0, s, p); break;
    case 128: hipLaunchKernelGGL(append_kernel<128>, grid, dim3(kThreads), 0, s, p); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

}  // namespace rq
