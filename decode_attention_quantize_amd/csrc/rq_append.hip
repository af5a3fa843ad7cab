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
#include "rq_fp16.hpp"
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

// Code of value v in a group with fp16 offset od and scale sd (§2.1): the
// nearest level to fl((v - od) / sd), ties to even, clamped to [0, 2^BITS - 1];
// 0 when sd = 0 (a constant group).
// The quotient is formed with rs, sd's single-precision reciprocal (v_rcp_f32,
// within one ulp): t is within |t| 2^-22.9 of the exact quotient, which is
// below 2^-18.9 wherever the clamp leaves a choice (|t| <= 16). So t and the
// correctly rounded quotient have the same nearest integer unless t lies within
// 2^-16 of a half-integer; there (rarely) the division itself decides.
__device__ __forceinline__ double recip_of(double sd) {
  return sd != 0.0 ? (double)__builtin_amdgcn_rcpf((float)sd) : 0.0;   // sd is an fp16 value: exact in fp32
}
template <int BITS>
__device__ __forceinline__ uint32_t code_of(double v, double od, double sd, double rs) {
  constexpr double qmax = (double)((1 << BITS) - 1);
  const double u = v - od;
  const double t = u * rs;
  double c = rint(t);
  if (fabs(fabs(t - c) - 0.5) < 0x1p-16) c = rint(u / (sd != 0.0 ? sd : 1.0));
  return sd != 0.0 ? (uint32_t)fmin(fmax(c, 0.0), qmax) : 0u;
}

// Quantize one row's pair of elements e0 = 32 gi + k, e1 = e0 + 16 (held by
// lane k of a 16-lane row) in one group of 32 channels, or, with G16, e0 in
// group 2 gi and e1 in group 2 gi + 1 of 16 channels each (INT2 only); store
// codes into the token's code row and metadata into its metadata row, and
// return the dequantized pair. A row with lane_on false (the same for its 16
// lanes) stores nothing.
template <int D, int BITS, bool G16>
__device__ __forceinline__ void quantize_pair_t(double v0, double v1, bool lane_on, int gi, int k, uint8_t* row,
                                                uint32_t* mrow, double& d0, double& d1, bool& sat) {
  constexpr double qmax = (double)((1 << BITS) - 1);
  if (!lane_on) {
    v0 = 0.0;
    v1 = 0.0;
  }
  auto mn = [](double a, double b) { return fmin(a, b); };
  auto mx = [](double a, double b) { return fmax(a, b); };
  double mn0, mx0, mn1, mx1;
  if constexpr (G16) {
    mn0 = row16_f64(v0, mn);
    mx0 = row16_f64(v0, mx);
    mn1 = row16_f64(v1, mn);
    mx1 = row16_f64(v1, mx);
  } else {
    mn0 = mn1 = row16_f64(fmin(v0, v1), mn);
    mx0 = mx1 = row16_f64(fmax(v0, v1), mx);
  }
  const uint16_t oa = f16_sat(f64_to_f16<kRoundDown>(mn0), sat);
  const double oda = f16_to_f64(oa);
  const uint16_t sa = f16_sat(f64_to_f16<kRoundUp>((mx0 - oda) / qmax), sat);
  const double sda = f16_to_f64(sa);
  uint16_t ob = oa, sb = sa;
  double odb = oda, sdb = sda;
  if constexpr (G16) {
    ob = f16_sat(f64_to_f16<kRoundDown>(mn1), sat);
    odb = f16_to_f64(ob);
    sb = f16_sat(f64_to_f16<kRoundUp>((mx1 - odb) / qmax), sat);
    sdb = f16_to_f64(sb);
  }
  const double rsa = recip_of(sda), rsb = G16 ? recip_of(sdb) : rsa;
  const uint32_t c0 = code_of<BITS>(v0, oda, sda, rsa), c1 = code_of<BITS>(v1, odb, sdb, rsb);
  d0 = oda + sda * (double)c0;
  d1 = odb + sdb * (double)c1;
  if constexpr (G16) {
    // one 32-bit word per group: element k at bit 16 (k / 8) + 2 (k mod 8)
    const int sh = 16 * (k >> 3) + 2 * (k & 7);
    const uint32_t wa = group_or<16>(c0 << sh), wb = group_or<16>(c1 << sh);
    if (lane_on && k == 0) {
      *reinterpret_cast<uint2*>(row + gi * 8) = make_uint2(wa, wb);
      *reinterpret_cast<uint2*>(mrow + 2 * gi) =
          make_uint2((uint32_t)oa | ((uint32_t)sa << 16), (uint32_t)ob | ((uint32_t)sb << 16));
    }
  } else {
    constexpr int per = 16 / BITS;             // codes per 16-bit half-word
    const int sh = BITS * (k % per);
    uint32_t word = (c0 << sh) | (c1 << (16 + sh));
    word = group_or<per>(word);
    if (lane_on) {
      if (k % per == 0) reinterpret_cast<uint32_t*>(row + gi * 4 * BITS)[k / per] = word;
      if (k == 0) mrow[gi] = (uint32_t)oa | ((uint32_t)sa << 16);
    }
  }
}

// Component kinds of the append: INT2 or INT4 in groups of 32, INT2 in groups of 16.
enum : int { kKind2 = 0, kKind4 = 1, kKind2h = 2 };
__device__ __forceinline__ int kind_of(int bits, bool g16) { return g16 ? kKind2h : (bits == 4 ? kKind4 : kKind2); }

// quantize_pair_t for a loop's kind known at run time (uniform over the wave);
// codes and meta are the loop's buffers, tok the token's row in them.
template <int D>
__device__ __forceinline__ void quantize_pair(double v0, double v1, int bits, bool g16, bool lane_on, int gi, int k,
                                              uint8_t* codes, uint32_t* meta, size_t tok, double& d0, double& d1,
                                              bool& sat) {
  uint8_t* row = codes + tok * (size_t)(D * bits / 8);
  uint32_t* mrow = meta + tok * (size_t)(g16 ? D / 16 : D / 32);
  switch (kind_of(bits, g16)) {
    case kKind4: quantize_pair_t<D, 4, false>(v0, v1, lane_on, gi, k, row, mrow, d0, d1, sat); break;
    case kKind2h: quantize_pair_t<D, 2, true>(v0, v1, lane_on, gi, k, row, mrow, d0, d1, sat); break;
    default: quantize_pair_t<D, 2, false>(v0, v1, lane_on, gi, k, row, mrow, d0, d1, sat); break;
  }
}

// All NG 32-channel groups of one row: the row's pairs (z0[gi], z1[gi]) -> dequantized (d0, d1).
template <int D, int BITS, bool G16>
__device__ __forceinline__ void quantize_row_t(const double (&z0)[D / 32], const double (&z1)[D / 32], bool on, int k,
                                               uint8_t* row, uint32_t* mrow, double (&d0)[D / 32], double (&d1)[D / 32],
                                               bool& sat) {
#pragma unroll
  for (int gi = 0; gi < D / 32; ++gi) quantize_pair_t<D, BITS, G16>(z0[gi], z1[gi], on, gi, k, row, mrow, d0[gi], d1[gi], sat);
}

// The bulk kernel's workgroup: eight waves, one workgroup per compute unit,
// sharing one copy of the rotation in LDS, held in fp64 (up to 133 KB at
// D = 128) so that the matrix-core operands need no conversion.
constexpr int kAppendWaves = 8;
constexpr int kAppendThreads = 64 * kAppendWaves;
constexpr long long kAppendWorkgroups = 256;

// RH: the rotations are stored fp16 (RQ_FLAG_ROT_F16), else fp32.
template <int D, int RH>
__global__ __launch_bounds__(kAppendThreads, 1) void append_kernel(AppendParams p) {
  constexpr int NT = D / 16;        // 16-column tiles of the product
  constexpr int NG = D / 32;        // 32-channel groups
  constexpr int KB = D / 16;        // 4-step blocks of the contraction per lane row
  constexpr int HS = D + 2;         // padded LDS row of the rotation (16-byte aligned, conflict-free rows)
  constexpr int XW = D / 8;         // 32-bit words of a lane's D/4 bf16 operands
  __shared__ double Hs[D * HS];     // Hs[n][k] = H[n][k], exact in fp64
  const int kv = blockIdx.z, h = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  {
    // four entries per piece: 16 bytes of fp32 or 8 bytes of fp16 (RQ_FLAG_ROT_F16),
    // both converted exactly
    const size_t e0 = (size_t)h * D * D;
    for (int idx = threadIdx.x; idx < D * D / 4; idx += kAppendThreads) {
      const int n = idx / (D / 4), c4 = idx % (D / 4);
      float4 v;
      if constexpr (RH) {
        const uint2 x = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.rot[kv]) + e0)[idx];
        v = make_float4(f16lo(x.x), f16hi(x.x), f16lo(x.y), f16hi(x.y));
      } else {
        v = reinterpret_cast<const float4*>(static_cast<const float*>(p.rot[kv]) + e0)[idx];
      }
      double2* dst = reinterpret_cast<double2*>(&Hs[n * HS + 4 * c4]);
      dst[0] = make_double2((double)v.x, (double)v.y);
      dst[1] = make_double2((double)v.z, (double)v.w);
    }
  }
  __syncthreads();

  const int L = p.L, G = p.G, n = p.n;
  const int units = p.B * n;
  const int quads = (units + 3) / 4;
  const int per_wg = (quads + gridDim.x - 1) / gridDim.x;
  const int q_begin = blockIdx.x * per_wg;
  const int q_end = min(q_begin + per_wg, quads);
  const int npiece = (G + 3) / 4;   // pieces of at most 4 loops per loop group
  const int tiles_per_quad = (L / G) * npiece;
  const bool last = p.policy == RQ_POLICY_LAST_LOOP, chain = p.policy == RQ_POLICY_PREV_LOOP;

  const int rsel = lane >> 4, k = lane & 15;   // unit within the quad; lane within its row
  // operand row of this lane: unit l % 4, loop l % 16 / 4 of the piece, contraction block l / 16
  const int a_unit = lane & 3, a_loop = (lane & 15) >> 2, a_blk = lane >> 4;
  bool sat = false;

  // tile tau of this wave's stream -> (quad, group start, first loop of the piece, loops in it)
  // (tiles tau of a wave's stream: quad q_begin + wave + kAppendWaves (tau / tiles_per_quad))
  auto tile_of = [&](int tau, int& quad, int& g0, int& l0, int& nl) {
    quad = q_begin + wave + kAppendWaves * (tau / tiles_per_quad);
    const int rest = tau % tiles_per_quad;
    const int g = rest / npiece, i = rest % npiece;
    const int pc = last ? (i == 0 ? npiece - 1 : i - 1) : i;  // anchor piece first
    g0 = g * G;
    l0 = g0 + 4 * pc;
    nl = min(4, g0 + G - l0);
  };
  auto load_x = [&](int tau, uint4 (&x)[XW / 4]) {
    int quad, g0, l0, nl;
    tile_of(tau, quad, g0, l0, nl);
    const int u = quad * 4 + a_unit;
    const bool ok = a_loop < nl && u < units;
    const int uu = ok ? u : 0;
    const int b = uu / n, i = uu % n;
    const uint4* src = reinterpret_cast<const uint4*>(
        p.kv + (((((size_t)kv * L + (ok ? l0 + a_loop : 0)) * p.B + b) * p.H + h) * n + i) * (size_t)D +
        a_blk * (D / 4));
#pragma unroll
    for (int w = 0; w < XW / 4; ++w) x[w] = ok ? src[w] : make_uint4(0, 0, 0, 0);
  };

  const int my_quads = q_end - q_begin > wave ? (q_end - q_begin - wave + kAppendWaves - 1) / kAppendWaves : 0;
  const int tiles = my_quads * tiles_per_quad;
  double rf0[NG], rf1[NG], den = 0.0;   // reference of the current loop group (this lane's unit)
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) rf0[gi] = rf1[gi] = 0.0;
  uint4 xa[XW / 4];
  if (tiles > 0) load_x(0, xa);
  for (int tau = 0; tau < tiles; ++tau) {
    int quad, g0, l0, nl;
    tile_of(tau, quad, g0, l0, nl);
    // ---- Z of the piece on the matrix cores; the next tile's operands load meanwhile
    d4 acc[NT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) acc[ct] = d4{0.0, 0.0, 0.0, 0.0};
    uint32_t xw[XW];
#pragma unroll
    for (int w = 0; w < XW / 4; ++w) {
      xw[4 * w] = xa[w].x; xw[4 * w + 1] = xa[w].y; xw[4 * w + 2] = xa[w].z; xw[4 * w + 3] = xa[w].w;
    }
    if (tau + 1 < tiles) load_x(tau + 1, xa);
    // rotation operands of the next half-block (two contraction steps) are read
    // from LDS while the products of the current one run; the scheduling barrier
    // keeps the compiler from hoisting all blocks' reads (their registers would
    // spill)
    auto read_h = [&](int hk, double2 (&hb)[NT]) {  // half-block hk: steps 2 hk, 2 hk + 1
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
        hb[ct] = *reinterpret_cast<const double2*>(&Hs[(16 * ct + k) * HS + a_blk * (D / 4) + 2 * hk]);
    };
    double2 hbuf[2][NT];
    read_h(0, hbuf[0]);
#pragma unroll
    for (int hk = 0; hk < 2 * KB; ++hk) {
      if (hk + 1 < 2 * KB) read_h(hk + 1, hbuf[(hk + 1) & 1]);
      const double2(&hb)[NT] = hbuf[hk & 1];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const uint32_t wv = xw[hk];
        const double a = (double)__uint_as_float(q2 ? (wv & 0xffff0000u) : (wv << 16));
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
          acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, q2 ? hb[ct].y : hb[ct].x, acc[ct], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- this lane's unit and its cache row
    const int u = quad * 4 + rsel;
    bool on = u < units;
    size_t tok = 0;
    if (on) {
      const int b = u / n, i = u % n;
      const int t = p.pos[b] + i;
      if (t < 0 || t >= p.T_max) {
        on = false;
        if (k == 0 && p.dev_err) atomicOr(p.dev_err, RQ_DEVERR_CAPACITY);
      } else if (!cache_row(p.table, p.maxblk, p.lbs, p.num_blocks, p.H, p.T_max, b, h, t, tok)) {
        on = false;
        if (k == 0 && p.dev_err) atomicOr(p.dev_err, RQ_DEVERR_BLOCK);
      }
    }

    // ---- quantization: the anchor first (when the piece holds it), then the
    // other loops in order; one step per loop, the loop's column j of acc
    // picked at run time so that the quantizer is instantiated once per kind
    const int a = last ? g0 + G - 1 : g0;
    const int ja = (a >= l0 && a < l0 + nl) ? a - l0 : -1;
#pragma unroll 1
    for (int st = 0; st < nl; ++st) {
      const int j = ja < 0 ? st : (st == 0 ? ja : (st - 1 < ja ? st - 1 : st));
      const int r = l0 + j;
      double z0[NG], z1[NG];
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        z0[gi] = j == 0 ? acc[2 * gi][0] : j == 1 ? acc[2 * gi][1] : j == 2 ? acc[2 * gi][2] : acc[2 * gi][3];
        z1[gi] = j == 0 ? acc[2 * gi + 1][0] : j == 1 ? acc[2 * gi + 1][1] : j == 2 ? acc[2 * gi + 1][2]
                                                                                   : acc[2 * gi + 1][3];
      }
      const bool is_anchor = r == a;
      double at = 0.0;
      if (!is_anchor) {                          // LS alpha against the reference, residual
        double s = 0.0;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) s += z0[gi] * rf0[gi] + z1[gi] * rf1[gi];
        const double num = row16_f64(on ? s : 0.0, [](double x, double y) { return x + y; });
        const double alpha = den > 0.0 ? num / den : 0.0;
        const uint16_t a16 = f16_sat(f64_to_f16<kRoundNearest>(alpha), sat);
        at = f16_to_f64(a16);
        if (on && k == 0) p.alpha[kv][r][tok] = a16;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          z0[gi] = z0[gi] - at * rf0[gi];
          z1[gi] = z1[gi] - at * rf1[gi];
        }
      }
      const bool g16 = (p.g16 >> r) & 1;
      uint8_t* row = p.codes[kv][r] + tok * (size_t)(D * p.bits[r] / 8);
      uint32_t* mrow = p.meta[kv][r] + tok * (size_t)(g16 ? D / 16 : D / 32);
      double q0[NG], q1[NG];
      switch (kind_of(p.bits[r], g16)) {
        case kKind4: quantize_row_t<D, 4, false>(z0, z1, on, k, row, mrow, q0, q1, sat); break;
        case kKind2h: quantize_row_t<D, 2, true>(z0, z1, on, k, row, mrow, q0, q1, sat); break;
        default: quantize_row_t<D, 2, false>(z0, z1, on, k, row, mrow, q0, q1, sat); break;
      }
      if (is_anchor || chain) {                  // the reference: A, or zhat_r = alpha_r zhat_{r-1} + D(c_r)
        double s2 = 0.0;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          rf0[gi] = on ? (is_anchor ? q0[gi] : at * rf0[gi] + q0[gi]) : 0.0;
          rf1[gi] = on ? (is_anchor ? q1[gi] : at * rf1[gi] + q1[gi]) : 0.0;
          s2 += rf0[gi] * rf0[gi] + rf1[gi] * rf1[gi];
        }
        den = row16_f64(s2, [](double x, double y) { return x + y; });
      }
    }
  }
  if (sat && p.dev_err) atomicOr(p.dev_err, RQ_DEVERR_RANGE);
}

// Few-token path (decode-time store of the current token, short chunks): one
// workgroup per run of p.upw consecutive (sequence, token) units, head, tensor
// and layer (blockIdx.z = 2 layer + tensor; the launch's p.nl layers find their
// cache pointers in p.slot, and layer i reads its inputs at kv + i * 2 L B H n
// D). The workgroup stages the head's rotation in LDS once for all its units;
// for each unit, wave w computes Z_r for its loops
// r = w, w + 4, .. on the fp64 vector units (lane k of group gi holds channels
// e0 = 32 gi + k and e1 = e0 + 16, the pair quantize_pair takes), so the four
// waves rotate in parallel. Then every loop group's anchor is quantized, and
// the other loops follow in the policy's dependency order: all at once against
// the shared anchor (Last-loop, First-loop), or one chain step per barrier
// (Previous-loop, all groups together). LM bounds the loop count: the LDS
// footprint grows with it, and at most 8 loops leave room for two workgroups
// per compute unit at D = 128.
template <int D, int LM, int RH>
__global__ __launch_bounds__(256) void append_unit(UnitParams p) {
  constexpr int kLoopsPerWave = LM / kWaves;
  constexpr int HS = D + 2;                // padded LDS row: 8-byte aligned pairs, 16 rows cover all banks
  constexpr int NF = D * D / 4 / kThreads; // float4 per thread of the rotation
  static_assert(NF * 4 * kThreads == D * D, "rotation staging must tile the block");
  __shared__ float Hs[D * HS];
  __shared__ float xs[LM][D];
  __shared__ double rec[LM][D];            // per loop group: current reference (reconstruction)
  __shared__ double dens[LM];              // its squared norm
  const int u0 = blockIdx.x * p.upw, h = blockIdx.y, kv = blockIdx.z & 1, layer = blockIdx.z >> 1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int L = p.L, G = p.G;
  // this layer's and tensor's pointers
  const void* const* sl = p.slot + (size_t)layer * unit_stride(L);
  const int32_t* table = p.maxblk ? static_cast<const int32_t*>(sl[0]) : nullptr;
  const void* const* st = sl + 1 + kv * (1 + 3 * L);
  const void* rot = st[0];                 // fp32, or fp16 (RH)
  auto codes_of = [&](int r) { return static_cast<uint8_t*>(const_cast<void*>(st[1 + r])); };
  auto meta_of = [&](int r) { return static_cast<uint32_t*>(const_cast<void*>(st[1 + L + r])); };
  auto alpha_of = [&](int r) { return static_cast<uint16_t*>(const_cast<void*>(st[1 + 2 * L + r])); };
  const uint16_t* kvin = p.kv + (size_t)layer * 2 * L * p.B * p.H * p.n * D;

  // ---- stage H (row-major, padded) once for all of the workgroup's units
  {
    // four entries per piece: 16 bytes of fp32 or 8 bytes of fp16, converted exactly
    float4 hv[NF];
    if constexpr (RH) {
      const uint2* Hg = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(rot) + (size_t)h * D * D);
      uint2 x[NF];
#pragma unroll
      for (int j = 0; j < NF; ++j) x[j] = Hg[tid + j * kThreads];
#pragma unroll
      for (int j = 0; j < NF; ++j) hv[j] = make_float4(f16lo(x[j].x), f16hi(x[j].x), f16lo(x[j].y), f16hi(x[j].y));
    } else {
      const float4* Hg = reinterpret_cast<const float4*>(static_cast<const float*>(rot) + (size_t)h * D * D);
#pragma unroll
      for (int j = 0; j < NF; ++j) hv[j] = Hg[tid + j * kThreads];
    }
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int f = 4 * (tid + j * kThreads), n = f / D, k = f % D;
      float2* dst = reinterpret_cast<float2*>(&Hs[n * HS + k]);
      dst[0] = make_float2(hv[j].x, hv[j].y);
      dst[1] = make_float2(hv[j].z, hv[j].w);
    }
  }

  bool sat = false;                        // an fp16 offset, scale or alpha was saturated
  const int u_end = min(u0 + p.upw, p.B * p.n);
  // The input rows of unit u + 1 load while unit u is processed: XI 16-byte
  // pieces per thread hold the L rows of a unit.
  constexpr int XI = (LM * (D / 8) + kThreads - 1) / kThreads;
  uint4 xn[XI];
  auto load_x = [&](int uu) {
    const int bb = uu / p.n, ii = uu % p.n;
#pragma unroll
    for (int q = 0; q < XI; ++q) {
      const int idx = tid + q * kThreads, xr = idx / (D / 8), xc = idx % (D / 8);
      const uint4* row = reinterpret_cast<const uint4*>(
          kvin + (((((size_t)kv * L + (xr < L ? xr : 0)) * p.B + bb) * p.H + h) * p.n + ii) * (size_t)D);
      xn[q] = xr < L ? row[xc] : make_uint4(0, 0, 0, 0);
    }
  };
  if (u0 < u_end) load_x(u0);
  for (int u = u0; u < u_end; ++u) {       // uniform over the workgroup
    uint4 xc[XI];
#pragma unroll
    for (int q = 0; q < XI; ++q) xc[q] = xn[q];
    if (u + 1 < u_end) load_x(u + 1);
    const int b = u / p.n, i = u % p.n;
    const int t = p.pos[b] + i;
    if (t < 0 || t >= p.T_max) {             // the whole unit, before any barrier
      if (tid == 0 && p.dev_err) atomicOr(p.dev_err, RQ_DEVERR_CAPACITY);
      continue;
    }
    size_t tok;
    if (!cache_row(table, p.maxblk, p.lbs, p.num_blocks, p.H, p.T_max, b, h, t, tok)) {  // likewise
      if (tid == 0 && p.dev_err) atomicOr(p.dev_err, RQ_DEVERR_BLOCK);
      continue;
    }
    __syncthreads();                         // the previous unit is done with xs, rec and dens

    // ---- stage the L input rows (bf16 -> fp32)
#pragma unroll
    for (int q = 0; q < XI; ++q) {
      const int idx = tid + q * kThreads, xr = idx / (D / 8), xcol = idx % (D / 8);
      if (xr < L) {
        const uint32_t w[4] = {xc[q].x, xc[q].y, xc[q].z, xc[q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xs[xr][8 * xcol + 2 * e] = __uint_as_float(w[e] << 16);
          xs[xr][8 * xcol + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
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
      const uint16_t a16 = f16_sat(f64_to_f16<kRoundNearest>(alpha), sat);
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
  }                                        // units
  if (sat && p.dev_err) atomicOr(p.dev_err, RQ_DEVERR_RANGE);
}

}  // namespace

namespace {
template <int D, int RH>
void launch_unit_d(const UnitParams& p, bool small, const dim3& grid, hipStream_t s) {
  if (small) hipLaunchKernelGGL((append_unit<D, 8, RH>), grid, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL((append_unit<D, RQ_MAX_LOOPS, RH>), grid, dim3(kThreads), 0, s, p);
}
}  // namespace

int launch_append_unit(const UnitParams& p, int D, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)((p.B * p.n + p.upw - 1) / p.upw), (unsigned)p.H, (unsigned)(2 * p.nl));
  const bool small = p.L <= 8, rh = p.rot_f16 != 0;
  switch (D) {
    case 64: rh ? launch_unit_d<64, 1>(p, small, grid, s) : launch_unit_d<64, 0>(p, small, grid, s); break;
    case 96: rh ? launch_unit_d<96, 1>(p, small, grid, s) : launch_unit_d<96, 0>(p, small, grid, s); break;
    case 128: rh ? launch_unit_d<128, 1>(p, small, grid, s) : launch_unit_d<128, 0>(p, small, grid, s); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

int launch_append(const AppendParams& p, int D, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  // About one resident workgroup per compute unit in one round (the rotation
  // takes 33-133 KB of LDS), each at least one quad per wave.
  const long long quads = ((long long)p.B * p.n + 3) / 4;
  long long chunks = kAppendWorkgroups / (2LL * p.H);
  const long long most = (quads + kAppendWaves - 1) / kAppendWaves;
  if (chunks > most) chunks = most;
  if (chunks < 1) chunks = 1;
  const dim3 grid((unsigned)chunks, (unsigned)p.H, 2);
  const dim3 block(kAppendThreads);
  switch (D) {
    case 64:
      if (p.rot_f16) hipLaunchKernelGGL((append_kernel<64, 1>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((append_kernel<64, 0>), grid, block, 0, s, p);
      break;
    case 96:
      if (p.rot_f16) hipLaunchKernelGGL((append_kernel<96, 1>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((append_kernel<96, 0>), grid, block, 0, s, p);
      break;
    case 128:
      if (p.rot_f16) hipLaunchKernelGGL((append_kernel<128, 1>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((append_kernel<128, 0>), grid, block, 0, s, p);
      break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

}  // namespace rq
