// Fused dequantize + split-K decode attention over the ResidualQuant cache
// (paper "KV Cache Quantization for Looped Transformers with 2-Bit Residuals":
// §4.1 kernel, §4.2 "Decode" past/current merge, App. G.2 "Reconstruction and
// attention"). Two launches per call: the fused kernel rotates the query in
// every workgroup, streams its range of the compressed cache and stores a
// split partial; the combine merges the partials of each (b, h) with the
// current bf16 token and applies the single inverse value rotation.
//
// Per (b, h) the attended keys are zhat_t = sum_c beta_{c,t} D(c_{c,t}) in the
// rotated domain, with components c = anchor, residual (Last-loop) or the
// chain anchor, residual 2, .., residual r (Previous-loop), and
// beta_{c,t} = prod_{j>c} alpha_{j,t} (so the last component has weight 1).
// With the rotation folded into the query (q' = H_K q) the score is
//   s_t = sum_c beta_{c,t} sum_groups [ s_{c,g} (q'_g . code_{c,g}) + o_{c,g} sum(q'_g) ],
// and values accumulate sum_t p_t zhat_V,t in the rotated domain with the same
// per-group split into a code part (weight p beta s) and an offset part.
//
// Keys: q' of a lane's group is held as fixed point in signed 8-bit limbs;
// masking a code word with 0x0F0F0F0F (INT4) or 0x03030303 (INT2) puts four
// codes in four bytes, and v_dot4c_i32_i8 against each limb gives an exact
// integer sum of q'_e code_e.
// Values: a masked code field read as an fp16 bit pattern is the subnormal
// number code * 2^(shift - 24), exactly, and the mixed-precision FMA takes fp16
// subnormal operands exactly. A byte permute pairs the same code byte of two
// tokens, and one mask then yields that element of both tokens.
//
// A lane always owns a block of 32 channels. A component is INT4 or INT2 in one
// group of 32 (offset, scale) per block, or INT2 in two groups of 16 (§5
// "Quantization setup": g = 16 for INT2): then word j of the block's codes is
// group j, the block carries two metadata words, and the key and value sums
// keep the two halves of the block apart.
#pragma once

#include <hip/hip_runtime.h>

#include "rq_combine.hpp"
#include "rq_device.hpp"
#include "rq_internal.hpp"

namespace rq {
namespace {

#ifndef RQ_WAVES_SMALL
#define RQ_WAVES_SMALL 3
#endif

constexpr float kTwo24 = 16777216.0f;  // a masked code field reads as code * 2^(shift - 24)

template <int BITS>
struct Words {
  uint32_t w[BITS];  // one group of 32 codes = BITS 32-bit words
};

// Cache policy of the streaming loads: non-temporal (the nt bit). Every cache
// byte is read once per call, so keeping it out of the caches' reuse state
// leaves L2 and MALL to the rotations and partials; measured ~10% faster.
constexpr int kAux = 2;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor over [base, base + bytes): loads past the end return zero
// without touching memory (raw buffer, hardware range check).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int BITS>
__device__ __forceinline__ Words<BITS> load_group(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  Words<BITS> w;
  if constexpr (BITS == 4) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAux);
    w.w[0] = v.x; w.w[1] = v.y; w.w[2] = v.z; w.w[3] = v.w;
  } else {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kAux);
    w.w[0] = v.x; w.w[1] = v.y;
  }
  return w;
}

// q' of one group as fixed point, v_e = round(q'_e 2^E) with |v| < 2^FIX
// (E per group, FIX = 7 LIMBS), written in balanced base 256 as LIMBS signed
// 8-bit limbs (most significant first) and packed four per register in the
// order the code bytes of a word come out of one mask (see kdot). Integer dot
// products of the codes with each limb are exact; the rounding of q' to FIX
// bits is the only error, a relative 2^-FIX of the group's largest |q'|, and the
// score error it causes grows with the size of the scores. Two limbs (14 bits,
// the default) keep scores within ~1e-3 (log2 units) of exact at 16k tokens with
// synthetic outlier keys; three limbs (21 bits, RQ_FLAG_PRECISE_QUERY) take
// them to ~1e-5 for sharper softmax distributions, for 16 more VALU
// instructions per tile and 16 more registers.
template <int LIMBS>
constexpr int fix_bits() { return 7 * LIMBS; }
template <int LIMBS>
struct QFix {
  uint32_t q4[4][2][LIMBS];   // INT4: word j, mask (low / high nibbles), limb
  uint32_t q2[2][4][LIMBS];   // INT2, one group of 32: word j, field s, limb
  uint32_t q2h[2][4][LIMBS];  // INT2, two groups of 16: word j (= group j), field s, limb
};

// Elements of the group that byte b (0..3) of a masked word holds.
//   INT4 word j, mask m (0: bits 0-3 of each byte, 1: bits 4-7):
//     bytes 0..3 = elements 4j + m, 4j + 2 + m, 16 + 4j + m, 18 + 4j + m.
//   INT2 word j, field s (bits 2s, 2s+1 of each byte):
//     bytes 0..3 = elements 8j + s, 8j + 4 + s, 16 + 8j + s, 20 + 8j + s.
//   INT2 in groups of 16, word j = group j, field s:
//     bytes 0..3 = elements 16j + s, 16j + 4 + s, 16j + 8 + s, 16j + 12 + s.
__host__ __device__ constexpr int int4_elem(int j, int m, int b) { return (b >> 1) * 16 + 4 * j + 2 * (b & 1) + m; }
__host__ __device__ constexpr int int2_elem(int j, int s, int b) { return (b >> 1) * 16 + 8 * j + 4 * (b & 1) + s; }
__host__ __device__ constexpr int int2h_elem(int j, int s, int b) { return 16 * j + 4 * b + s; }
// Their inverses: word (j * 2 + m, or j * 4 + s) and byte of element e in each table.
__host__ __device__ constexpr int int4_word(int e) { return ((e & 15) >> 2) * 2 + (e & 1); }
__host__ __device__ constexpr int int4_byte(int e) { return 2 * (e >> 4) + ((e >> 1) & 1); }
__host__ __device__ constexpr int int2_word(int e) { return ((e & 15) >> 3) * 4 + (e & 3); }
__host__ __device__ constexpr int int2_byte(int e) { return 2 * (e >> 4) + ((e >> 2) & 1); }
__host__ __device__ constexpr int int2h_word(int e) { return (e >> 4) * 4 + (e & 3); }
__host__ __device__ constexpr int int2h_byte(int e) { return (e >> 2) & 3; }
constexpr bool tables_invert() {
  for (int e = 0; e < 32; ++e)
    if (int4_elem(int4_word(e) >> 1, int4_word(e) & 1, int4_byte(e)) != e ||
        int2_elem(int2_word(e) >> 2, int2_word(e) & 3, int2_byte(e)) != e ||
        int2h_elem(int2h_word(e) >> 2, int2h_word(e) & 3, int2h_byte(e)) != e)
      return false;
  return true;
}
static_assert(tables_invert(), "word and byte positions invert the element maps");

// Component kind, one nibble of a plan: the bit width in bits 0-2, and
// kGroup16 for INT2 in groups of 16 channels (else one group of 32).
constexpr int kGroup16 = 8;
__host__ __device__ constexpr int kbits(int k) { return k & 7; }
__host__ __device__ constexpr bool kg16(int k) { return (k & kGroup16) != 0; }

// sum_e v_e code_e over each group of 16 of an INT2 block (exact in int32).
template <int LIMBS>
__device__ __forceinline__ void kdot16(const Words<2>& c, const QFix<LIMBS>& Q, int& d0, int& d1) {
  int r[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int a[LIMBS];
#pragma unroll
    for (int l = 0; l < LIMBS; ++l) a[l] = 0;
    const uint32_t x = c.w[j];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int m = (int)((x >> (2 * f)) & 0x03030303u);
#pragma unroll
      for (int l = 0; l < LIMBS; ++l) a[l] = __builtin_amdgcn_sdot4(m, (int)Q.q2h[j][f][l], a[l], false);
    }
    r[j] = a[0];
#pragma unroll
    for (int l = 1; l < LIMBS; ++l) r[j] = r[j] * 256 + a[l];
  }
  d0 = r[0];
  d1 = r[1];
}

// sum_e v_e code_e over one group (exact in int32: |v| < 2^21, 32 codes < 16).
template <int BITS, int LIMBS>
__device__ __forceinline__ int kdot(const Words<BITS>& c, const QFix<LIMBS>& Q) {
  int a[LIMBS];
#pragma unroll
  for (int l = 0; l < LIMBS; ++l) a[l] = 0;
  if constexpr (BITS == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x = c.w[j];
      const int m0 = (int)(x & 0x0F0F0F0Fu), m1 = (int)((x >> 4) & 0x0F0F0F0Fu);
#pragma unroll
      for (int l = 0; l < LIMBS; ++l) {
        a[l] = __builtin_amdgcn_sdot4(m0, (int)Q.q4[j][0][l], a[l], false);
        a[l] = __builtin_amdgcn_sdot4(m1, (int)Q.q4[j][1][l], a[l], false);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t x = c.w[j];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int m = (int)((x >> (2 * f)) & 0x03030303u);
#pragma unroll
        for (int l = 0; l < LIMBS; ++l) a[l] = __builtin_amdgcn_sdot4(m, (int)Q.q2[j][f][l], a[l], false);
      }
    }
  }
  int r = a[0];
#pragma unroll
  for (int l = 1; l < LIMBS; ++l) r = r * 256 + a[l];
  return r;
}

// Field scale 2^shift of element e of a group (index k = e mod 16 in its half)
// as vpairs() presents it: INT4 k even 1, odd 16; INT2 4^(k mod 4).
template <int BITS>
__host__ __device__ constexpr float vclass(int e) {
  return BITS == 4 ? (((e & 15) & 1) ? 16.0f : 1.0f) : (float)(1 << (2 * ((e & 15) & 3)));
}

// acc[e] += W.lo code_{t0,e} + W.hi code_{t1,e} for the 32 elements of a group,
// accumulated at the field scale of reference width REF (the widest component),
// so that every component shares one accumulator per element.
// Code pairs (token t0 in the low half, t1 in the high half, as fp16 subnormal
// patterns at the reference field class) of elements e = 16 half + 4 blk + q,
// q = 0..3, of one component.
// INT4: half-word blk of each half holds k = 4 blk .. 4 blk + 3; bytes 2 half and
// 2 half + 1 of word blk carry them, low nibble at class 1, high nibble at 16.
// INT2: element block blk lies in byte 2 half + (blk & 1) of word blk / 2, fields
// at classes 1, 4, 16, 64. Under an INT4 reference (classes 1, 16, 1, 16) the
// upper two fields are shifted down by 4 bits, so they land at classes 1 and 4
// and q = 1, 3 take the weight 4W (x4 in vw4()).
__device__ __forceinline__ uint32_t pair_byte(uint32_t w0, uint32_t w1, int by) {
  // [t0 byte `by`, 0, t1 byte `by`, 0]
  return __builtin_amdgcn_perm(w1, w0, 0x0c000c00u | ((uint32_t)(4 + by) << 16) | (uint32_t)by);
}

// INT2 in groups of 16: elements 16 half + 4 blk + q are field q of byte blk of
// word half (group `half`), at the same classes as above.
template <int K, int REF>
__device__ __forceinline__ void vpairs(const Words<kbits(K)>& c0, const Words<kbits(K)>& c1, int half, int blk,
                                       uint32_t (&x)[4]) {
  constexpr int BITS = kbits(K);
  if constexpr (BITS == 4) {
    const uint32_t b0 = pair_byte(c0.w[blk], c1.w[blk], 2 * half), b1 = pair_byte(c0.w[blk], c1.w[blk], 2 * half + 1);
    x[0] = b0 & 0x000F000Fu;
    x[1] = b0 & 0x00F000F0u;
    x[2] = b1 & 0x000F000Fu;
    x[3] = b1 & 0x00F000F0u;
  } else {
    const uint32_t b = kg16(K) ? pair_byte(c0.w[half], c1.w[half], blk)
                               : pair_byte(c0.w[blk >> 1], c1.w[blk >> 1], 2 * half + (blk & 1));
    if constexpr (REF == 4) {
      const uint32_t b4 = b >> 4;
      x[0] = b & 0x00030003u;
      x[1] = b & 0x000C000Cu;
      x[2] = b4 & 0x00030003u;
      x[3] = b4 & 0x000C000Cu;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = b & (0x00030003u << (2 * q));
    }
  }
}

// Whether field q of a BITS-wide component takes 4W under reference REF.
template <int BITS, int REF>
__host__ __device__ constexpr bool vw4(int q) {
  return BITS == 2 && REF == 4 && (q & 1);
}

template <uint32_t CB, int c>
constexpr int ckind() {
  return (int)((CB >> (4 * c)) & 0xF);
}

template <uint32_t CB, int NC>
constexpr int ref_bits() {
  int r = 2;
  for (int c = 0; c < NC; ++c)
    if (kbits((int)((CB >> (4 * c)) & 0xF)) == 4) r = 4;
  return r;
}

template <uint32_t CB, int NC>
constexpr bool any_g16() {
  bool r = false;
  for (int c = 0; c < NC; ++c) r = r || kg16((int)((CB >> (4 * c)) & 0xF));
  return r;
}

// Whether some component is BITS wide with the given group size (g16: 16).
template <uint32_t CB, int NC>
constexpr bool any_bits(int bits, bool g16) {
  bool r = false;
  for (int c = 0; c < NC; ++c) {
    const int k = (int)((CB >> (4 * c)) & 0xF);
    r = r || (kbits(k) == bits && kg16(k) == g16);
  }
  return r;
}

// Per-component tile data of one lane: codes of tokens t0, t1 for K and V,
// metadata (one word per group of the lane's block), alpha.
template <int K>
struct CompTile {
  static constexpr int NM = kg16(K) ? 2 : 1;
  Words<kbits(K)> k0, k1, v0, v1;
  uint32_t km0[NM], km1[NM], vm0[NM], vm1[NM];
  uint16_t ka0, ka1, va0, va1;
};

// Descriptors of one component's six streams over this workgroup's token range.
struct CompRsrc {
  __amdgpu_buffer_rsrc_t kc, vc, km, vm, ka, va;
};

// Contiguous cache: rows [row0, row0 + ntok) of the (b, h) series. Paged cache:
// row0 = 0 and ntok = every row of the block pool.
template <int D, int K>
__device__ __forceinline__ CompRsrc comp_rsrc(const DecodeParams& p, int c, size_t row0, uint32_t ntok) {
  constexpr int G = kg16(K) ? D / 16 : D / 32;  // metadata words per token
  constexpr uint32_t RB = D * kbits(K) / 8;
  CompRsrc r;
  r.kc = make_rsrc(p.kcodes[c] + row0 * RB, ntok * RB);
  r.vc = make_rsrc(p.vcodes[c] + row0 * RB, ntok * RB);
  r.km = make_rsrc(p.kmeta[c] + row0 * G, ntok * G * 4);
  r.vm = make_rsrc(p.vmeta[c] + row0 * G, ntok * G * 4);
  if (c > 0) {
    r.ka = make_rsrc(p.kalpha[c] + row0, ntok * 2);
    r.va = make_rsrc(p.valpha[c] + row0, ntok * 2);
  } else {
    r.ka = r.va = r.kc;
  }
  return r;
}

// Byte offsets of this lane's rows in the current tile: codes (per width),
// metadata and alpha of token t0; token t1 = t0 + TPW sits a fixed distance
// further in a contiguous cache, or at its own row (the `1` fields) in a paged one.
struct Offs {
  uint32_t c4, c2, m, a;
  uint32_t c4_1, c2_1, m_1, a_1;
};

// SEP1: token t1 has its own row offsets (per-lane paged rows); else it sits
// TPW rows after t0.
template <int D, int K, bool SEP1>
__device__ __forceinline__ void load_comp(CompTile<K>& T, const CompRsrc& r, bool has_alpha, const Offs& o) {
  constexpr int BITS = kbits(K);
  constexpr int G = D / 32;
  constexpr int TPW = 64 / G;
  constexpr uint32_t RB = D * BITS / 8;
  const uint32_t oc = BITS == 4 ? o.c4 : o.c2;
  const uint32_t oc1 = SEP1 ? (BITS == 4 ? o.c4_1 : o.c2_1) : oc + TPW * RB;
  const uint32_t om1 = SEP1 ? o.m_1 : o.m + TPW * G * 4;
  const uint32_t oa1 = SEP1 ? o.a_1 : o.a + TPW * 2;
  T.k0 = load_group<BITS>(r.kc, oc);
  T.k1 = load_group<BITS>(r.kc, oc1);
  T.v0 = load_group<BITS>(r.vc, oc);
  T.v1 = load_group<BITS>(r.vc, oc1);
  if constexpr (kg16(K)) {               // two groups of 16 per block: 8 bytes of metadata
    const uint32_t m0 = 2 * o.m, m1 = 2 * om1;
    const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(r.km, m0, 0, kAux);
    const u32x2 b = __builtin_amdgcn_raw_buffer_load_b64(r.km, m1, 0, kAux);
    const u32x2 c = __builtin_amdgcn_raw_buffer_load_b64(r.vm, m0, 0, kAux);
    const u32x2 d = __builtin_amdgcn_raw_buffer_load_b64(r.vm, m1, 0, kAux);
    T.km0[0] = a.x; T.km0[1] = a.y; T.km1[0] = b.x; T.km1[1] = b.y;
    T.vm0[0] = c.x; T.vm0[1] = c.y; T.vm1[0] = d.x; T.vm1[1] = d.y;
  } else {
    T.km0[0] = __builtin_amdgcn_raw_buffer_load_b32(r.km, o.m, 0, kAux);
    T.km1[0] = __builtin_amdgcn_raw_buffer_load_b32(r.km, om1, 0, kAux);
    T.vm0[0] = __builtin_amdgcn_raw_buffer_load_b32(r.vm, o.m, 0, kAux);
    T.vm1[0] = __builtin_amdgcn_raw_buffer_load_b32(r.vm, om1, 0, kAux);
  }
  if (has_alpha) {
    T.ka0 = __builtin_amdgcn_raw_buffer_load_b16(r.ka, o.a, 0, kAux);
    T.ka1 = __builtin_amdgcn_raw_buffer_load_b16(r.ka, oa1, 0, kAux);
    T.va0 = __builtin_amdgcn_raw_buffer_load_b16(r.va, o.a, 0, kAux);
    T.va1 = __builtin_amdgcn_raw_buffer_load_b16(r.va, oa1, 0, kAux);
  } else {
    T.ka0 = T.ka1 = T.va0 = T.va1 = 0x3c00;  // 1.0, unused
  }
}

// Calls f(integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Tile data of up to kMaxComp components (members past NC are never used).
template <int D, int NC, uint32_t CB>
struct Tile {
  CompTile<ckind<CB, 0>()> c0;
  CompTile<ckind<CB, (NC > 1 ? 1 : 0)>()> c1;
  CompTile<ckind<CB, (NC > 2 ? 2 : 0)>()> c2;
  CompTile<ckind<CB, (NC > 3 ? 3 : 0)>()> c3;
  CompTile<ckind<CB, (NC > 4 ? 4 : 0)>()> c4;
  CompTile<ckind<CB, (NC > 5 ? 5 : 0)>()> c5;
  CompTile<ckind<CB, (NC > 6 ? 6 : 0)>()> c6;
  CompTile<ckind<CB, (NC > 7 ? 7 : 0)>()> c7;
};
static_assert(kMaxComp == 8, "Tile holds eight components");

// Component I of a tile.
template <int I, class T>
__device__ __forceinline__ auto& tc(T& t) {
  if constexpr (I == 0) return t.c0;
  else if constexpr (I == 1) return t.c1;
  else if constexpr (I == 2) return t.c2;
  else if constexpr (I == 3) return t.c3;
  else if constexpr (I == 4) return t.c4;
  else if constexpr (I == 5) return t.c5;
  else if constexpr (I == 6) return t.c6;
  else return t.c7;
}

template <int D, int NC, uint32_t CB, bool SEP1>
__device__ __forceinline__ void load_tile(Tile<D, NC, CB>& T, const CompRsrc (&R)[NC], const Offs& o) {
  static_for<0, NC>([&](auto ic) {
    constexpr int c = decltype(ic)::value;
    load_comp<D, ckind<CB, c>(), SEP1>(tc<c>(T), R[c], c > 0, o);
  });
}

// Waves per SIMD the register budget is tuned for: three for plans whose tile
// data is small enough (one INT4 and one INT2 component at most), two otherwise.
// The 21-bit query (a third of its registers more) does not fit three waves'
// registers without spilling.
template <int NC, uint32_t CB, int LIMBS>
constexpr int waves_for() {
  int bits = 0;
  for (int c = 0; c < NC; ++c) bits += kbits((int)((CB >> (4 * c)) & 0xF));
  if (NC > 4) return 1;                        // long chains: two tiles of up to eight components
  if (LIMBS > 2) return 2;
  return (NC <= 2 && bits <= 6) ? RQ_WAVES_SMALL : 2;
}

// The paged instances keep block ids and per-lane row offsets live as well;
// with groups of 16 that no longer fits three waves' registers without
// spilling.
template <int NC, uint32_t CB, int LIMBS>
constexpr int waves_for_paged() {
  return any_g16<CB, NC>() ? 2 : waves_for<NC, CB, LIMBS>();
}

// Cache addressing of the streaming kernel.
//   kContig: the (b, h) series is contiguous; the descriptors cover the slot.
//   kPagedLane: rows through the block table (token t of sequence b lives in row
//     (blk H + h) BS + t mod BS of the pool, blk = table[b][t / BS]), looked up
//     per lane; descriptors cover the pool. Any block size.
// (A mode with one block id per tile and per-tile descriptors covering exactly
// the tile's rows, for block sizes that are multiples of the tile, measured no
// faster for one plan and 5-9 % slower for the others: its descriptors took
// more scalar registers than a wave has, and the overflow went through vector
// registers.)
enum : int { kContig = 0, kPagedLane = 1 };

// One (b, h, slot) work item: stream the slot's tokens of the compressed
// cache and store the slot's partial.
template <int D, int NC, uint32_t CB, int DEPTH, int MODE, int LIMBS, int RH>
__device__ __forceinline__ void decode_body(const DecodeParams& p) {
  constexpr int G = D / 32;
  constexpr int TPW = 64 / G;
  constexpr int TILE = 2 * TPW;
  static_assert(TILE == tile_tokens(D), "slot unit must be the wave tile");
  constexpr int REF = ref_bits<CB, NC>();
  __shared__ float red[kWaves][64][33];
  __shared__ PartialLds S;

  int split, b, h;
  split_item(p.nsplit, p.B, p.H, split, b, h);
  const int bh = b * p.H + h;
  // the wave index is uniform across the wave: say so, so that tile positions and
  // everything derived from them (paged descriptors) live in scalar registers
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;

  // The prologue overlaps its memory round trips: the sequence length (a scalar
  // load, issued before anything that could be taken to write memory), q (once
  // per workgroup, into LDS) and the query rotation's rows of H_K (half a row
  // per thread) are requested together, then the first tile of the cache; only
  // then does the rotation wait for its operands. What bounds the prologue is
  // the data the compute unit's loads return (64 KB of H_K per workgroup), so q
  // is not loaded per thread.
  // (A paged cache first requests the block ids of its first tiles: the tile
  // loads wait for them, and vector loads complete in issue order.)
  int len = p.past_len[b];
  constexpr int RJ = D / 16;
  const bool rot_on = tid < 2 * D;
  __shared__ uint4 qs[D / 8];
  uint4 qg = make_uint4(0, 0, 0, 0);
  // The thread's half row of H_K as raw words, four entries per piece: fp32
  // entries fill a piece, fp16 ones (RH: RQ_FLAG_ROT_F16) its first two words.
  uint4 hu[RJ], hw[RJ];
  // Loaded by every thread, with clamped indices (only the threads that need
  // them use the values): loads outside branches keep the waits for later
  // loads exact.
  auto load_rotation = [&]() {
    qg = reinterpret_cast<const uint4*>(p.q + (size_t)bh * D)[tid % (D / 8)];
    const int row = min(tid >> 1, D - 1), half = tid & 1;
    const size_t e0 = ((size_t)h * D + row) * D + half * (D / 2);  // first entry of the half row
    if constexpr (RH) {
      const uint2* hr = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.rotk) + e0);
#pragma unroll
      for (int j = 0; j < RJ; ++j) {
        const uint2 a = hr[2 * j], c = hr[2 * j + 1];
        hu[j].x = a.x;
        hu[j].y = a.y;
        hw[j].x = c.x;
        hw[j].y = c.y;
      }
    } else {
      const uint4* hr = reinterpret_cast<const uint4*>(static_cast<const float*>(p.rotk) + e0);
#pragma unroll
      for (int j = 0; j < RJ; ++j) {
        hu[j] = hr[2 * j];
        hw[j] = hr[2 * j + 1];
      }
    }
  };
  if constexpr (MODE == kContig) {
    load_rotation();
    asm volatile("" ::: "memory");  // those loads are issued here, ahead of the ones below
  }

  // A slot past the sequence's last used one streams nothing and stores no
  // partial; its workgroup still runs to the end (no return with loads in flight).
  len = len < 0 ? 0 : (len > p.T_max ? p.T_max : len);
  const bool active = split < slots_used(len, p.nsplit, p.unit);  // uniform over the workgroup
  const int chunk = slot_len(len, p.nsplit, p.unit);
  const int start = active ? split * chunk : 0;
  const int end = active ? min(start + chunk, len) : 0;

  // This workgroup reads rows [start, end) of its (b, h); the descriptors cover
  // exactly that range, so tiles running past its end load zeros (masked). A
  // paged cache's descriptors cover the whole pool; a token past the end, or
  // with an invalid block id, is pointed at the first row past the pool, which
  // also loads zeros.
  const size_t row0 = MODE == kContig ? (size_t)bh * p.T_max + start : 0;
  const uint32_t ntok = MODE == kContig ? (uint32_t)(end - start) : p.pool_rows;
  const int pi = lane / G, gi = lane % G;
  const bool lane_on = pi < TPW;
  const int gsel = lane_on ? gi : 0;
  CompRsrc R[NC];
  static_for<0, NC>([&](auto ic) {
    constexpr int c = decltype(ic)::value;
    R[c] = comp_rsrc<D, ckind<CB, c>()>(p, c, row0, ntok);
  });

  constexpr int STRIDE = kWaves * TILE;  // tokens between a wave's consecutive tiles
  // Paged: the block ids of a tile's two tokens are loaded DEPTH fetches ahead
  // of the tile itself, so the dependent load never waits on the tile stream.
  const int32_t* table = MODE != kContig ? p.table + (size_t)b * p.maxblk : nullptr;
  constexpr int TAHEAD = DEPTH;
  int32_t tq[TAHEAD][2];                 // block ids for the next TAHEAD fetches, oldest first
  // The ids are loaded unconditionally, from an index clamped into the
  // sequence's table row, and replaced by -1 past the range: with no branch
  // around the loads, the waits for them stay exact and do not also wait for
  // loads issued after them.
  const int last_tok = max(end - 1, 0);
  auto table_load = [&](int base, int32_t (&e)[2]) {
    const int t0 = base + pi, t1 = t0 + TPW;
    const int32_t v0 = table[min(t0, last_tok) >> p.lbs], v1 = table[min(t1, last_tok) >> p.lbs];
    e[0] = (lane_on && t0 < end) ? v0 : -1;
    e[1] = (lane_on && t1 < end) ? v1 : -1;
  };
  auto page_row = [&](int t, int32_t blk) -> uint32_t {
    if (!lane_on || t >= end) return p.pool_rows;
    if ((uint32_t)blk >= (uint32_t)p.num_blocks) {
      if (p.dev_err) atomicOr(p.dev_err, RQ_DEVERR_BLOCK);
      return p.pool_rows;
    }
    return ((uint32_t)blk * (uint32_t)p.H + (uint32_t)h) * (1u << p.lbs) + ((uint32_t)t & ((1u << p.lbs) - 1u));
  };
  auto fetch = [&](Tile<D, NC, CB>& T, int base) {
    Offs o;
    if constexpr (MODE == kPagedLane) {
      const int32_t b0 = tq[0][0], b1 = tq[0][1];
#pragma unroll
      for (int k = 0; k + 1 < TAHEAD; ++k) {
        tq[k][0] = tq[k + 1][0];
        tq[k][1] = tq[k + 1][1];
      }
      table_load(base + TAHEAD * STRIDE, tq[TAHEAD - 1]);
      const uint32_t r0 = page_row(base + pi, b0), r1 = page_row(base + pi + TPW, b1);
      o.c4 = r0 * (D / 2) + gsel * 16;
      o.c2 = r0 * (D / 4) + gsel * 8;
      o.m = (r0 * G + gsel) * 4;
      o.a = r0 * 2;
      o.c4_1 = r1 * (D / 2) + gsel * 16;
      o.c2_1 = r1 * (D / 4) + gsel * 8;
      o.m_1 = (r1 * G + gsel) * 4;
      o.a_1 = r1 * 2;
    } else {
      const uint32_t rel = (uint32_t)(base - start) + (uint32_t)pi;  // row of token t0 in the range
      o.c4 = rel * (D / 2) + gsel * 16;
      o.c2 = rel * (D / 4) + gsel * 8;
      o.m = (rel * G + gsel) * 4;
      o.a = rel * 2;
    }
    load_tile<D, NC, CB, MODE == kPagedLane>(T, R, o);
  };

  // Each wave keeps DEPTH tiles in flight: tile i is
  // processed while tiles i+1 .. i+DEPTH-1 load. Loads are issued
  // unconditionally (past the range they return zeros, masked) so the wait
  // counts are the same on every path and the compiler does not drain the
  // pipeline early.
  int base = start + wave * TILE;
  Tile<D, NC, CB> A, B, C;

  // first tile(s) (and paged block ids) requested before the rotation waits
  if constexpr (MODE != kContig) {
#pragma unroll
    for (int k = 0; k < TAHEAD; ++k) table_load(base + k * STRIDE, tq[k]);
    asm volatile("" ::: "memory");
    load_rotation();
    asm volatile("" ::: "memory");
  }
  fetch(A, base);
  if constexpr (DEPTH == 3) fetch(B, base + STRIDE);
  asm volatile("" ::: "memory");
  if (tid < D / 8) qs[tid] = qg;
  __syncthreads();

  // ---- q' = scale log2(e) H_K q for this (b, h): two threads per row, each
  // with half of the row and half of q. Wave w then holds group w of q' (rows
  // 32 w .. 32 w + 31, element e in lanes 2e and 2e + 1) and turns it into fixed
  // point once for the workgroup (per-group exponent): the limbs go into LDS at
  // the byte positions of the packed words each key table needs (see kdot), and
  // the group's qsum and scale beside them. qsum, which multiplies the group
  // offsets, is the sum of the same fixed-point values, so a stored value
  // o + s c meets one consistent q'.
  constexpr int QW = 8 * LIMBS;                 // words of one key table of one group
  constexpr bool T4 = any_bits<CB, NC>(4, false), T2 = any_bits<CB, NC>(2, false), T2H = any_g16<CB, NC>();
  __shared__ __attribute__((aligned(16))) uint32_t qtab[3][G][QW];  // INT4, INT2, INT2 in groups of 16
  __shared__ float4 qmeta[G];                   // qsum, scale, qsum of each 16-channel half
  if (rot_on) {
    const int row = tid >> 1, half = tid & 1;
    float a0 = 0.0f, a1 = 0.0f;
    // the same products in the same order for either storage (fp16 entries are
    // converted exactly), so equal matrix values give bit-equal q'
    auto rotate = [&](auto entries) {
#pragma unroll
      for (int j = 0; j < RJ; ++j) {
        const uint4 w = qs[half * RJ + j];
        const float4 u = entries(hu[j]), v = entries(hw[j]);
        a0 = fmaf(u.x, bf16lo(w.x), a0);
        a1 = fmaf(u.y, bf16hi(w.x), a1);
        a0 = fmaf(u.z, bf16lo(w.y), a0);
        a1 = fmaf(u.w, bf16hi(w.y), a1);
        a0 = fmaf(v.x, bf16lo(w.z), a0);
        a1 = fmaf(v.y, bf16hi(w.z), a1);
        a0 = fmaf(v.z, bf16lo(w.w), a0);
        a1 = fmaf(v.w, bf16hi(w.w), a1);
      }
    };
    if constexpr (RH)
      rotate([](const uint4& x) { return make_float4(f16lo(x.x), f16hi(x.x), f16lo(x.y), f16hi(x.y)); });
    else
      rotate([](const uint4& x) {
        return make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w));
      });
    float acc = a0 + a1;
    acc += __shfl_xor(acc, 1, 64);
    const float qv = acc * p.scale_log2;          // q'_e, e = row mod 32, of group `wave`
    float mx = fabsf(qv);
#pragma unroll
    for (int s = 2; s < 64; s <<= 1) mx = fmaxf(mx, __shfl_xor(mx, s, 64));
    int ex = 0;
    (void)frexpf(mx, &ex);                        // mx in [2^(ex-1), 2^ex)
    const int E = mx > 0.0f ? fix_bits<LIMBS>() - ex : 0;  // |q' 2^E| < 2^FIX
    const float qscale = ldexpf(1.0f, -E);
    int v = __float2int_rn(ldexpf(qv, E));
    int vh = v;                                   // sum over the element's 16-channel half
#pragma unroll
    for (int s = 2; s < 32; s <<= 1) vh += __shfl_xor(vh, s, 64);
    const int vo = __shfl_xor(vh, 32, 64);        // and over the other half
    if (lane == 0) qmeta[wave] = make_float4((float)(vh + vo) * qscale, qscale, (float)vh * qscale, (float)vo * qscale);
    const int e = row & 31;
    uint8_t* tb = reinterpret_cast<uint8_t*>(&qtab[0][0][0]);
#pragma unroll
    for (int l = LIMBS - 1; l >= 0; --l) {        // balanced base-256 digits, least significant first
      const int d = l == 0 ? v : ((v + 128) & 255) - 128;
      v = (v - d) >> 8;
      const uint8_t byte = (uint8_t)(d & 255);
      // the even lane of a pair writes the INT4 table, the odd one the INT2 tables
      if (half == 0) {
        if constexpr (T4) tb[((0 * G + wave) * QW + int4_word(e) * LIMBS + l) * 4 + int4_byte(e)] = byte;
      } else {
        if constexpr (T2) tb[((1 * G + wave) * QW + int2_word(e) * LIMBS + l) * 4 + int2_byte(e)] = byte;
        if constexpr (T2H) tb[((2 * G + wave) * QW + int2h_word(e) * LIMBS + l) * 4 + int2h_byte(e)] = byte;
      }
    }
  }
  __syncthreads();

  // This lane's group: its key tables and sums, read back from LDS.
  QFix<LIMBS> Q;
  float qsum, qscale, qsum_h[2];  // qsum_h: the two 16-channel halves of the lane's block
  {
    const float4 qm = qmeta[gsel];
    qsum = qm.x;
    qscale = qm.y;
    qsum_h[0] = qm.z;
    qsum_h[1] = qm.w;
    auto read_table = [&](int t, auto&& put) {
      const uint4* src = reinterpret_cast<const uint4*>(&qtab[t][gsel][0]);
#pragma unroll
      for (int w4 = 0; w4 < QW / 4; ++w4) {
        const uint4 x = src[w4];
        put(4 * w4 + 0, x.x);
        put(4 * w4 + 1, x.y);
        put(4 * w4 + 2, x.z);
        put(4 * w4 + 3, x.w);
      }
    };
    if constexpr (T4) read_table(0, [&](int w, uint32_t x) { Q.q4[w / (2 * LIMBS)][(w / LIMBS) % 2][w % LIMBS] = x; });
    if constexpr (T2) read_table(1, [&](int w, uint32_t x) { Q.q2[w / (4 * LIMBS)][(w / LIMBS) % 4][w % LIMBS] = x; });
    if constexpr (T2H) read_table(2, [&](int w, uint32_t x) { Q.q2h[w / (4 * LIMBS)][(w / LIMBS) % 4][w % LIMBS] = x; });
  }

  float acc[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) acc[e] = 0.0f;
  // Offsets enter one sum per 16-channel half of the block; with groups of 32
  // only, both halves share bias[0].
  constexpr bool G16 = any_g16<CB, NC>();
  float bias[2] = {0.0f, 0.0f};
  float lsum = 0.0f, m = -INFINITY;
  auto process = [&](Tile<D, NC, CB>& T, int base) {
    const int t0 = base + pi, t1 = t0 + TPW;
    const bool ok0 = lane_on && t0 < end, ok1 = lane_on && t1 < end;

    // ---- keys: per-component partial scores of this lane's group
    float kp0[NC], kp1[NC];
    float kb0[NC], kb1[NC], vb0[NC], vb1[NC];  // beta weights, K and V
    auto kpart = [&](auto& C, int c, auto kind_tag) {
      constexpr int KK = decltype(kind_tag)::value;
      if constexpr (kg16(KK)) {
        int a0, b0, a1, b1;
        kdot16(C.k0, Q, a0, b0);
        kdot16(C.k1, Q, a1, b1);
        kp0[c] = fmaf(f16hi(C.km0[0]) * qscale, (float)a0, f16lo(C.km0[0]) * qsum_h[0]) +
                 fmaf(f16hi(C.km0[1]) * qscale, (float)b0, f16lo(C.km0[1]) * qsum_h[1]);
        kp1[c] = fmaf(f16hi(C.km1[0]) * qscale, (float)a1, f16lo(C.km1[0]) * qsum_h[0]) +
                 fmaf(f16hi(C.km1[1]) * qscale, (float)b1, f16lo(C.km1[1]) * qsum_h[1]);
      } else {
        const float d0 = (float)kdot<kbits(KK), LIMBS>(C.k0, Q), d1 = (float)kdot<kbits(KK), LIMBS>(C.k1, Q);
        kp0[c] = fmaf(f16hi(C.km0[0]) * qscale, d0, f16lo(C.km0[0]) * qsum);
        kp1[c] = fmaf(f16hi(C.km1[0]) * qscale, d1, f16lo(C.km1[0]) * qsum);
      }
    };
    static_for<0, NC>([&](auto ic) {
      constexpr int c = decltype(ic)::value;
      kpart(tc<c>(T), c, std::integral_constant<int, ckind<CB, c>()>{});
    });
    // beta_c = prod_{j > c} alpha_j, from the last component down (the product
    // starts with alpha_{NC-1} itself: multiplying by 1.0f first is exact)
    kb0[NC - 1] = kb1[NC - 1] = vb0[NC - 1] = vb1[NC - 1] = 1.0f;
    static_for<0, NC - 1>([&](auto ic) {
      constexpr int c = NC - 2 - decltype(ic)::value;
      const auto& C = tc<c + 1>(T);
      kb0[c] = kb0[c + 1] * f16u(C.ka0); kb1[c] = kb1[c + 1] * f16u(C.ka1);
      vb0[c] = vb0[c + 1] * f16u(C.va0); vb1[c] = vb1[c + 1] * f16u(C.va1);
    });
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

    // ---- online softmax (log2 domain); the max is wave-uniform, so the rare
    // rescale is a scalar branch
    const float tmax = wave_max_uniform(fmaxf(s0, s1));
    if (tmax > m) {
      const float f = __builtin_amdgcn_exp2f(m - tmax);
      m = tmax;
      lsum *= f;
      bias[0] *= f;
      if constexpr (G16) bias[1] *= f;
#pragma unroll
      for (int e = 0; e < 32; ++e) acc[e] *= f;
    }
    const float p0 = ok0 ? __builtin_amdgcn_exp2f(s0 - m) : 0.0f;
    const float p1 = ok1 ? __builtin_amdgcn_exp2f(s1 - m) : 0.0f;
    lsum += p0 + p1;

    // ---- values. Token t of component c contributes p_t beta_c (o + s c) to
    // every element of a group. The code part goes through the mixed-precision
    // FMA (fp16 code operand, fp32 weight p beta s, fp32 accumulate, one rounding)
    // and the offset part into one sum per lane (per half with groups of 16),
    // both exact to fp32 rounding. (v_dot2c_f32_f16 would take two tokens per
    // instruction with fp16 weights, but with subnormal operands it rounds a small
    // addend into a large accumulator low by about two ulps, measured; over a long
    // range that biased the outputs by 1e-3 at 16k tokens.)
    float Wa[NC][2], Wb[NC][2];  // [component][half of the block]
    auto vweight = [&](auto& C, int c, auto kind_tag) {
      constexpr int KK = decltype(kind_tag)::value;
      const float pb0 = ok0 ? p0 * vb0[c] : 0.0f, pb1 = ok1 ? p1 * vb1[c] : 0.0f;
#pragma unroll
      for (int hh = 0; hh < (kg16(KK) ? 2 : 1); ++hh) {
        Wa[c][hh] = pb0 * f16hi(C.vm0[hh]);
        Wb[c][hh] = pb1 * f16hi(C.vm1[hh]);
        const float ob = fmaf(pb0, f16lo(C.vm0[hh]), pb1 * f16lo(C.vm1[hh]));
        if constexpr (kg16(KK)) {
          bias[hh] += ob;
        } else {
          bias[0] += ob;
          if constexpr (G16) bias[1] += ob;
        }
      }
      if constexpr (!kg16(KK)) {
        Wa[c][1] = Wa[c][0];
        Wb[c][1] = Wb[c][0];
      }
    };
    static_for<0, NC>([&](auto ic) {
      constexpr int c = decltype(ic)::value;
      vweight(tc<c>(T), c, std::integral_constant<int, ckind<CB, c>()>{});
    });

#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        uint32_t x[NC][4];
        static_for<0, NC>([&](auto ic) {
          constexpr int c = decltype(ic)::value;
          vpairs<ckind<CB, c>(), REF>(tc<c>(T).v0, tc<c>(T).v1, half, blk, x[c]);
        });
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float& a = acc[16 * half + 4 * blk + q];
          auto comp = [&](int c, bool w4) {
            a = fmaf(f16lo(x[c][q]), w4 ? 4.0f * Wa[c][half] : Wa[c][half], a);
            a = fmaf(f16hi(x[c][q]), w4 ? 4.0f * Wb[c][half] : Wb[c][half], a);
          };
          static_for<0, NC>([&](auto ic) {
            constexpr int c = decltype(ic)::value;
            comp(c, vw4<kbits(ckind<CB, c>()), REF>(q));
          });
        }
      }
  };
  if constexpr (DEPTH == 2) {
    for (;;) {
      if (base >= end) break;
      fetch(B, base + STRIDE);
      process(A, base);
      base += STRIDE;
      if (base >= end) break;
      fetch(A, base + STRIDE);
      process(B, base);
      base += STRIDE;
    }
  } else {
    for (;;) {
      if (base >= end) break;
      fetch(C, base + 2 * STRIDE);
      process(A, base);
      base += STRIDE;
      if (base >= end) break;
      fetch(A, base + 2 * STRIDE);
      process(B, base);
      base += STRIDE;
      if (base >= end) break;
      fetch(B, base + 2 * STRIDE);
      process(C, base);
      base += STRIDE;
    }
  }

  if (!active) return;
  float val[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) val[e] = fmaf(acc[e], kTwo24 / vclass<REF>(e), bias[G16 ? (e >> 4) : 0]);
  write_partial<D, 32, G, TPW>(val, (lane_on && gi == 0) ? lsum : 0.0f, m, lane_on, red, S,
                               p.part + ((size_t)bh * p.nsplit + split) * part_floats(D));
}

// RH: the rotation H_K is stored fp16 (RQ_FLAG_ROT_F16), else fp32.
template <int D, int NC, uint32_t CB, int DEPTH, int LIMBS, int RH>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(waves_for<NC, CB, LIMBS>()))) void decode_fused(
    DecodeParams p) {
  decode_body<D, NC, CB, DEPTH, kContig, LIMBS, RH>(p);
}

template <int D, int NC, uint32_t CB, int DEPTH, int LIMBS, int RH>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(waves_for_paged<NC, CB, LIMBS>()))) void
decode_fused_paged(DecodeParams p) {
  decode_body<D, NC, CB, DEPTH, kPagedLane, LIMBS, RH>(p);
}


// ---------------------------------------------------------------- plan tables
typedef void (*MainFn)(DecodeParams);
struct PlanEntry {
  int D, nc;
  uint32_t cb;
  int limbs;
  int rh;  // rotation stored fp16
  MainFn fn;
};

#ifndef RQ_DEPTH
#define RQ_DEPTH 2
#endif
// Plans with kernels: one nibble per component, anchor first (0xA = INT2 in
// groups of 16). RQ_E(D, NC, CB, LIMBS) gives the table entries of a plan, one
// per rotation storage (fp32, fp16); every plan has a 14-bit (2 limbs) and a
// 21-bit (3 limbs) query instance.
// Covered: one or two components of any kinds (every Last-loop and First-loop
// plan), and chains of three or four whose INT4 components all precede their
// INT2 ones, the INT2 ones in one group size (the descending Previous-loop plans).
#define RQ_PLANS_L(D, LB)                                                                                   \
  RQ_E(D, 1, 0x2, LB), RQ_E(D, 1, 0x4, LB), RQ_E(D, 2, 0x22, LB), RQ_E(D, 2, 0x24, LB), RQ_E(D, 2, 0x42, LB), \
      RQ_E(D, 2, 0x44, LB), RQ_E(D, 3, 0x244, LB), RQ_E(D, 3, 0x224, LB), RQ_E(D, 3, 0x222, LB),               \
      RQ_E(D, 3, 0x444, LB), RQ_E(D, 4, 0x2244, LB), RQ_E(D, 4, 0x2224, LB), RQ_E(D, 4, 0x2222, LB),           \
      RQ_E(D, 4, 0x4444, LB), RQ_E(D, 1, 0xA, LB), RQ_E(D, 2, 0xAA, LB), RQ_E(D, 2, 0xA4, LB),                 \
      RQ_E(D, 3, 0xAA4, LB), RQ_E(D, 4, 0xAAA4, LB), RQ_E(D, 3, 0xAAA, LB), RQ_E(D, 4, 0xAAAA, LB),          \
      RQ_E(D, 3, 0xA44, LB), RQ_E(D, 4, 0xAA44, LB), RQ_E(D, 4, 0x2444, LB), RQ_E(D, 4, 0xA444, LB),           \
      RQ_E(D, 2, 0x2A, LB), RQ_E(D, 2, 0x4A, LB), RQ_E(D, 2, 0xA2, LB)
#define RQ_PLANS(D) RQ_PLANS_L(D, 2), RQ_PLANS_L(D, 3)

template <size_t N>
const PlanEntry* find_plan(const PlanEntry (&table)[N], int D, int nc, const int* kinds, int limbs, int rh) {
  uint32_t cb = 0;
  for (int c = 0; c < nc; ++c) cb |= (uint32_t)kinds[c] << (4 * c);
  for (const PlanEntry& e : table)
    if (e.D == D && e.nc == nc && e.cb == cb && e.limbs == limbs && e.rh == rh) return &e;
  return nullptr;
}

}  // namespace
}  // namespace rq
