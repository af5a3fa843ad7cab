// Prefill attention of one loop (paper "KV Cache Quantization for Looped
// Transformers with 2-Bit Residuals", §4.2 "Prefill": every loop attends
// causally over its own BF16 prompt K/V; after the final loop the prompt is
// quantized into the cache, which rq_quantize_append does).
//
// A flash-attention forward pass on the matrix cores of gfx950. One workgroup
// owns 128 queries of one (b, h); each of its four waves owns 32 of them and
// walks the key tiles of 64 tokens that causality lets it see. Per tile:
//   S^T = K Q^T    v_mfma_f32_16x16x32_bf16: K rows (A operand) from LDS, the
//                  wave's queries (B operand) held in registers for the whole
//                  pass; bf16 products are exact, sums in fp32;
//   online softmax in the log2 domain, per query column (a lane's column is
//                  lane % 16, so the rescale of its accumulators is lane-local);
//   O^T += V^T P^T v_mfma_f32_16x16x32_f16: P in fp16 (2^-11 relative
//                  rounding; bf16 would cost 2^-9) and V^T (A operand) in fp16,
//                  transposed and converted once per call by a first pass
//                  (prefill_vt_kernel) into the caller's workspace, so the
//                  workgroups that read a key tile (up to T / 128 of them) only
//                  copy it into LDS.
// The key rows of each 16-row S tile are permuted (rows 4i..4i+3 of tile 2c+h
// are keys 32c + 8i + 4h + 0..3) so that the S accumulators a lane holds are
// exactly the eight consecutive keys its P operand needs: no lane exchange
// between the two products.
#include <hip/hip_runtime.h>

#include "rq_device.hpp"
#include "rq_internal.hpp"

namespace rq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// LDS row paddings (elements): 32 bytes keep the 16-byte operand reads of a
// 16-row tile free of bank conflicts (measured: 16 bytes left half the LDS
// cycles in conflicts, none with 32).
#ifndef RQ_PF_KPAD
#define RQ_PF_KPAD 16
#endif
#ifndef RQ_PF_VPAD
#define RQ_PF_VPAD 16
#endif

constexpr int kBQ = 128;          // queries per workgroup (32 per wave)
constexpr int kBK = 64;           // keys per tile

// Key of row r (0..15) of S tile mt (0..3) within a key tile.
__host__ __device__ constexpr int tile_key(int mt, int r) { return 32 * (mt >> 1) + 8 * (r >> 2) + 4 * (mt & 1) + (r & 3); }
// LDS row of key k of the tile: the tile's rows read together (one 16-row S
// tile) are stored consecutively, so the A-operand reads do not collide on banks.
__host__ __device__ constexpr int k_row(int k) { return (k & 32) | ((k & 4) << 2) | ((k >> 1) & 12) | (k & 3); }

// IEEE 754-2019 maximum (NaN-propagating): unlike fmaxf it needs no quieting
// of its operands in the kernel's IEEE mode, and chains of it fold into
// three-input instructions. Scores are finite or -inf.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Maximum over the four lanes of a query column (lanes l, l ^ 16, l ^ 32,
// l ^ 48): the lane-swap instructions exchange half-waves and 16-lane rows in
// the vector unit, without a round trip through LDS.
__device__ __forceinline__ float col_max(float t) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(t), __float_as_int(t), false, false);
  t = vmax(__int_as_float(a[0]), __int_as_float(a[1]));           // max(x[l], x[l ^ 32])
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(t), __float_as_int(t), false, false);
  return vmax(__int_as_float(b[0]), __int_as_float(b[1]));        // and of l ^ 16
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

#ifndef RQ_PF_GROUP
#define RQ_PF_GROUP 1
#endif

// Work item (query block, b h) of this workgroup. Consecutive workgroup ids go
// round-robin over the 8 XCDs, each with its own L2. Every (b, h) stays on one
// XCD, and an XCD takes its (b, h) series RQ_PF_GROUP at a time, all of a
// series' query blocks, heaviest (most keys under the causal mask) first. The
// workgroups resident on an XCD at once then read the same series' K and V
// tiles at about the same pace, and those reads hit the L2. Ordered by query
// block alone, an XCD interleaved all of its series: the misses fetched 22.5
// GiB per 16k launch (B8, H16), against 3.4 GiB this way (22 % faster).
// Shapes with B H not a multiple of 8 RQ_PF_GROUP keep that plain order.
__device__ __forceinline__ void prefill_item(const PrefillParams& p, int& qblk, int& bh) {
  const int nqb = (p.T + kBQ - 1) / kBQ;
  const int BH = p.B * p.H;
  const int i = (int)blockIdx.x;
  constexpr int GB = RQ_PF_GROUP;
  if (GB > 0 && BH % (kXcds * GB) == 0) {
    const int x = i % kXcds, j = i / kXcds;            // XCD, position in its dispatch order
    const int g = j / (GB * nqb), r = j % (GB * nqb);   // series group, position in the group
    qblk = nqb - 1 - r / GB;
    bh = x + kXcds * (g * GB + r % GB);
  } else {
    qblk = nqb - 1 - i / BH;
    bh = i % BH;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void prefill_attn_kernel(
    PrefillParams p) {
  constexpr int KS = D / 32;      // k-steps of S (32 channels each)
  constexpr int MD = D / 16;      // 16-channel tiles of O^T
  constexpr int KP = D + RQ_PF_KPAD;   // padded LDS row of K (bf16)
  constexpr int VP = kBK + RQ_PF_VPAD; // padded LDS row of V^T (fp16)
  constexpr int KC = kBK * (D / 8);                       // 16-byte chunks of a K tile
  constexpr int VC = D * (kBK / 8);                       // 16-byte chunks (8 keys of a channel) of a V^T tile
  constexpr int KPF = (KC + kThreads - 1) / kThreads;     // per thread
  constexpr int VPF = (VC + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBK * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];

  int qblk, bh;
  prefill_item(p, qblk, bh);
  const int nqb = (p.T + kBQ - 1) / kBQ;
  const int BH = p.B * p.H;
  const int b = bh / p.H;
  int len = p.lens[b];
  // flagged once per sequence: by the last query block of its head 0
  if ((len < 0 || len > p.T) && threadIdx.x == 0 && qblk == nqb - 1 && bh % p.H == 0 && p.dev_err)
    atomicOr(p.dev_err, RQ_DEVERR_LENGTH);
  len = len < 0 ? 0 : (len > p.T ? p.T : len);
  const int q0 = qblk * kBQ;
  if (q0 >= len) return;                               // whole block, before any barrier

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int qw = q0 + 32 * wave;                       // this wave's first query
  const size_t head = (size_t)bh * p.T * D;            // element offset of (b, h) in q, k, v, out

  // ---- the wave's queries as B operands, held for the whole pass: query
  // qw + 16 nt + col (rows past the tensor clamp to its last row), channels
  // 32 ks + 8 grp ..
  bf16x8 qb[2][KS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const uint4* src = reinterpret_cast<const uint4*>(p.q + head + (size_t)min(qw + 16 * nt + col, p.T - 1) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[nt][ks] = __builtin_bit_cast(bf16x8, src[4 * ks + grp]);
  }

  // ---- next tile's K and V, held in registers while the current tile is computed
  // Raw buffer loads over the sequence's own rows [0, len) of K and V: rows past
  // the end (and items past the tile) read as zeros through the hardware range
  // check, so the loads need no branches.
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.k + head), (short)0, (int)((uint32_t)len * D * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      p.vt + (size_t)bh * D * p.Tp, (short)0, (int)((uint32_t)p.Tp * D * 2), 0x00020000);
  constexpr uint32_t kOut = 0x80000000u;               // an offset past any sequence
  uint4 kpf[KPF], vpf[VPF];
  auto ld16 = [](__amdgpu_buffer_rsrc_t r, uint32_t off) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
  };
  auto prefetch = [&](int k0) {
#pragma unroll
    for (int j = 0; j < KPF; ++j) {
      const int c = tid + j * kThreads;
      const int key = c / (D / 8), d0 = 8 * (c % (D / 8));
      kpf[j] = ld16(krs, (KC % kThreads == 0 || c < KC) ? (uint32_t)((k0 + key) * D + d0) * 2u : kOut);
    }
#pragma unroll
    for (int j = 0; j < VPF; ++j) {
      const int c = tid + j * kThreads;
      const int d = c / (kBK / 8), kc = c % (kBK / 8);
      vpf[j] = ld16(vrs, (VC % kThreads == 0 || c < VC) ? (uint32_t)(d * p.Tp + k0 + 8 * kc) * 2u : kOut);
    }
  };
  auto stage = [&]() {                                 // K row-major (rows in read order); V^T
#pragma unroll
    for (int j = 0; j < KPF; ++j) {
      const int c = tid + j * kThreads;
      if (KC % kThreads == 0 || c < KC) *reinterpret_cast<uint4*>(&Ks[k_row(c / (D / 8)) * KP + 8 * (c % (D / 8))]) = kpf[j];
    }
#pragma unroll
    for (int j = 0; j < VPF; ++j) {
      const int c = tid + j * kThreads;
      if (VC % kThreads == 0 || c < VC) *reinterpret_cast<uint4*>(&Vt[(c / (kBK / 8)) * VP + 8 * (c % (kBK / 8))]) = vpf[j];
    }
  };

  f32x4 o[2][MD];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int md = 0; md < MD; ++md) o[nt][md] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-INFINITY, -INFINITY};             // per query column (log2 domain)
  // Column sums of P^T on the matrix cores: an all-ones A operand gives, in every
  // row of the 16x16 result, sum_k P[k][query]: the softmax denominator of the
  // same fp16 P the value product uses, with no lane reduction.
  f32x4 lsum[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  const f16x8 ones = {(_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f,
                      (_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f};

  const int kend = min(len, q0 + kBQ);                 // keys any query of the block may see
  const int nkt = (kend + kBK - 1) / kBK;
  prefetch(0);
  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * kBK;
    __syncthreads();                                   // the previous tile is consumed
    stage();
    __syncthreads();
    if (kt + 1 < nkt) prefetch(k0 + kBK);              // lands while this tile is computed
    // (A wave whose queries see nothing of this tile, at most the last one or two
    // tiles of a block, still runs it fully masked: a skip would split the
    // accumulators' live ranges into two paths and cost register copies on every tile.)

    // ---- S^T tiles: [mt][nt], rows = keys tile_key(mt, 4 grp + i), column = query.
    // B operands: query qw + 16 nt + col, channels 32 ks + 8 grp .. + 7
    f32x4 s[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      bf16x8 ka[KS];
      const uint16_t* kr = &Ks[k_row(tile_key(mt, col)) * KP + 8 * grp];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ka[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kr + 32 * ks));
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks], qb[nt][ks], acc, 0, 0, 0);
        s[mt][nt] = acc;
      }
    }

    // ---- causal and length mask (tiles that reach past a query or the sequence)
    if (k0 + kBK - 1 > qw || k0 + kBK > len) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int lim = min(qw + 16 * nt + col, len - 1) - (k0 + 8 * grp);   // last visible key, relative
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (32 * (mt >> 1) + 4 * (mt & 1) + i > lim) s[mt][nt][i] = -INFINITY;
      }
    }

    // ---- online softmax per query column (log2 domain; the scale is positive, so the
    // column max of the raw scores gives the max of the scaled ones)
    f16x8 pb[2][2];                                    // [nt][32-key chunk]: P^T as B operands
    float fcol[2], bases[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float tmax = s[0][nt][0];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = (mt == 0 ? 1 : 0); i < 4; ++i) tmax = vmax(tmax, s[mt][nt][i]);
      tmax = col_max(tmax);
      const float mnew = vmax(mrow[nt], tmax * p.scale_log2);
      const float base = mnew == -INFINITY ? 0.f : mnew;          // a column with nothing visible yet
      fcol[nt] = __builtin_amdgcn_exp2f(mrow[nt] - base);
      mrow[nt] = mnew;
      bases[nt] = base;
    }
    // the accumulators are rescaled only when some column's max moved (rare after
    // the first tiles)
    if (__builtin_amdgcn_ballot_w64(fcol[0] != 1.0f || fcol[1] != 1.0f)) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
        for (int md = 0; md < MD; ++md) o[nt][md] *= fcol[nt];
        lsum[nt] *= fcol[nt];
      }
    }

    // ---- per 32-key chunk c: P^T (exponentials, fp16) and O^T += V^T P^T with
    // A = V^T rows (channel 16 md + col), keys 32 c + 8 grp ... The matrix-core
    // products of chunk 0 are issued interleaved with the exponentials of chunk 1
    // (independent work for the vector unit while each product runs).
    auto exps = [&](int c) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            pb[nt][c][4 * h + i] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[2 * c + h][nt][i], p.scale_log2, -bases[nt]));
    };
    auto pv = [&](int c) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) lsum[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[nt][c], lsum[nt], 0, 0, 0);
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const f16x8 va =
            __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(&Vt[(16 * md + col) * VP + 8 * grp + 32 * c]));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) o[nt][md] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[nt][c], o[nt][md], 0, 0, 0);
      }
    };
    exps(0);
    __builtin_amdgcn_sched_barrier(0);
    pv(0);
    exps(1);
#ifndef RQ_PF_NO_INTERLEAVE
    // 2 + 2 MD products, MD reads of V^T, 16 exponentials with their fma and 8 packs
    __builtin_amdgcn_sched_group_barrier(0x100, MD, 0);   // V^T operand reads first
#pragma unroll
    for (int k = 0; k < 2 + 2 * MD; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three vector instructions
    }
#endif
    __builtin_amdgcn_sched_barrier(0);
    pv(1);
  }

  // ---- normalize and store: lane holds O^T[16 md + 4 grp + i][query col of tile nt]
  if (qw >= len) return;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float l = lsum[nt][0];
    const int qi = qw + 16 * nt + col;
    if (qi >= len) continue;
    const float inv = 1.0f / l;
    float* dst = p.out + head + (size_t)qi * D + 4 * grp;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      const f32x4 v = o[nt][md] * inv;
      *reinterpret_cast<float4*>(dst + 16 * md) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// First pass: V^T in fp16, vt[b][h][d][key] with keys padded to Tp (a
// multiple of the key tile); keys at or past the sequence's length are zero,
// so the attention pass reads whole tiles without checks. One workgroup per
// (key tile, b, h): rows are read coalesced, transposed through LDS, and
// written as 128-byte channel rows.
template <int D>
__global__ __launch_bounds__(kThreads) void prefill_vt_kernel(PrefillParams p) {
  constexpr int VP = kBK + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];
  const int k0 = (int)blockIdx.x * kBK, bh = (int)blockIdx.y, b = bh / p.H, tid = threadIdx.x;
  int len = p.lens[b];
  len = len < 0 ? 0 : (len > p.T ? p.T : len);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.v + (size_t)bh * p.T * D), (short)0, (int)((uint32_t)len * D * 2), 0x00020000);
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  for (int c = tid; c < (kBK / 2) * (D / 8); c += kThreads) {
    const int key = 2 * (c % (kBK / 2)), dc = c / (kBK / 2);
    const uint32_t off = (uint32_t)((k0 + key) * D + 8 * dc) * 2u;
    const u32x4 w0 = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0);
    const u32x4 w1 = __builtin_amdgcn_raw_buffer_load_b128(vrs, off + D * 2, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = (uint32_t)f32_to_f16_bits(bf16lo(w0[i])) | ((uint32_t)f32_to_f16_bits(bf16lo(w1[i])) << 16);
      const uint32_t hi = (uint32_t)f32_to_f16_bits(bf16hi(w0[i])) | ((uint32_t)f32_to_f16_bits(bf16hi(w1[i])) << 16);
      *reinterpret_cast<uint32_t*>(&Vt[(8 * dc + 2 * i) * VP + key]) = lo;
      *reinterpret_cast<uint32_t*>(&Vt[(8 * dc + 2 * i + 1) * VP + key]) = hi;
    }
  }
  __syncthreads();
  uint16_t* dst = p.vt + (size_t)bh * D * p.Tp + k0;
  for (int c = tid; c < D * (kBK / 8); c += kThreads) {
    const int d = c / (kBK / 8), kc = c % (kBK / 8);
    *reinterpret_cast<uint4*>(dst + (size_t)d * p.Tp + 8 * kc) = *reinterpret_cast<const uint4*>(&Vt[d * VP + 8 * kc]);
  }
}

}  // namespace

size_t prefill_workspace_bytes(int B, int H, int D, int T) {
  const size_t Tp = (size_t)(T + kBK - 1) / kBK * kBK;
  return (size_t)B * H * D * Tp * 2;
}

int launch_prefill(const PrefillParams& p, int D, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nqb = (p.T + kBQ - 1) / kBQ;
  const dim3 grid((unsigned)(nqb * p.B * p.H));
  const dim3 vgrid((unsigned)(p.Tp / kBK), (unsigned)(p.B * p.H));
  switch (D) {
    case 64:
      hipLaunchKernelGGL(prefill_vt_kernel<64>, vgrid, dim3(kThreads), 0, s, p);
      hipLaunchKernelGGL(prefill_attn_kernel<64>, grid, dim3(kThreads), 0, s, p);
      break;
    case 96:
      hipLaunchKernelGGL(prefill_vt_kernel<96>, vgrid, dim3(kThreads), 0, s, p);
      hipLaunchKernelGGL(prefill_attn_kernel<96>, grid, dim3(kThreads), 0, s, p);
      break;
    case 128:
      hipLaunchKernelGGL(prefill_vt_kernel<128>, vgrid, dim3(kThreads), 0, s, p);
      hipLaunchKernelGGL(prefill_attn_kernel<128>, grid, dim3(kThreads), 0, s, p);
      break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

}  // namespace rq
