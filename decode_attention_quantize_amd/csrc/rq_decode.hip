// Decode launches of librq over a contiguous cache ([B][H][T_max] rows per
// loop): the streaming kernel instances, the combine kernel and the dispatch.
// The streaming kernel itself is in rq_decode_kernel.hpp; the paged instances
// are in rq_decode_paged.hip.
#include "rq_decode_kernel.hpp"

namespace rq {
namespace {

// ---------------------------------------------------------------- combine
// Per (b, h): merge the split partials with the current token (scored in the
// original domain from bf16 q and k_cur) and, for the compressed cache, rotate
// the value sum back once: out = (H_V^T acc + p_cur v_cur) / l.
//
// Its reads are latency-bound. With few (b, h), the H_V^T product of each is
// spread over D / COLS workgroups (COLS = 32), each producing COLS output
// columns from a D x COLS block of H_V (16 KB at D = 128), so that no compute
// unit waits for a whole matrix; each merges all D elements of the partials (a
// few hundred bytes per slot). At D = 128, where D / 32 workgroups per (b, h)
// would exceed the compute units but two would not, COLS = 64. With more (b, h),
// or no rotation, one workgroup per (b, h) (COLS = D) costs less: more
// workgroups than compute units only add to the launch. split_item places a (b, h)'s workgroups on the XCD whose
// workgroups wrote its partials (both launches map consecutive (b, h) blocks to
// XCDs in proportion, when their workgroup counts are multiples of the XCD
// count), where the partials are still in L2.
// RH: the value rotation is stored fp16 (RQ_FLAG_ROT_F16), else fp32.
template <int D, int COLS, int RH>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
  constexpr int NS = D / COLS;               // workgroups per (b, h)
  constexpr int NR = kThreads / COLS;        // row parts of the product
  constexpr int RPT = D / NR;                // rows per thread
  constexpr int PF = (int)part_floats(D);
  static_assert(D % COLS == 0 && D % NR == 0 && RPT % 4 == 0, "product layout");
  __shared__ float acc_s[D];
  __shared__ float red_s[NR][COLS];
  __shared__ float wsum[kWaves];
  int slice, b, h;
  split_item(NS, p.B, p.H, slice, b, h);
  const int bh = b * p.H + h, tid = threadIdx.x;
  const int c = tid % COLS, r = tid / COLS, col = slice * COLS + c;
  const bool rot = p.rotv != nullptr, prod = r < NR;  // threads past NR * COLS only merge

  // Loads in the order their values are needed: the partials of the first CH
  // slots, q/k_cur/v_cur, then the thread's block of H_V. A round's loads are
  // all issued before the first is used, so a call waits for memory about once
  // per CH slots (slots past the last one are loaded clamped and ignored).
  constexpr int CH = 16;
  const bool on = tid < D;
  const float* part = p.part + (size_t)bh * p.nsplit * PF;
  float ms[CH], ls[CH], as[CH];
  auto load_slots = [&](int s0) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const float* ps = part + (size_t)min(s0 + i, p.nsplit - 1) * PF;
      ms[i] = ps[0];
      ls[i] = ps[1];
      as[i] = ps[4 + (on ? tid : 0)];
    }
  };
  load_slots(0);
  const int raw_len = p.past_len[b];
  const size_t qo = (size_t)bh * D + (on ? tid : 0);
  const uint16_t qh = p.q[qo], kh = p.kcur[qo], vh = p.vcur[(size_t)bh * D + col];
  float hv[RPT];
  if (rot && prod) {
    const size_t e0 = ((size_t)h * D + (size_t)r * RPT) * D + col;
    if constexpr (RH) {  // fp16 entries, converted exactly
      const uint16_t* Hm = static_cast<const uint16_t*>(p.rotv) + e0;
#pragma unroll
      for (int i = 0; i < RPT; ++i) hv[i] = f16u(Hm[(size_t)i * D]);
    } else {
      const float* Hm = static_cast<const float*>(p.rotv) + e0;
#pragma unroll
      for (int i = 0; i < RPT; ++i) hv[i] = Hm[(size_t)i * D];
    }
  }

  if ((raw_len < 0 || raw_len > p.T_max) && h == 0 && slice == 0 && tid == 0 && p.dev_err)
    atomicOr(p.dev_err, RQ_DEVERR_LENGTH);
  const int len = raw_len < 0 ? 0 : (raw_len > p.T_max ? p.T_max : raw_len);
  const int nvalid = slots_used(len, p.nsplit, p.unit);

  // Online merge of the splits' (m, l, acc) relative to their running max M
  // (the same M and l in every thread).
  float M = -INFINITY, l = 0.0f, a = 0.0f;
  for (int s0 = 0;;) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (s0 + i < nvalid && ms[i] > -INFINITY) {
        const float Mn = fmaxf(M, ms[i]);
        const float fo = exp2f(M - Mn), fs = exp2f(ms[i] - Mn);
        l = fmaf(l, fo, ls[i] * fs);
        a = fmaf(a, fo, as[i] * fs);
        M = Mn;
      }
    }
    s0 += CH;
    if (s0 >= nvalid) break;
    load_slots(s0);
  }
  float x = on ? bf16f(qh) * bf16f(kh) : 0.0f;
  const float vc = bf16f(vh);
  if (on) acc_s[tid] = a;
  x = wave_sum(x);
  if ((tid & 63) == 0) wsum[tid >> 6] = x;
  __syncthreads();

  float scur = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) scur += wsum[w];
  scur *= p.scale_log2;
  const float Mt = fmaxf(M, scur);
  const float g = (M == -INFINITY) ? 0.0f : exp2f(M - Mt);
  const float pcur = exp2f(scur - Mt);
  const float lt = fmaf(l, g, pcur);

  float o = 0.0f;
  if (rot) {
    if (prod) {
      float o0 = 0.0f, o1 = 0.0f, o2 = 0.0f, o3 = 0.0f;
#pragma unroll
      for (int i = 0; i < RPT; i += 4) {
        o0 = fmaf(hv[i + 0], acc_s[r * RPT + i + 0], o0);
        o1 = fmaf(hv[i + 1], acc_s[r * RPT + i + 1], o1);
        o2 = fmaf(hv[i + 2], acc_s[r * RPT + i + 2], o2);
        o3 = fmaf(hv[i + 3], acc_s[r * RPT + i + 3], o3);
      }
      red_s[r][c] = (o0 + o1) + (o2 + o3);
    }
    __syncthreads();
    if (tid < COLS) {
#pragma unroll
      for (int q = 0; q < NR; ++q) o += red_s[q][tid];
    }
  } else if (tid < COLS) {
    o = acc_s[col];
  }
  if (tid < COLS) p.out[(size_t)bh * D + col] = fmaf(g, o, pcur * vc) / lt;
}

// ---------------------------------------------------------------- dispatch
#define RQ_E(D, NC, CB, LB) \
  {D, NC, CB, LB, 0, decode_fused<D, NC, CB, RQ_DEPTH, LB, 0>}, {D, NC, CB, LB, 1, decode_fused<D, NC, CB, RQ_DEPTH, LB, 1>}
const PlanEntry kTable[] = {RQ_PLANS(64), RQ_PLANS(96), RQ_PLANS(128)};
#undef RQ_E

}  // namespace

bool have_decode_kernel(int D, int nc, const int* bits, int limbs, bool paged) {
  if (nc > 4) return !paged && have_decode_kernel_long(D, nc, bits, limbs);
  return find_plan(kTable, D, nc, bits, limbs, 0) != nullptr;
}

int launch_decode(const DecodeParams& p, int D, int nc, const int* bits, int limbs, int nsplit, void* stream) {
  if (nc > 4) return launch_decode_long(p, D, nc, bits, limbs, nsplit, stream);
  if (p.table) return launch_decode_paged(p, D, nc, bits, limbs, nsplit, stream);
  const PlanEntry* e = find_plan(kTable, D, nc, bits, limbs, p.rot_f16);
  if (!e) return -1;
  const dim3 grid((unsigned)(nsplit * p.B * p.H));
  hipLaunchKernelGGL(e->fn, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

namespace {
template <int D, int RH>
void launch_combine_d(const CombineParams& p, int cols, const dim3& grid, hipStream_t s) {
  if (cols == 32) hipLaunchKernelGGL((combine_kernel<D, 32, RH>), grid, dim3(kThreads), 0, s, p);
  else if (cols == 64 && D == 128)  // (D == 128 ? 64 : D) only instantiates what D divides
    hipLaunchKernelGGL((combine_kernel<D, (D == 128 ? 64 : D), RH>), grid, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL((combine_kernel<D, D, RH>), grid, dim3(kThreads), 0, s, p);
}
}  // namespace

int launch_combine(const CombineParams& p, int D, int cols, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(p.B * p.H * (D / cols)));
  const bool rh = p.rot_f16 && p.rotv;
  switch (D) {
    case 64: rh ? launch_combine_d<64, 1>(p, cols, grid, s) : launch_combine_d<64, 0>(p, cols, grid, s); break;
    case 96: rh ? launch_combine_d<96, 1>(p, cols, grid, s) : launch_combine_d<96, 0>(p, cols, grid, s); break;
    case 128:
      rh ? launch_combine_d<128, 1>(p, cols, grid, s) : launch_combine_d<128, 0>(p, cols, grid, s);
      break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

}  // namespace rq
