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
// Its reads are latency-bound; they are ordered and batched as described below.
template <int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
  constexpr int NQ = kThreads / D;  // row slices of the H_V^T product
  constexpr int RS = D / NQ;        // rows per slice
  constexpr int PF = (int)part_floats(D);
  __shared__ float acc_s[D];
  __shared__ float red_s[kThreads];
  __shared__ float wsum[kWaves];
  const int bh = blockIdx.x, b = bh / p.H, h = bh % p.H, tid = threadIdx.x;
  const int j = tid % D, sl = tid / D;
  const bool rot = p.rotv != nullptr;

  // Loads in the order their values are needed: the partials of the first CH
  // slots, q/k_cur/v_cur, then the thread's slice of H_V. A round's loads are all
  // issued before the first is used, so a call waits for memory about once per
  // CH slots (slots past the last one are loaded clamped and ignored).
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
  const uint16_t qh = p.q[qo], kh = p.kcur[qo], vh = p.vcur[qo];
  float hv[RS];
  if (rot && sl < NQ) {
    const float* Hm = p.rotv + ((size_t)h * D + (size_t)sl * RS) * D + j;
#pragma unroll
    for (int i = 0; i < RS; ++i) hv[i] = Hm[(size_t)i * D];
  }

  if ((raw_len < 0 || raw_len > p.T_max) && h == 0 && tid == 0 && p.dev_err) atomicOr(p.dev_err, RQ_DEVERR_LENGTH);
  const int len = raw_len < 0 ? 0 : (raw_len > p.T_max ? p.T_max : raw_len);
  const int nvalid = slots_used(len, p.nsplit, p.unit);

  // Online merge of the splits' (m, l, acc) relative to their running max M.
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
    if (sl < NQ) {
      float o0 = 0.0f, o1 = 0.0f, o2 = 0.0f, o3 = 0.0f;
#pragma unroll
      for (int i = 0; i < RS; i += 4) {
        o0 = fmaf(hv[i + 0], acc_s[sl * RS + i + 0], o0);
        o1 = fmaf(hv[i + 1], acc_s[sl * RS + i + 1], o1);
        o2 = fmaf(hv[i + 2], acc_s[sl * RS + i + 2], o2);
        o3 = fmaf(hv[i + 3], acc_s[sl * RS + i + 3], o3);
      }
      red_s[tid] = (o0 + o1) + (o2 + o3);
    }
    __syncthreads();
    if (on) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) o += red_s[q * D + tid];
    }
  } else if (on) {
    o = acc_s[tid];
  }
  if (on) p.out[(size_t)bh * D + tid] = fmaf(g, o, pcur * vc) / lt;
}

// ---------------------------------------------------------------- dispatch
#define RQ_E(D, NC, CB, LB) {D, NC, CB, LB, decode_fused<D, NC, CB, RQ_DEPTH, LB>}
const PlanEntry kTable[] = {RQ_PLANS(64), RQ_PLANS(96), RQ_PLANS(128)};
#undef RQ_E

}  // namespace

bool have_decode_kernel(int D, int nc, const int* bits, int limbs, bool paged) {
  if (nc > 4) return !paged && have_decode_kernel_long(D, nc, bits, limbs);
  return find_plan(kTable, D, nc, bits, limbs) != nullptr;
}

int launch_decode(const DecodeParams& p, int D, int nc, const int* bits, int limbs, int nsplit, void* stream) {
  if (nc > 4) return launch_decode_long(p, D, nc, bits, limbs, nsplit, stream);
  if (p.table) return launch_decode_paged(p, D, nc, bits, limbs, nsplit, stream);
  const PlanEntry* e = find_plan(kTable, D, nc, bits, limbs);
  if (!e) return -1;
  const dim3 grid((unsigned)(nsplit * p.B * p.H));
  hipLaunchKernelGGL(e->fn, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

int launch_combine(const CombineParams& p, int D, int B, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(B * p.H));
  switch (D) {
    case 64: hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(kThreads), 0, s, p); break;
    case 96: hipLaunchKernelGGL(combine_kernel<96>, grid, dim3(kThreads), 0, s, p); break;
    case 128: hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(kThreads), 0, s, p); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

}  // namespace rq
