// Decode launches of librq for Previous-loop chains longer than four stored
// components (paper "KV Cache Quantization for Looped Transformers with 2-Bit
// Residuals", App. D "Logical reference count": decoding the j-th loop of a
// chain reads j components, 528 reads at L = 32 against 63 for a shared
// anchor; §3.2 "Reference KV"). The streaming kernel is the one of
// rq_decode_kernel.hpp with five to eight components, one wave per SIMD (two
// tiles of up to eight components do not fit a smaller register budget), over
// a contiguous cache; the combine launch is shared.
#include "rq_decode_kernel.hpp"

namespace rq {
namespace {

// Chains of an INT4 or INT2 anchor, at most one more INT4 loop, then INT2
// loops (anchor first): the plans of the chained comparators of the workloads.
#define RQ_LONG(D, LB)                                                                                      \
  RQ_E(D, 5, 0x22222, LB), RQ_E(D, 6, 0x222222, LB), RQ_E(D, 7, 0x2222222, LB), RQ_E(D, 8, 0x22222222, LB), \
      RQ_E(D, 5, 0x22224, LB), RQ_E(D, 6, 0x222224, LB), RQ_E(D, 7, 0x2222224, LB),                          \
      RQ_E(D, 8, 0x22222224, LB), RQ_E(D, 5, 0x22244, LB), RQ_E(D, 6, 0x222244, LB),                         \
      RQ_E(D, 7, 0x2222244, LB), RQ_E(D, 8, 0x22222244, LB)

#define RQ_E(D, NC, CB, LB) \
  {D, NC, CB, LB, 0, decode_fused<D, NC, CB, RQ_DEPTH, LB, 0>}, {D, NC, CB, LB, 1, decode_fused<D, NC, CB, RQ_DEPTH, LB, 1>}
const PlanEntry kLongTable[] = {RQ_LONG(64, 2), RQ_LONG(96, 2), RQ_LONG(128, 2),
                                RQ_LONG(64, 3), RQ_LONG(96, 3), RQ_LONG(128, 3)};
#undef RQ_E

}  // namespace

bool have_decode_kernel_long(int D, int nc, const int* bits, int limbs) {
  return find_plan(kLongTable, D, nc, bits, limbs, 0) != nullptr;
}

int launch_decode_long(const DecodeParams& p, int D, int nc, const int* bits, int limbs, int nsplit,
                       void* stream) {
  const PlanEntry* e = find_plan(kLongTable, D, nc, bits, limbs, p.rot_f16);
  if (!e || p.table) return -1;
  const dim3 grid((unsigned)(nsplit * p.B * p.H));
  hipLaunchKernelGGL(e->fn, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

}  // namespace rq
