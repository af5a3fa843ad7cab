// Decode launches of librq over a paged cache in the blocked layout (rq.h,
// rq_layer_cache.block_bytes): block ids looked up lane by lane, as in
// rq_decode_paged.hip, and each stored loop's arrays sharing 32-row blocks.
#include "rq_decode_kernel.hpp"

namespace rq {
namespace {

#define RQ_E(D, NC, CB, LB) {D, NC, CB, LB, decode_fused_paged<D, NC, CB, RQ_DEPTH, LB, true>}
const PlanEntry kPagedBlockedTable[] = {RQ_PLANS(64), RQ_PLANS(96), RQ_PLANS(128)};
#undef RQ_E

}  // namespace

int launch_decode_paged_blocked(const DecodeParams& p, int D, int nc, const int* bits, int limbs, int nsplit,
                                void* stream) {
  const PlanEntry* e = find_plan(kPagedBlockedTable, D, nc, bits, limbs);
  if (!e) return -1;
  const dim3 grid((unsigned)(nsplit * p.B * p.H));
  hipLaunchKernelGGL(e->fn, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

}  // namespace rq
