// Decode launches of librq over a contiguous cache in the blocked layout (rq.h,
// rq_layer_cache.block_bytes): each stored loop's K and V codes, metadata and
// alpha share blocks of 32 token rows, so that a wave's tile of one component
// is one contiguous stretch of memory. The streaming kernel is the one of
// rq_decode_kernel.hpp.
#include "rq_decode_kernel.hpp"

namespace rq {
namespace {

#define RQ_E(D, NC, CB, LB) {D, NC, CB, LB, decode_fused<D, NC, CB, RQ_DEPTH, LB, true>}
const PlanEntry kBlockedTable[] = {RQ_PLANS(64), RQ_PLANS(96), RQ_PLANS(128)};
#undef RQ_E

}  // namespace

int launch_decode_blocked(const DecodeParams& p, int D, int nc, const int* bits, int limbs, int nsplit,
                          void* stream) {
  const PlanEntry* e = find_plan(kBlockedTable, D, nc, bits, limbs);
  if (!e) return -1;
  const dim3 grid((unsigned)(nsplit * p.B * p.H));
  hipLaunchKernelGGL(e->fn, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

}  // namespace rq
