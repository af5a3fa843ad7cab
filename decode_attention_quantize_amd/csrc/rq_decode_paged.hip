// Decode launches of librq over a paged cache: the streaming kernel instances
// that find each token's row through a block table, lane by lane (rq.h: token t
// of sequence b lives in row (table[b][t / BS] H + h) BS + t mod BS of every
// buffer's block pool), for any block size. The kernel is the one of
// rq_decode_kernel.hpp; the combine launch is shared with the contiguous cache.
#include "rq_decode_kernel.hpp"

namespace rq {
namespace {

#define RQ_E(D, NC, CB, LB) \
  {D, NC, CB, LB, 0, decode_fused_paged<D, NC, CB, RQ_DEPTH, LB, 0>}, {D, NC, CB, LB, 1, decode_fused_paged<D, NC, CB, RQ_DEPTH, LB, 1>}
const PlanEntry kPagedTable[] = {RQ_PLANS(64), RQ_PLANS(96), RQ_PLANS(128)};
#undef RQ_E

}  // namespace

int launch_decode_paged(const DecodeParams& p, int D, int nc, const int* bits, int limbs, int nsplit,
                        void* stream) {
  const PlanEntry* e = find_plan(kPagedTable, D, nc, bits, limbs, p.rot_f16);
  if (!e) return -1;
  const dim3 grid((unsigned)(nsplit * p.B * p.H));
  hipLaunchKernelGGL(e->fn, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

}  // namespace rq
