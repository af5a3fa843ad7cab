// Decode launches of librq over a paged cache whose block size is a multiple
// of the wave tile (64 tokens at D = 64, 32 at D = 128): every tile lies in
// one block, so the kernel takes one block id per tile and addresses the
// tile's rows through per-tile buffer descriptors (rq_decode_kernel.hpp,
// kPagedTile). D = 96 tiles (42 tokens) never align; that size takes the
// lane-by-lane path, and so do four-component plans, whose per-tile
// descriptors (24 scalar registers per component) would spill.
#include "rq_decode_kernel.hpp"

namespace rq {
namespace {

#define RQ_E(D, NC, CB) {D, NC, CB, decode_fused_paged_tile<D, NC, CB, RQ_DEPTH>}
const PlanEntry kTileTable[] = {RQ_PLANS_UP3(64), RQ_PLANS_UP3(128)};
#undef RQ_E

}  // namespace

int launch_decode_paged_tile(const DecodeParams& p, int D, int nc, const int* bits, int nsplit, void* stream) {
  const PlanEntry* e = find_plan(kTileTable, D, nc, bits);
  if (!e) return -1;
  const dim3 grid((unsigned)(nsplit * p.B * p.H));
  hipLaunchKernelGGL(e->fn, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

}  // namespace rq
