// Route compaction into per-expert row lists (the "compact" step of the
// forward pipeline in "feat(moe_ep): add SM90 push FP8 mega-MoE backend for
// Hopper", flashinfer PR #4069, Description).
//
// Output, for the staged routes r = t*K + k (expert -1 = masked):
//   counts[e]        kept routes of expert e
//   offsets[e]       exclusive prefix of counts (E+1 entries)
//   sorted_route[p]  route ids, expert-major, ascending r within an expert
//   route_pos[r]     p such that sorted_route[p] == r, or -1
//   tiles[m]         (expert, first sorted row, rows, only-tile flag) of each BLOCK_M row tile
// Routes whose expert-major position reaches the row capacity are dropped
// and flagged (MOE_DEV_CAPACITY).
//
// Ranking is stable and deterministic: within a wavefront, lanes holding the
// same expert find each other with one ballot per expert-id bit, and a lane's
// rank is the popcount of its peers below it; waves walk contiguous route
// ranges in order and keep running per-expert counts in LDS.  Workgroups
// take whole tokens, at most kCompactChunk routes each; the counting runs in
// the staging launch (moe_stage.hip), beside the activation quantisation.
#include <hip/hip_runtime.h>

#include "moe_compact_dev.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// Scatter of a compaction over several workgroups (the staging launch has
// counted, and its last workgroup has turned the counts into per-workgroup
// bases): recompute the ranks and write each route's position.
__global__ __launch_bounds__(kCompactThreads) void compact_scatter_kernel(CompactArgs a) {
  extern __shared__ int lds[];
  const int E = a.num_experts;
  int* hist = lds;
  int* start = hist + kCompactWaves * E;
  int rank[kItems], expert[kItems];
  clear_hist(hist, kCompactWaves * E);
  for (int e = threadIdx.x; e < E; e += kCompactThreads) start[e] = a.blk_base[(int64_t)blockIdx.x * E + e];
  __syncthreads();
  sweep(a, blockIdx.x, hist, rank, expert);
  __syncthreads();
  scatter(a, blockIdx.x, hist, start, rank, expert);
}

int launch_compact_scatter(const CompactArgs& a, void* stream) {
  const size_t lds_hist = (size_t)(kCompactWaves * a.num_experts + a.num_experts) * 4;
  hipLaunchKernelGGL(compact_scatter_kernel, dim3(a.blocks), dim3(kCompactThreads), lds_hist,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
