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
// ranges in order and keep running per-expert counts in LDS.
#include <hip/hip_runtime.h>

#include "moe_compact_dev.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// Single-workgroup path (routes <= kCompactChunk): count, scan, scatter.
__global__ __launch_bounds__(kCompactThreads) void compact_fused_kernel(CompactArgs a) {
  extern __shared__ int lds[];
  compact_one_workgroup(a, lds);
}

// Multi-workgroup path, kernel 1: per-block per-expert counts -> blk_base.
__global__ __launch_bounds__(kCompactThreads) void compact_count_kernel(CompactArgs a) {
  extern __shared__ int lds[];
  const int E = a.num_experts;
  int* hist = lds;
  int rank[kItems], expert[kItems];
  clear_hist(hist, kCompactWaves * E);
  __syncthreads();
  sweep(a, blockIdx.x, hist, rank, expert);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kCompactThreads) {
    int s = 0;
    for (int w = 0; w < kCompactWaves; ++w) s += hist[w * E + e];
    a.blk_base[(int64_t)blockIdx.x * E + e] = s;
  }
}

// Kernel 2 (one workgroup): per-expert totals, offsets, per-block bases, tiles.
__global__ __launch_bounds__(kCompactThreads) void compact_scan_kernel(CompactArgs a) {
  extern __shared__ int lds[];
  const int E = a.num_experts;
  int* cnt = lds;
  int* tmp = cnt + E;
  int* scalar = tmp + E + 1;
  for (int e = threadIdx.x; e < E; e += kCompactThreads) {
    int run = 0;
    for (int b = 0; b < a.blocks; ++b) {
      const int c = a.blk_base[(int64_t)b * E + e];
      a.blk_base[(int64_t)b * E + e] = run;  // exclusive within the expert
      run += c;
    }
    cnt[e] = run;
  }
  __syncthreads();
  finish_counts(a, cnt, tmp, scalar);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kCompactThreads)
    for (int b = 0; b < a.blocks; ++b) a.blk_base[(int64_t)b * E + e] += tmp[e];
}

// Kernel 3: recompute the ranks and scatter.
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

int launch_compact(const CompactArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int E = a.num_experts;
  if (a.blocks <= 1) {
    hipLaunchKernelGGL(compact_fused_kernel, dim3(1), dim3(kCompactThreads), compact_one_workgroup_lds(E), s, a);
  } else {
    const size_t lds_hist = (size_t)(kCompactWaves * E + E) * 4;
    const size_t lds_scan = (size_t)(E + E + 1 + 2) * 4;
    hipLaunchKernelGGL(compact_count_kernel, dim3(a.blocks), dim3(kCompactThreads), lds_hist, s, a);
    hipLaunchKernelGGL(compact_scan_kernel, dim3(1), dim3(kCompactThreads), lds_scan, s, a);
    hipLaunchKernelGGL(compact_scatter_kernel, dim3(a.blocks), dim3(kCompactThreads), lds_hist, s, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
