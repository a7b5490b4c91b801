// Owner-side weighted top-k combine: one BF16 row per token, the routes'
// FC2 rows reduced in FP32 in ascending slot order ("feat(moe_ep): add SM90
// push FP8 mega-MoE backend for Hopper", flashinfer PR #4069, Description:
// grouped combine performs FP32 route reduction on the owner; with a single
// owner the BF16 reduction of received owner rows is this store).  The same
// arithmetic runs fused at the end of FC2 (moe_combine_dev.h).
#include <hip/hip_runtime.h>

#include "moe_combine_dev.h"
#include "moe_internal.h"

namespace moe {

constexpr int kCombineThreads = 128;  // 8 columns each: 1024 columns of one token per workgroup

// Workgroup b: token b / col_blocks, columns of its column block; one thread
// per 8 consecutive columns.  The token is the same for the whole
// workgroup, so its K positions and weights come through the scalar cache
// (one load each per wave) and every vector load is a y row piece.
template <int K>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a, int col_blocks) {
  const int b = (int)blockIdx.x;
  const int t = b / col_blocks;
  const int c = ((b - t * col_blocks) * kCombineThreads + (int)threadIdx.x) * 8;
  typedef __attribute__((address_space(4))) const int32_t c_i32;
  typedef __attribute__((address_space(4))) const float c_f32;
  int pos[K];
  float w[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    pos[k] = ((c_i32*)a.route_pos)[(int64_t)t * K + k];
    w[k] = ((c_f32*)a.staged_w)[(int64_t)t * K + k];
  }
  if (c >= a.hidden) return;
  combine8_pw<K, false>(a.y, pos, w, t, a.hidden, c, a.out);
}

int launch_combine(const CombineArgs& a, void* stream) {
  if (a.tokens <= 0) return 0;
  const int col_blocks = (a.hidden / 8 + kCombineThreads - 1) / kCombineThreads;
  if ((int64_t)a.tokens * col_blocks > 0x7fffffff) return -1;
  const dim3 grid((unsigned)(a.tokens * col_blocks)), block(kCombineThreads);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (a.top_k) {
    case 1: hipLaunchKernelGGL(combine_kernel<1>, grid, block, 0, s, a, col_blocks); break;
    case 2: hipLaunchKernelGGL(combine_kernel<2>, grid, block, 0, s, a, col_blocks); break;
    case 4: hipLaunchKernelGGL(combine_kernel<4>, grid, block, 0, s, a, col_blocks); break;
    case 6: hipLaunchKernelGGL(combine_kernel<6>, grid, block, 0, s, a, col_blocks); break;
    case 8: hipLaunchKernelGGL(combine_kernel<8>, grid, block, 0, s, a, col_blocks); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* p, int64_t words) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += stride) p[i] = 0u;
}

int launch_fill_zero(uint32_t* p, int64_t words, void* stream) {
  if (words <= 0) return 0;
  int64_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream), p,
                     words);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
