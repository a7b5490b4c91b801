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

// One thread per (token, 8 consecutive columns).
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int chunks = a.hidden >> 3;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= (int64_t)a.tokens * chunks) return;
  const int64_t t = g / chunks;
  const int c = (int)(g - t * chunks) * 8;
  combine8<false>(a.y, a.route_pos, a.staged_w, t, a.top_k, a.hidden, c, a.out);
}

int launch_combine(const CombineArgs& a, void* stream) {
  if (a.tokens <= 0) return 0;
  const int64_t threads = (int64_t)a.tokens * (a.hidden / 8);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
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
