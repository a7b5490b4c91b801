// Owner-side weighted top-k combine: one BF16 row per token, the routes'
// FC2 rows reduced in FP32 in ascending slot order ("feat(moe_ep): add SM90
// push FP8 mega-MoE backend for Hopper", flashinfer PR #4069, Description:
// grouped combine performs FP32 route reduction on the owner; with a single
// owner the BF16 reduction of received owner rows is this store).
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// One wave per token; each lane reduces 8 consecutive columns per pass
// (16-byte loads and stores, 512 columns per wave pass).
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.tokens) return;
  const int lane = threadIdx.x & 63;
  const int K = a.top_k;
  int64_t pos[8];
  float w[8];
  for (int k = 0; k < K; ++k) {
    const int p = a.route_pos[(int64_t)t * K + k];
    pos[k] = p;
    w[k] = p >= 0 ? a.staged_w[(int64_t)t * K + k] : 0.0f;
  }
  for (int c = lane * 8; c < a.hidden; c += 512) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int k = 0; k < K; ++k) {
      if (pos[k] < 0) continue;
      const uint4 raw = *reinterpret_cast<const uint4*>(a.y + pos[k] * a.hidden + c);
      const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(w[k], bf16_to_f32(u[i] & 0xffffu), acc[2 * i]);
        acc[2 * i + 1] = fmaf(w[k], bf16_to_f32(u[i] >> 16), acc[2 * i + 1]);
      }
    }
    uint4 o;
    o.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
    o.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
    o.z = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
    o.w = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
    *reinterpret_cast<uint4*>(a.out + (int64_t)t * a.hidden + c) = o;
  }
}

int launch_combine(const CombineArgs& a, void* stream) {
  if (a.tokens <= 0) return 0;
  hipLaunchKernelGGL(combine_kernel, dim3((a.tokens + 3) / 4), dim3(256), 0, static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
