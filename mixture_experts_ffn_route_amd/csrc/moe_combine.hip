// Owner-side weighted top-k combine: one BF16 row per token, the routes'
// FC2 rows reduced in FP32 in ascending slot order ("feat(moe_ep): add SM90
// push FP8 mega-MoE backend for Hopper", flashinfer PR #4069, Description:
// grouped combine performs FP32 route reduction on the owner; with a single
// owner the BF16 reduction of received owner rows is this store).
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One thread per (token, 8 consecutive columns): the K route rows are loaded
// first (16 bytes each, independent), then reduced in ascending slot order.
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int chunks = a.hidden >> 3;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= (int64_t)a.tokens * chunks) return;
  const int64_t t = g / chunks;
  const int c = (int)(g - t * chunks) * 8;
  const int K = a.top_k;
  float w[8];
  u32x4 raw[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    w[k] = 0.f;
    raw[k] = u32x4{0u, 0u, 0u, 0u};
    if (k < K) {
      const int p = a.route_pos[t * K + k];
      if (p >= 0) {
        w[k] = a.staged_w[t * K + k];
        raw[k] = *reinterpret_cast<const u32x4*>(a.y + (int64_t)p * a.hidden + c);
      }
    }
  }
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < K) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(w[k], bf16_to_f32(raw[k][i] & 0xffffu), acc[2 * i]);
        acc[2 * i + 1] = fmaf(w[k], bf16_to_f32(raw[k][i] >> 16), acc[2 * i + 1]);
      }
    }
  }
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16_rne(acc[2 * i]) | (f32_to_bf16_rne(acc[2 * i + 1]) << 16);
  *reinterpret_cast<u32x4*>(a.out + t * a.hidden + c) = o;
}

int launch_combine(const CombineArgs& a, void* stream) {
  if (a.tokens <= 0) return 0;
  const int64_t threads = (int64_t)a.tokens * (a.hidden / 8);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
