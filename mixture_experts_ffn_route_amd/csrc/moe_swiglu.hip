// Second half of the unfused FC1 (MOE_FLAG_UNFUSED_FC1): SwiGLU and the
// 1x128 e4m3 requantisation of the FP32 gate/up rows the FC1 GEMM stored.
// The fused FC1 epilogue computes exactly this from the same FP32 values, so
// both paths give the same codes and scales ("feat(moe_ep): add SM90 push FP8
// mega-MoE backend for Hopper", flashinfer PR #4069, Description: the fused
// FC1 reproduces the unfused path).
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

typedef float v4f __attribute__((ext_vector_type(4)));

// 16 lanes per (row, 128-column block of h); each lane owns 8 columns.
__global__ __launch_bounds__(256) void swiglu_quant_kernel(const float* gateup, int64_t groups, int32_t inter,
                                                           const uint32_t* hdr, uint8_t* hq, float* hs) {
  const int64_t grp = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  if (grp >= groups) return;
  const int ib = inter / 128;
  const int64_t p = grp / ib;
  const int j = (int)(grp - p * ib);
  if (p >= (int64_t)hdr[kHdrRoutes]) return;  // rows past the kept routes hold nothing
  const int lane16 = threadIdx.x & 15;
  const int col = j * 128 + lane16 * 8;
  const float* g = gateup + p * (2 * (int64_t)inter) + col;
  const float* u = g + inter;
  const v4f g0 = *reinterpret_cast<const v4f*>(g), g1 = *reinterpret_cast<const v4f*>(g + 4);
  const v4f u0 = *reinterpret_cast<const v4f*>(u), u1 = *reinterpret_cast<const v4f*>(u + 4);
  float h[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = swiglu(g0[i], u0[i]);
    h[4 + i] = swiglu(g1[i], u1[i]);
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(h[i]));
  float amax = group_max<16>(m);
  const float s = amax / kE4m3Max;
  const float pre = requant_prescale(amax);
  const float inv = requant_inv(amax, s);
  if (pre != 1.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] *= pre;
  }
  int w0 = cvt2_e4m3(h[0] * inv, h[1] * inv, 0, false);
  w0 = cvt2_e4m3(h[2] * inv, h[3] * inv, w0, true);
  int w1 = cvt2_e4m3(h[4] * inv, h[5] * inv, 0, false);
  w1 = cvt2_e4m3(h[6] * inv, h[7] * inv, w1, true);
  *reinterpret_cast<uint2*>(hq + p * inter + col) = make_uint2((uint32_t)w0, (uint32_t)w1);
  if (lane16 == 0) hs[p * ib + j] = s;
}

int launch_swiglu_quant(const float* gateup, int32_t row_cap, int32_t inter, const uint32_t* hdr, uint8_t* hq,
                        float* hs, void* stream) {
  const int64_t groups = (int64_t)row_cap * (inter / 128);
  const int64_t blocks = (groups * 16 + 255) / 256;
  hipLaunchKernelGGL(swiglu_quant_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     gateup, groups, inter, hdr, hq, hs);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
