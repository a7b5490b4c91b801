// Second half of the unfused FC1 (MOE_FLAG_UNFUSED_FC1): SwiGLU and the
// 1x128 e4m3 requantisation of the gate/up rows the FC1 GEMM stored.  From
// FP32 rows the fused FC1 epilogue computes exactly this from the same
// values, so both paths give the same codes and scales ("feat(moe_ep): add
// SM90 push FP8 mega-MoE backend for Hopper", flashinfer PR #4069,
// Description: the fused FC1 reproduces the unfused path); from BF16 rows
// (MOE_FLAG_BF16_GATEUP, the unfused path's BF16 gate/up buffer of the same
// passage) the values are the rounded ones, widened exactly.
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

typedef float v4f __attribute__((ext_vector_type(4)));

// Eight gate/up values of a row from FP32 or BF16 storage.
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const v4f a = *reinterpret_cast<const v4f*>(p), b = *reinterpret_cast<const v4f*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(u[i] & 0xffffu);
    v[2 * i + 1] = bf16_to_f32(u[i] >> 16);
  }
}

// 16 lanes per (row, 128-column block of h); each lane owns 8 columns.
template <typename T>
__global__ __launch_bounds__(256) void swiglu_quant_kernel(const T* gateup, int64_t groups, int32_t inter,
                                                           const uint32_t* hdr, uint8_t* hq, float* hs) {
  const int64_t grp = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  if (grp >= groups) return;
  const int ib = inter / 128;
  const int64_t p = grp / ib;
  const int j = (int)(grp - p * ib);
  if (p >= (int64_t)hdr[kHdrRoutes]) return;  // rows past the kept routes hold nothing
  const int lane16 = threadIdx.x & 15;
  const int col = j * 128 + lane16 * 8;
  const T* g = gateup + p * (2 * (int64_t)inter) + col;
  float gv[8], uv[8];
  load8(g, gv);
  load8(g + inter, uv);
  float h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = swiglu(gv[i], uv[i]);
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

int launch_swiglu_quant(const void* gateup, bool bf16, int32_t row_cap, int32_t inter, const uint32_t* hdr,
                        uint8_t* hq, float* hs, void* stream) {
  const int64_t groups = (int64_t)row_cap * (inter / 128);
  const int64_t blocks = (groups * 16 + 255) / 256;
  if (bf16)
    hipLaunchKernelGGL(swiglu_quant_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(gateup), groups, inter, hdr, hq,
                       hs);
  else
    hipLaunchKernelGGL(swiglu_quant_kernel<float>, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const float*>(gateup), groups, inter, hdr, hq, hs);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
