// Small device helpers shared by the HIP kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr float kE4m3Max = 448.0f;

// bfloat16 bits -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// float -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats -> two e4m3 codes in the low (hi=false) or high (hi=true) 16
// bits of `old`.  The hardware conversion rounds to nearest even; inputs are
// clamped to +-448 first so out-of-range magnitudes saturate instead of
// producing NaN.
__device__ __forceinline__ int cvt2_e4m3(float a, float b, int old, bool hi) {
  a = fminf(fmaxf(a, -kE4m3Max), kE4m3Max);
  b = fminf(fmaxf(b, -kE4m3Max), kE4m3Max);
  return hi ? __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, true)
            : __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
}

// Maximum over groups of `width` consecutive lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = 1; m < WIDTH; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, WIDTH));
  return v;
}

}  // namespace moe
