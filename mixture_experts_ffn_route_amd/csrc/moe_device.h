// Small device helpers shared by the HIP kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int32_t tile_rec_t __attribute__((ext_vector_type(4)));

// Row tile m of the compaction's tile list: (expert, first sorted row, rows,
// 1 if it is the expert's only row tile).  Written by an earlier launch and
// read through the scalar cache (one 16-byte load, counted on lgkmcnt); `m`
// is wave-uniform.
__device__ __forceinline__ tile_rec_t load_tile_rec(const int32_t* tiles, int m) {
  return ((const __attribute__((address_space(4))) tile_rec_t*)tiles)[m];
}

constexpr float kE4m3Max = 448.0f;

// bfloat16 bits -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Two floats -> two bfloat16 in one word (a in the low half), round to
// nearest even, on the gfx950 packed conversion (v_cvt_pk_bf16_f32).  It
// matches the bit-field rounding (add 0x7fff plus the kept LSB, NaN made
// quiet) on every float tested, ties and NaNs included.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// float -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return bf16x2_rne(f, 0.0f) & 0xffffu; }

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

// e4m3 code (OCP E4M3FN, finite) -> float, from its bit fields:
// exponent field 0 is subnormal m/8 * 2^-6, otherwise (1 + m/8) * 2^(e-7).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const int m = (int)(c & 7u), e = (int)((c >> 3) & 15u);
  const float mag = e ? ldexpf((float)(8 + m), e - 10) : ldexpf((float)m, -9);
  return (c & 0x80u) ? -mag : mag;
}

// E8M0 exponent of one 32-element block for the two-term split of BF16
// values: the block maximum lands in [128, 256), so no e4m3 code of the
// block saturates.  An all-zero block gets 2^0 (its codes are zero).
__device__ __forceinline__ int mx_block_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  const int e = __builtin_amdgcn_frexp_expf(amax) - 8;  // amax in [2^(x-1), 2^x) -> x - 8
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Four values of one block -> four e4m3 codes of v / 2^e (packed, code i in
// byte i), and the residuals v - code_i * 2^e, which are exact in float for
// BF16 inputs.
__device__ __forceinline__ uint32_t mx_term4(const float v[4], int e, float r[4]) {
  const int neg = -e;
  int w = cvt2_e4m3(ldexpf(v[0], neg), ldexpf(v[1], neg), 0, false);
  w = cvt2_e4m3(ldexpf(v[2], neg), ldexpf(v[3], neg), w, true);
  const uint32_t u = (uint32_t)w;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = v[i] - ldexpf(e4m3_to_f32((u >> (8 * i)) & 0xffu), e);
  return u;
}

// SwiGLU of one (gate, up) pair: silu(g) * u = g / (1 + 2^(-g log2 e)) * u on
// the hardware exp2 and reciprocal.  The fused FC1 epilogue and the unfused
// SwiGLU kernel both use this, so the two paths give the same bits.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.44269504f)) * u;
}

// 1x128 requantisation factor: codes are RNE_sat(h * inv) with
// inv = 448 / amax, and 0 when the block's scale s = amax / 448 is 0.
// `amax` must be at least 2^-64 (see requant_prescale), so that the
// reciprocal cannot overflow.
__device__ __forceinline__ float requant_inv(float amax, float s) {
  return s != 0.f ? kE4m3Max * __builtin_amdgcn_rcpf(amax) : 0.f;
}

// A block whose amax lies below 2^-64 (down to FP32 subnormals, where
// 1 / amax overflows) is requantised from h * 2^64 and amax * 2^64: both
// products are exact, and the codes of (h * 2^64) * 448 / (amax * 2^64) are
// those of h * 448 / amax.  Returns the factor to apply to h (1 or 2^64).
__device__ __forceinline__ float requant_prescale(float& amax) {
  const float f = amax < 0x1p-64f ? 0x1p64f : 1.0f;
  amax *= f;
  return f;
}

// Block-scale promotion of the FP8 GEMMs.  An output accumulates
// sum_kb F_kb * P_kb over K-blocks, with F_kb = sx * sw the product of the
// activation and weight block scales and P_kb the K-block's FP8 code product.
// The accumulator is kept in units of m * 2^ref, where m in [1/4, 1) is the
// mantissa product of the current block's two scales and ref the largest
// exponent sum seen so far; the MFMA applies each block's own 2^(e - ref)
// as its E8M0 operand scale (exact), and before a block's MFMA the
// accumulator is multiplied by
//   r = (m_prev / m) * 2^(ref_prev - ref)      (|r| < 4)
// so no ratio of scales, however far apart, overflows or is lost.  After the
// last block, out = ldexp(acc * m_last, ref).  A block whose scale is zero
// contributes nothing (its products enter at 2^-127 of the current unit, or
// are discarded with r = 0 when no block with a nonzero scale preceded it);
// with no such block at all the output is 0.
struct Promo {
  float m;  // mantissa product of the last nonzero block, 0 while none
  int e;    // ref: largest exponent sum so far
};

// One K-block: returns the accumulator ratio r and sets `sh` to the E8M0
// byte (127 + e - ref, at least 0) of the block's MFMA.  Branch-free (the
// three cases are selected), so that the promotion threads of a wave, which
// take different cases, stay on one path.
__device__ __forceinline__ float promo_step(float sx, float sw, Promo& p, int& sh) {
  const float m = __builtin_amdgcn_frexp_mantf(sx) * __builtin_amdgcn_frexp_mantf(sw);
  const int e = __builtin_amdgcn_frexp_expf(sx) + __builtin_amdgcn_frexp_expf(sw);
  const bool zero = m == 0.f;      // the block adds nothing
  const bool first = p.m == 0.f;   // the first block with a nonzero scale starts the sum
  const int ref = max(p.e, e);
  const float ratio = __builtin_amdgcn_ldexpf(p.m * __builtin_amdgcn_rcpf(m), p.e - ref);
  const float r = zero ? 1.f : (first ? 0.f : ratio);
  sh = zero ? 0 : (first ? 127 : max(127 + e - ref, 0));
  p.e = zero ? p.e : (first ? e : ref);
  p.m = zero ? p.m : m;
  return r;
}

// Maximum over groups of `width` consecutive lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = 1; m < WIDTH; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, WIDTH));
  return v;
}

}  // namespace moe
