// Raw buffer stores shared by the FP8 and MX grouped GEMMs (gfx9 buffer
// resource: base, stride 0, num_records in bytes, word 3 = 32-bit data
// format, no swizzle).  A store whose VGPR offset lies past num_records is
// dropped by the hardware (the SGPR offset is not part of that check, so it
// stays 0 here): a store can be issued by every lane, masked lanes out of
// range.  The stores are volatile asm so that the compiler neither merges
// nor removes any, because the GEMMs' ring waits count them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint32_t st_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t st_u32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kBufferRsrcWord3 = 0x00020000u;

// `base` and `num_records` are wave-uniform; readfirstlane says so, so the
// descriptor sits in SGPRs as the instruction requires.
__device__ __forceinline__ st_u32x4 buffer_rsrc(const void* base, uint32_t num_records) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return st_u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b),
                  (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xffffu),
                  (uint32_t)__builtin_amdgcn_readfirstlane(num_records), kBufferRsrcWord3};
}

// 8 bytes at base + voff + IMM (SGPR offset 0)
template <int IMM>
__device__ __forceinline__ void buffer_store8(st_u32x2 v, uint32_t voff, const st_u32x4& rsrc) {
  static_assert(IMM >= 0 && IMM < 4096, "MUBUF offset field");
  asm volatile("buffer_store_dwordx2 %0, %1, %2, 0 offen offset:%3"
               :: "v"(v), "v"(voff), "s"(rsrc), "n"(IMM) : "memory");
}

// 16 bytes at base + voff (SGPR offset 0).  A vector-memory store of more
// than 64 bits reads its data VGPRs after issue: a VALU write to them within
// the next two wait states (gfx940 and later) would be what gets stored.
// The compiler inserts those wait states only after stores it emits itself,
// not after inline asm, so the s_nop is part of the statement.
__device__ __forceinline__ void buffer_store16(st_u32x4 v, uint32_t voff, const st_u32x4& rsrc) {
  asm volatile("buffer_store_dwordx4 %0, %1, %2, 0 offen\n\ts_nop 1" :: "v"(v), "v"(voff), "s"(rsrc) : "memory");
}
// The same, non-temporal: rows written once and read once much later (the
// 256-token FC2 tiles' y rows, which at those token counts outgrow the
// caches before the combine reads them).
__device__ __forceinline__ void buffer_store16_nt(st_u32x4 v, uint32_t voff, const st_u32x4& rsrc) {
  asm volatile("buffer_store_dwordx4 %0, %1, %2, 0 offen nt\n\ts_nop 1" :: "v"(v), "v"(voff), "s"(rsrc) : "memory");
}

// A store that writes nothing (an empty buffer): it only counts as an
// outstanding vector-memory operation.
__device__ __forceinline__ void buffer_store_none(const st_u32x4& empty_rsrc) {
  asm volatile("buffer_store_dword %0, off, %1, 0" :: "v"(0u), "s"(empty_rsrc) : "memory");
}

}  // namespace moe
