// Create-time weight transform: expert weights in checkpoint layout
// ([E, N, K] e4m3, K contiguous) become K-block tiles in MFMA fragment order,
// so the GEMMs fetch one contiguous 32 KB block per (expert, column tile,
// K-block) and read LDS lane-linearly.  This is the one-time conversion of
// static weights to the kernel layout that the stateful layer binds at
// construction ("feat(moe_ep): add SM90 push FP8 mega-MoE backend for
// Hopper", flashinfer PR #4069, Contracts).
//
// Tile (e, nt, kb) = 256 weight rows x 128 K-bytes, stored as 16 row blocks
// x {lo, hi} x 64 lanes x 16 bytes.  Lane l of the 16x16x128 MFMA operand of
// row block rb holds row rb*16 + l%16, K-bytes [32*(l/16), 32*(l/16)+32):
// its first 16 bytes are in the "lo" half, the next 16 in the "hi" half.
//   FC1 (w13): row block rb < 8 -> gate row nt*128 + rb*16 + l%16,
//              rb >= 8 -> up row I + nt*128 + (rb-8)*16 + l%16.
//   FC2 (w2):  row nt*256 + rb*16 + l%16; rows >= H (last tile when H is an
//              odd multiple of 128) are zero.
//
// MX operand order (MXFP8 weights): the scaled MFMA applies the E8M0 scale of
// 32-element block j to logical K elements [32j, 32j+32), and lane l holds
// logical elements [16*(l/16), +16) in its "lo" 16 bytes and [64 + 16*(l/16),
// +16) in its "hi" 16 bytes.  So lane l's lo half takes K-bytes 16*(l/16) and
// its hi half K-bytes 64 + 16*(l/16) of the 128-wide block, and the scale for
// (row, block j) comes from lane row%16 + 16*j.  The plain FP8 MFMA only pairs
// equal byte positions of both operands, so either order gives its product.
// Scale tile (e, nt, kb) = 4 groups x 64 lanes x 4 bytes: group q, lane l,
// byte b holds the exponent of row block 4q+b, row l%16, 32-block l/16.

#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One thread per 16-byte chunk of the destination.
__global__ __launch_bounds__(256) void tile_weights_kernel(const uint8_t* src, uint8_t* dst, int64_t chunks,
                                                           int n_rows, int k_dim, int n_tiles, int inter,
                                                           int fc1, int order) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  const int kbs = k_dim / 128;
  const int lane = (int)(c & 63);
  const int hilo = (int)((c >> 6) & 1);
  const int64_t tile = c >> 11;  // 2048 chunks per (e, nt, kb) tile
  const int kb = (int)(tile % kbs);
  const int nt = (int)((tile / kbs) % n_tiles);
  const int64_t e = tile / ((int64_t)kbs * n_tiles);
  const int rb = (int)((c >> 7) & 15);
  int row;
  if (fc1)
    row = (rb < 8 ? nt * 128 + rb * 16 : inter + nt * 128 + (rb - 8) * 16) + (lane & 15);
  else
    row = nt * 256 + rb * 16 + (lane & 15);
  const int kbyte = kb * 128 + (order == kTileOrderMx ? 16 * (lane >> 4) + 64 * hilo : 32 * (lane >> 4) + 16 * hilo);
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row < n_rows) v = *reinterpret_cast<const u32x4*>(src + (e * n_rows + row) * (int64_t)k_dim + kbyte);
  *reinterpret_cast<u32x4*>(dst + c * 16) = v;
}

// One thread per 4-byte word of the destination scale tiles.  src is the
// caller's E8M0 tensor [E, n_rows, k_dim/32]; rows past n_rows get 2^0.
__global__ __launch_bounds__(256) void tile_mx_scales_kernel(const uint8_t* src, uint32_t* dst, int64_t words,
                                                             int n_rows, int k_dim, int n_tiles, int inter, int fc1) {
  const int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (d >= words) return;
  const int kbs = k_dim / 128, q32 = k_dim / 32;
  const int lane = (int)(d & 63);
  const int grp = (int)((d >> 6) & 3);
  const int64_t tile = d >> 8;  // 256 words per (e, nt, kb) tile
  const int kb = (int)(tile % kbs);
  const int nt = (int)((tile / kbs) % n_tiles);
  const int64_t e = tile / ((int64_t)kbs * n_tiles);
  uint32_t word = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int rb = 4 * grp + b;
    int row;
    if (fc1)
      row = (rb < 8 ? nt * 128 + rb * 16 : inter + nt * 128 + (rb - 8) * 16) + (lane & 15);
    else
      row = nt * 256 + rb * 16 + (lane & 15);
    const uint32_t v = row < n_rows ? src[(e * n_rows + row) * (int64_t)q32 + kb * 4 + (lane >> 4)] : 127u;
    word |= v << (8 * b);
  }
  dst[d] = word;
}

int launch_tile_weights(const uint8_t* src, uint8_t* dst, int experts, int n_rows, int k_dim, int n_tiles,
                        int inter, bool fc1, int order, void* stream) {
  const int64_t chunks = (int64_t)experts * n_tiles * (k_dim / 128) * 2048;
  const int64_t blocks = (chunks + 255) / 256;
  hipLaunchKernelGGL(tile_weights_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream), src,
                     dst, chunks, n_rows, k_dim, n_tiles, inter, fc1 ? 1 : 0, order);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_tile_mx_scales(const uint8_t* src, uint32_t* dst, int experts, int n_rows, int k_dim, int n_tiles,
                          int inter, bool fc1, void* stream) {
  const int64_t words = (int64_t)experts * n_tiles * (k_dim / 128) * 256;
  const int64_t blocks = (words + 255) / 256;
  hipLaunchKernelGGL(tile_mx_scales_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     src, dst, words, n_rows, k_dim, n_tiles, inter, fc1 ? 1 : 0);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
