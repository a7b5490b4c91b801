// FP8 e4m3 block-scale grouped GEMMs of the MoE layer on gfx950 MFMA.
//
// FC1: for each sorted route row p (expert e, token t)
//   gu[p, n] = sum_kb sx[t, kb] * s13[e, n/128, kb] * sum_{k in kb} xq[t, k] * w13[e, n, k]
//   h = silu(gate) * up, then per 1x128 block of h: s = amax/448, q = RNE_sat(h/s)
// FC2: y[p, n] = sum_kb sh[p, kb] * s2[e, n/128, kb] * sum_{k in kb} hq[p, k] * w2[e, n, k]  -> bf16
//
// These are the "FC1 with fused SwiGLU + 1x128 quantization" and "FC2" steps
// of the forward pipeline in "feat(moe_ep): add SM90 push FP8 mega-MoE backend
// for Hopper" (flashinfer PR #4069, Description), with the DeepSeek-style FP8
// block scaling (128x128 weight scales, 1x128 activation scales) of its
// Limitations.
//
// Design (CDNA4):
//  * One K-block of 128 is exactly one 16x16x128 f8f6f4 MFMA.  The block
//    scales are applied by keeping the accumulator in units of the current
//    block's scale product (promo_step in moe_device.h): the MFMA's E8M0
//    operand scale applies the product's power-of-two part exactly, one
//    multiply per output per K-block applies the mantissa ratio, and the
//    MFMA accumulates in place, so no MFMA result needs registers of its
//    own.
//  * Weights are the MFMA row operand and tokens the column operand, so a
//    lane's four outputs of a 16x16 block share one token and one weight
//    block: one scale product per lane per token block.
//  * Workgroup tile: 256 weight rows x BT tokens, 8 waves (two per SIMD, so
//    one wave's rescaling multiplies run beside the other's MFMAs).  FC1's 256
//    weight rows are the gate and up rows of one 128-wide block of h, so the
//    SwiGLU and the 1x128 amax of the epilogue see whole blocks; FC2's are
//    two 128-row blocks of H.
//  * K-blocks move global -> LDS by LDS-DMA (global_load_lds_dwordx4), a
//    multi-stage ring, no staging registers.  Both operands land in LDS in
//    MFMA fragment order (16-row block x {lo, hi} x 64 lanes x 16 bytes), so
//    every operand read is one lane-linear 1 KB ds_read_b128 (no bank
//    conflicts, no address math).  Weights were tiled in that order at create
//    time, so a weight K-block is one contiguous 32 KB copy; token rows are
//    gathered per lane (FC1 through the sorted route list: one staged row per
//    token).
//  * Persistent workgroups: the (token tile, column tile) space is split into
//    eight contiguous ranges, one per XCD (workgroup i runs on XCD i % 8), so
//    neighbouring tiles on an XCD share rows and weights in its L2.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "moe_combine_dev.h"
#include "moe_device.h"
#include "moe_internal.h"
#include "moe_store_dev.h"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kBN = 256;          // weight rows per tile
constexpr int kKB = 128;          // bytes (= e4m3 elements) per K-block
constexpr int kGroupM = 4;        // token tiles per XCD-local group
constexpr int kPrefetchAhead = 3; // weight K-blocks prefetched into L2 ahead of the stage loads
constexpr int kLdsBytes = 160 * 1024;
constexpr int kMaxKBlocks = 128;  // K <= 16384
constexpr int kWsBytes = 2 * kMaxKBlocks * 4;  // per-tile weight-scale columns
constexpr int kRingBytes = kLdsBytes - kWsBytes;

// One 16x16x128 e4m3 MFMA whose products are scaled by 2^(byte - 127),
// `byte` taken from byte OB of the token operand's scale word (lane l
// supplies it for token l % 16; every lane of a token holds the same word),
// the weight operand at 2^0.  This is the block-scale promotion's exact
// power-of-two part (promo_step in moe_device.h).
template <int OB>
__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, OB, sb);
}

// LDS is addressed through 32-bit address-space-3 pointers throughout: no
// generic-pointer casts, so offsets fold into instruction immediates.
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) const float lds_f32;

// Operand of a 16x16x128 MFMA from a fragment-ordered LDS tile: each 16-row
// block holds its "lo" 1 KB then its "hi" 1 KB, lane-linear.  `p` points at
// this lane's 16 bytes of the block's lo half (block*2048 + lane*16).
__device__ __forceinline__ v8i lds_frag(const lds_u8* p) {
  const u32x4 lo = *reinterpret_cast<lds_u32x4*>(p);
  const u32x4 hi = *reinterpret_cast<lds_u32x4*>(p + 1024);
  v8i r;
  r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
  r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
  return r;
}

// Token operand layout in LDS, per 16-token block (2 KB): the 128-byte
// K-block of token t is 8 chunks of 16 bytes, and chunk c of token t sits at
// position 8 t + (c ^ tok_swz(t)).  One DMA instruction then fills 64
// consecutive positions = 8 whole token rows, one 128-byte line each (gathers
// of partial lines run at a fraction of the L2 rate), and the fragment reads
// (lane l: token l % 16, chunk 2 (l / 16) + half) hit 16 distinct 16-byte
// bank groups in every 8 and every 16 consecutive lanes.
__device__ __forceinline__ int tok_swz(int t) { return (t & 7) ^ ((t >> 3) & 1); }

// Fragment whose "lo" and "hi" 16 bytes come from two per-lane addresses.
__device__ __forceinline__ v8i lds_frag2(const lds_u8* lo_p, const lds_u8* hi_p) {
  const u32x4 lo = *reinterpret_cast<lds_u32x4*>(lo_p);
  const u32x4 hi = *reinterpret_cast<lds_u32x4*>(hi_p);
  v8i r;
  r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
  r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
  return r;
}

// LDS-DMA (global_load_lds): lane L's bytes land at lds_wave_base + L * size;
// lds_wave_base is wave-uniform and goes through M0.  Issued as inline asm so
// the compiler's wait insertion, which cannot follow which ring stage a DMA
// fills across the loop back-edge, never drains the ring; the K loop waits
// on the vector-memory counter itself.  The "memory" clobber keeps every LDS
// access in program order around these instructions.
// LDS and global bases of the DMAs are wave-uniform; readfirstlane says so
// (the asm takes them in SGPRs), and costs nothing where the compiler
// already holds them in SGPRs.
__device__ __forceinline__ uint32_t lds_addr(const lds_u8* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma4(const float* src, const lds_u8* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(lds_addr(lds_wave_base)) : "memory", "m0");
}

// The same loads from a wave-uniform base (an SGPR pair) plus a 32-bit
// per-lane byte offset: the K loop keeps one 32-bit VGPR per gathered
// address instead of a 64-bit pointer.  No instruction offset: on these
// loads it would move the LDS destination as well as the source.
__device__ __forceinline__ void dma16o(const void* base, uint32_t off, const lds_u8* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(uniform_ptr(base)), "s"(lds_addr(lds_wave_base)) : "memory", "m0");
}
// The weight stream of a tile that no other workgroup reads: non-temporal,
// so the lines do not displace reused data on their way through the
// caches (measured at T=8: W13 streams at 6.6 TB/s against 5.9 with the
// default policy).
__device__ __forceinline__ void dma16o_nt(const void* base, uint32_t off, const lds_u8* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :: "v"(off), "s"(uniform_ptr(base)), "s"(lds_addr(lds_wave_base)) : "memory", "m0");
}
__device__ __forceinline__ void dma4o(const void* base, uint32_t off, const lds_u8* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(off), "s"(uniform_ptr(base)), "s"(lds_addr(lds_wave_base)) : "memory", "m0");
}

// Scale loads of the persistent FC2 phase read rows that FC1 tiles on other
// XCDs have just written, and two rows share a cache line, so they are made
// at agent scope (sc1) instead of from a possibly stale L2 line.
template <bool kCoherent>
__device__ __forceinline__ void dma4o_scale(const void* base, uint32_t off, const lds_u8* lds_wave_base) {
  if constexpr (kCoherent)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1 sc1"
                 :: "v"(off), "s"(uniform_ptr(base)), "s"(lds_addr(lds_wave_base)) : "memory", "m0");
  else
    dma4o(base, off, lds_wave_base);
}

// Write-through store (agent scope) of h codes and scales in the persistent
// launch, where FC2 tiles on other XCDs read them within the same kernel.
__device__ __forceinline__ void store_wt_u32(uint8_t* p, uint32_t v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polls of a readiness counter before a persistent FC2 tile gives up (each
// poll sleeps ~0.25 us: ~0.25 s in all, far beyond any FC1 phase).
constexpr int kSpinLimit = 1 << 20;

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Workgroup barrier without a memory fence (no implied wait on the ring).
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// Wait for this wave's LDS accesses (the ratio writes before a barrier).
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int BT>
struct Cfg {
  static constexpr int WN = BT >= 256 ? 4 : (BT >= 64 ? 2 : (BT == 32 ? 4 : 8));  // waves along weight rows
  static constexpr int WT = kWaves / WN;                          // waves along tokens
  static constexpr int G = 128 / WN;                              // rows of each 128-row block per wave
  static constexpr int NB = 2 * G / 16;                           // 16-row weight blocks per wave
  static constexpr int TW = BT / WT;                              // tokens per wave
  static constexpr int TBW = TW / 16;                             // 16-token blocks per wave
  static constexpr int A_BYTES = kBN * kKB;
  static constexpr int B_BYTES = BT * kKB;
  static constexpr int S_BYTES = ((BT * 4 + 255) / 256) * 256;
  static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
  static constexpr int STAGES = (kRingBytes / STAGE) > 4 ? 4 : (kRingBytes / STAGE);
  static constexpr int A_INSTR = A_BYTES / 1024 / kWaves;         // 4
  static constexpr int B_INSTR = (BT + 63) / 64;                  // token-chunk loads per wave
  static constexpr int B_LANES = BT < 64 ? BT : 64;
  static constexpr int S_LANES = BT / kWaves;                     // scale loads per wave
  static constexpr int N_LD = A_INSTR + B_INSTR + 2;              // vector loads per wave per stage
  static_assert(TBW >= 1 && NB >= 2 && STAGES >= 2, "tile shape");
  // FC2 output: the tile's BF16 rows go through a free ring stage (the last
  // slot, which the next tile's prologue leaves empty), Y_ROWS rows per pass,
  // and leave it as 16-byte stores of whole rows: BT / 16 per wave.
  static constexpr int Y_PASSES = BT <= 64 ? 1 : 2;
  static constexpr int Y_ROWS = BT / Y_PASSES;
  static constexpr int EPI_STORES = BT / 16;                      // FC2 output stores per wave per tile
  static_assert(Y_ROWS * 512 <= STAGE && Y_ROWS % 16 == 0 && TW % 16 == 0, "output staging");
  static_assert((STAGES - 2) * N_LD + EPI_STORES < 64, "vmcnt range");
};

template <int BT, bool FC1>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_kernel(GemmArgs a) {
  using C = Cfg<BT>;
  constexpr bool PERSIST = false;
  const PersistArgs q{};
  // One LDS object per ring stage: the compiler tracks LDS-DMA per object,
  // so reading one stage never waits for the DMA still filling another.
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[C::STAGES > 2 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t ring3[C::STAGES > 3 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(16))) float wsc[2 * kMaxKBlocks];  // weight scales [block 0 | block 1][kb]
  __shared__ __attribute__((aligned(16))) float sx0[BT];               // token scales of K-block 0
  __shared__ __attribute__((aligned(16))) float rsc[2][BT][4];          // promotion records, double-buffered
  __shared__ __attribute__((aligned(16))) float fsc[BT][4];             // final scales (m0, m1, e0, e1)
  __shared__ __attribute__((aligned(16))) uint32_t l2sink[kThreads];    // L2 prefetch landing words (never read)
  __shared__ __attribute__((aligned(16))) float red_s[FC1 ? C::WN * BT : 4];  // FC1 epilogue: partial amax
  __shared__ int32_t cb_list[FC1 ? 1 : BT];  // FC2 fused combine: tokens this tile completes
  __shared__ int32_t cb_count;
  auto ring = [&](auto stage) -> lds_u8* {
    constexpr int S = decltype(stage)::value;
    if constexpr (S == 0) return (lds_u8*)ring0;
    else if constexpr (S == 1) return (lds_u8*)ring1;
    else if constexpr (S == 2) return (lds_u8*)ring2;
    else return (lds_u8*)ring3;
  };
  const lds_f32* wscl = (const lds_f32*)wsc;

#include "moe_gemm_fp8_body.inc"
}

// FC1 then FC2 in one launch: each workgroup runs its FC1 tiles, then its
// FC2 tiles, each of which first waits for its row tile's FC1 rows.  A
// cooperative launch (every workgroup resident, or the launch fails): a
// waiting workgroup only waits for FC1 tiles, which belong to resident
// workgroups and never wait themselves, so every wait ends.
template <int BT>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_persist_kernel(GemmArgs a1, GemmArgs a2, PersistArgs q) {
  using C = Cfg<BT>;
  constexpr bool PERSIST = true;
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[C::STAGES > 2 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t ring3[C::STAGES > 3 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(16))) float wsc[2 * kMaxKBlocks];
  __shared__ __attribute__((aligned(16))) float sx0[BT];
  __shared__ __attribute__((aligned(16))) float rsc[2][BT][4];
  __shared__ __attribute__((aligned(16))) float fsc[BT][4];
  __shared__ __attribute__((aligned(16))) uint32_t l2sink[kThreads];
  __shared__ __attribute__((aligned(16))) float red_s[C::WN * BT];
  __shared__ int32_t cb_list[BT];
  __shared__ int32_t cb_count;
  auto ring = [&](auto stage) -> lds_u8* {
    constexpr int S = decltype(stage)::value;
    if constexpr (S == 0) return (lds_u8*)ring0;
    else if constexpr (S == 1) return (lds_u8*)ring1;
    else if constexpr (S == 2) return (lds_u8*)ring2;
    else return (lds_u8*)ring3;
  };
  const lds_f32* wscl = (const lds_f32*)wsc;
  {
    constexpr bool FC1 = true;
    const GemmArgs& a = a1;
#include "moe_gemm_fp8_body.inc"
  }
  __syncthreads();  // the FC2 phase's first loads reuse the LDS the last FC1 epilogue read
  {
    constexpr bool FC1 = false;
    const GemmArgs& a = a2;
#include "moe_gemm_fp8_body.inc"
  }
}

template <int BT>
static int launch_persist(const GemmArgs& a1, const GemmArgs& a2, const PersistArgs& q, int grid, void* stream) {
  GemmArgs x1 = a1, x2 = a2;
  PersistArgs xq = q;
  void* args[] = {&x1, &x2, &xq};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&gemm_fp8_persist_kernel<BT>), dim3(grid),
                                    dim3(kThreads), args, 0, static_cast<hipStream_t>(stream)) == hipSuccess
             ? 0
             : -1;
}

int launch_fc1_fc2(const GemmArgs& a1, const GemmArgs& a2, const PersistArgs& q, int block_m, int grid, void* stream) {
  switch (block_m) {
    case 16: return launch_persist<16>(a1, a2, q, grid, stream);
    case 32: return launch_persist<32>(a1, a2, q, grid, stream);
    case 64: return launch_persist<64>(a1, a2, q, grid, stream);
    case 128: return launch_persist<128>(a1, a2, q, grid, stream);
  }
  return -1;
}

template <int BT>
static int occ_persist() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_fp8_persist_kernel<BT>, kThreads, 0) != hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

int gemm_persist_max_workgroups_per_cu(int block_m) {
  switch (block_m) {
    case 16: return occ_persist<16>();
    case 32: return occ_persist<32>();
    case 64: return occ_persist<64>();
    default: return occ_persist<128>();
  }
}

#ifndef MOE_SLOT_TIMERS
#define MOE_SLOT_TIMERS 0
#endif
#if MOE_SLOT_TIMERS
__device__ unsigned long long g_slot_timers[MOE_SLOT_TIMER_WORDS];
#endif

#include "moe_gemm_fp8_pp.inc"
#include "moe_gemm_fp8_stream.inc"

// 64-token tiles run the streaming kernel on two column tiles per tile
// (512 weight rows, two K-blocks = 128 KB of weights in flight) where K has
// an even number of blocks and the column tiles pair up.
constexpr int kStreamBT = 64, kStreamD = 2, kStreamCT = 2;
int gemm_stream_depth(int block_m, int kbs, int n_tiles) {
  return block_m == kStreamBT && kbs % kStreamD == 0 && n_tiles % kStreamCT == 0 ? kStreamD : 0;
}

template <bool FC1>
static int launch_stream(const GemmArgs& a, void* stream) {
  if (a.gateup != nullptr || a.fc.out != nullptr || a.stream_depth != kStreamD ||
      a.k_dim % (kStreamD * kKB) != 0 || a.n_tiles % kStreamCT != 0)
    return -1;
  hipLaunchKernelGGL((gemm_fp8_stream_kernel<kStreamBT, kStreamD, kStreamCT, FC1>), dim3(a.grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int BT, bool FC1>
static int launch_one(const GemmArgs& a, void* stream) {
  if constexpr (BT == kStreamBT) {
    if (a.stream_depth != 0) return launch_stream<FC1>(a, stream);
  }
  if constexpr (BT == 256 || BT == 192) {
    // 192- and 256-token tiles: the ping-pong schedule (the tactic gives the
    // variants with a gate/up output or the fused combine 128-token tiles)
    if (a.gateup != nullptr || a.fc.out != nullptr) return -1;
    hipLaunchKernelGGL((gemm_fp8_pp_kernel<FC1, BT>), dim3(a.grid), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), a);
  } else {
    hipLaunchKernelGGL((gemm_fp8_kernel<BT, FC1>), dim3(a.grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <bool FC1>
static int launch_bt(const GemmArgs& a, int block_m, void* stream) {
  switch (block_m) {
    case 16: return launch_one<16, FC1>(a, stream);
    case 32: return launch_one<32, FC1>(a, stream);
    case 64: return launch_one<64, FC1>(a, stream);
    case 128: return launch_one<128, FC1>(a, stream);
    case 192: return launch_one<192, FC1>(a, stream);
    case 256: return launch_one<256, FC1>(a, stream);
  }
  return -1;
}

int launch_fc1(const GemmArgs& a, int block_m, void* stream) { return launch_bt<true>(a, block_m, stream); }
int launch_fc2(const GemmArgs& a, int block_m, void* stream) { return launch_bt<false>(a, block_m, stream); }

template <int BT, bool FC1>
static int occ(int depth) {
  int n = 0;
  hipError_t r;
  if constexpr (BT == kStreamBT) {
    if (depth != 0)
      r = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_fp8_stream_kernel<kStreamBT, kStreamD, kStreamCT, FC1>,
                                                       kThreads, 0);
    else
      r = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_fp8_kernel<BT, FC1>, kThreads, 0);
  } else if constexpr (BT == 256 || BT == 192)
    r = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_fp8_pp_kernel<FC1, BT>, kThreads, 0);
  else
    r = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_fp8_kernel<BT, FC1>, kThreads, 0);
  if (r != hipSuccess) return 1;
  return n > 0 ? n : 1;
}

int gemm_max_workgroups_per_cu(int which, int block_m, int stream_depth) {
  const bool f1 = which == 1;
  const int d = stream_depth;
  switch (block_m) {
    case 16: return f1 ? occ<16, true>(0) : occ<16, false>(0);
    case 32: return f1 ? occ<32, true>(d) : occ<32, false>(d);
    case 64: return f1 ? occ<64, true>(d) : occ<64, false>(d);
    case 128: return f1 ? occ<128, true>(d) : occ<128, false>(d);
    case 192: return f1 ? occ<192, true>(0) : occ<192, false>(0);
    default: return f1 ? occ<256, true>(0) : occ<256, false>(0);
  }
}

}  // namespace moe

extern "C" moe_status_t moe_debug_slot_timers(uint64_t* out, int32_t count) {
  moe::clear_error();
#if MOE_SLOT_TIMERS
  if (!out || count < MOE_SLOT_TIMER_WORDS)
    return moe::fail(MOE_ERR_INVALID_ARG, "out must hold %d words", MOE_SLOT_TIMER_WORDS);
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpyFromSymbol(out, HIP_SYMBOL(moe::g_slot_timers), MOE_SLOT_TIMER_WORDS * sizeof(uint64_t)) != hipSuccess)
    return moe::fail(MOE_ERR_HIP, "reading the slot timers failed");
  const uint64_t zero[MOE_SLOT_TIMER_WORDS] = {};
  if (hipMemcpyToSymbol(HIP_SYMBOL(moe::g_slot_timers), zero, sizeof(zero)) != hipSuccess)
    return moe::fail(MOE_ERR_HIP, "clearing the slot timers failed");
  return MOE_OK;
#else
  (void)out;
  (void)count;
  return moe::fail(MOE_ERR_UNSUPPORTED, "this library was built without slot timers (build.py --slot-timers)");
#endif
}
