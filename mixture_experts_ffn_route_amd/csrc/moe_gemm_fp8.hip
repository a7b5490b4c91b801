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
//  * One K-block of 128 is exactly one v_mfma_f32_16x16x128_f8f6f4.  The
//    block scales are applied by keeping the accumulator divided by the
//    current block's scale product (see carry_scale): one multiply per output
//    per K-block rescales it and the MFMA accumulates in place, so no MFMA
//    result needs registers of its own.
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

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Scale product of one K-block for the promotion recursion.  The accumulator
// is kept divided by the current block's product F = sx * sw:
//   acc_kb = acc_{kb-1} * (F_{kb-1} / F_kb) + sum_k a*b     (MFMA with C input)
// and multiplied by the last F after the K loop, which equals
// sum_kb F_kb * sum_k a*b.  A block whose F is zero or subnormal carries the
// previous F (its product is zero: its codes are all zero).
__device__ __forceinline__ float carry_scale(float f, float prev) {
  return fabsf(f) >= 0x1p-100f ? f : prev;
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
__device__ __forceinline__ uint32_t lds_addr(const lds_u8* p) { return (uint32_t)(uintptr_t)p; }
__device__ __forceinline__ void dma16(const uint8_t* src, const lds_u8* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds_addr(lds_wave_base)) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const float* src, const lds_u8* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(lds_addr(lds_wave_base)) : "memory", "m0");
}

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
  static_assert((STAGES - 2) * N_LD < 64, "vmcnt range");
};

template <int BT, bool FC1>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_kernel(GemmArgs a) {
  using C = Cfg<BT>;
  // One LDS object per ring stage: the compiler tracks LDS-DMA per object,
  // so reading one stage never waits for the DMA still filling another.
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[C::STAGES > 2 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t ring3[C::STAGES > 3 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(16))) float wsc[2 * kMaxKBlocks];  // weight scales [block 0 | block 1][kb]
  __shared__ __attribute__((aligned(16))) float sx0[BT];               // token scales of K-block 0
  __shared__ __attribute__((aligned(16))) float rsc[2][BT][2];          // promotion ratios, double-buffered
  __shared__ __attribute__((aligned(16))) float fsc[BT][2];             // final scale products
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

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % C::WN, wt = wave / C::WN;
  const int kbs = a.k_dim / kKB;
  const int nblk_w = a.n_rows / 128;
  const int total_m = __builtin_amdgcn_readfirstlane((int)a.hdr[kHdrMTiles]);
  const int64_t total = (int64_t)total_m * a.n_tiles;
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int per_xcd = gridDim.x >> 3;
  const int64_t v_begin = total * xcd / 8, v_end = total * (xcd + 1) / 8;
  // lane's offset of its first weight block and (two halves of) token block
  const uint32_t a_lane = (uint32_t)(wn * (C::G / 16)) * 2048u + (uint32_t)lane * 16u;
  const int tl = lane & 15;
  const uint32_t b_lane0 = (uint32_t)(wt * C::TBW) * 2048u + 16u * (uint32_t)(8 * tl + ((2 * (lane >> 4)) ^ tok_swz(tl)));
  const uint32_t b_lane1 =
      (uint32_t)(wt * C::TBW) * 2048u + 16u * (uint32_t)(8 * tl + ((2 * (lane >> 4) + 1) ^ tok_swz(tl)));
  const int t_lane = wt * C::TW + tl;  // token of this lane's outputs in token block 0
  // Promotion role: thread (pb, pt) keeps the running scale product
  // F = sx[pt] * sw[pb] of weight block pb (gate / first 128 rows or up /
  // second) for token pt, and publishes r = F_prev / F_next per K-block.
  const bool prole = tid < 2 * BT;
  const int pt = tid % BT, pb = (tid / BT) & 1;

  // ---- tile state -----------------------------------------------------------
  // Coordinates and per-lane DMA sources of the tile whose loads are in
  // flight.  They are set one tile ahead: the next tile's first stages are
  // issued before the current tile's epilogue, which then hides their latency.
  int e = 0, p0 = 0, rows_valid = 1, nt = 0, mt = 0, m0 = 0, gm = 1, nb0 = 0, nb1 = 0, pf_lanes = 8;
  const uint8_t* a_src = a.w;
  const uint8_t* b_src[C::B_INSTR];
  const float* s_src = a.a_scale;
  const uint8_t* pf_src = a.w;
  auto src_row = [&](int t) -> int64_t {
    const int p = p0 + min(t, rows_valid - 1);
    if (!FC1) return p;
    const int r = a.sorted_route[p];
    return a.a_mode == 2 ? r : r / a.top_k;
  };
  auto setup = [&](int64_t v) {
    const int64_t group = v / ((int64_t)kGroupM * a.n_tiles);
    const int64_t rem = v - group * kGroupM * a.n_tiles;
    m0 = (int)(group * kGroupM);
    gm = min(kGroupM, total_m - m0);
    nt = (int)(rem / gm);
    mt = m0 + (int)(rem % gm);
    // tile scalars are wave-uniform; saying so keeps their dependents
    // (weight-scale addresses) on the scalar unit
    e = __builtin_amdgcn_readfirstlane(a.tiles[2 * mt]);
    p0 = __builtin_amdgcn_readfirstlane(a.tiles[2 * mt + 1]);
    rows_valid = min(BT, __builtin_amdgcn_readfirstlane(a.offsets[e + 1]) - p0);
    if (FC1) {
      nb0 = nt;                  // gate block
      nb1 = a.inter / 128 + nt;  // up block
    } else {
      nb0 = 2 * nt;
      nb1 = min(2 * nt + 1, nblk_w - 1);
    }
    // weights: the tile's K-blocks are contiguous 32 KB pieces
    a_src = a.w + ((int64_t)e * a.n_tiles + nt) * kbs * (int64_t)C::A_BYTES + (wave * C::A_INSTR * 64 + lane) * 16;
    // tokens: LDS position V (16 bytes) of the stage holds chunk
    // (V % 8) ^ tok_swz(token) of token V / 8 (see tok_swz)
#pragma unroll
    for (int j = 0; j < C::B_INSTR; ++j) {
      const int v8 = wave * BT + j * 64 + (lane < C::B_LANES ? lane : 0);
      const int t = v8 >> 3;
      const int chunk = (v8 & 7) ^ tok_swz(t & 15);
      b_src[j] = a.a + src_row(t) * a.k_dim + chunk * 16;
    }
    // token scales: a stage carries those of the next K-block (the promotion
    // threads turn them into ratios one K-block ahead of their use)
    s_src = a.a_scale + src_row(wave * C::S_LANES + (lane < C::S_LANES ? lane : 0)) * kbs;
    // L2 prefetch of weights kPrefetchAhead K-blocks ahead of the stage
    // being loaded: the gm token tiles of a group share this weight tile
    // (they run side by side on one XCD), so each prefetches every gm-th of
    // its 256 lines; one word per line lands in l2sink.  Weight K-blocks are
    // first touches (the token rows are L2 hits by then), and a stage waits
    // for its slowest load.
    pf_lanes = 32 / gm;  // lines per wave per K-block
    const int pf_line = (wave * pf_lanes + (lane < pf_lanes ? lane : 0)) * gm + (mt - m0);
    pf_src = a.w + ((int64_t)e * a.n_tiles + nt) * kbs * (int64_t)C::A_BYTES + pf_line * 128;
  };

  auto issue = [&](auto stage, int kb) {
    const lds_u8* As = ring(stage);
    const lds_u8* Bs = As + C::A_BYTES;
    const lds_u8* Ss = Bs + C::B_BYTES;
#pragma unroll
    for (int j = 0; j < C::A_INSTR; ++j)
      dma16(a_src + (int64_t)kb * C::A_BYTES + j * 1024, As + (wave * C::A_INSTR + j) * 1024);
#pragma unroll
    for (int j = 0; j < C::B_INSTR; ++j)
      if (lane < C::B_LANES) dma16(b_src[j] + kb * kKB, Bs + (wave * BT + j * 64) * 16);
    if (lane < C::S_LANES) dma4(s_src + min(kb + 1, kbs - 1), Ss + wave * C::S_LANES * 4);
    if (lane < pf_lanes)
      dma4(reinterpret_cast<const float*>(pf_src + (int64_t)min(kb + kPrefetchAhead, kbs - 1) * C::A_BYTES),
           (const lds_u8*)l2sink + wave * 256);
  };

  // The loads a tile needs before its first step: its two weight-scale
  // columns (waves 0-3), the token scales of K-block 0 and the first
  // STAGES - 1 stages.  The scale loads are older than every stage load, so
  // the first stage's wait covers them.
  auto prologue = [&]() {
    if (wave < 4) {
      const int blk = wave >> 1, half = wave & 1;
      const int kb = half * 64 + lane;
      if (kb < kbs)
        dma4(a.w_scale + ((int64_t)e * nblk_w + (blk ? nb1 : nb0)) * kbs + kb,
             (const lds_u8*)wsc + (blk * kMaxKBlocks + half * 64) * 4);
    }
    if (lane < C::S_LANES) dma4(s_src, (const lds_u8*)sx0 + wave * C::S_LANES * 4);
    // K-block 0 meets a zero accumulator: any finite ratio will do
    if (prole) rsc[0][pt][pb] = 0.0f;
    issue(std::integral_constant<int, 0>{}, 0);
    if (C::STAGES > 2 && 1 < kbs) issue(std::integral_constant<int, 1>{}, 1);
    if (C::STAGES > 3 && 2 < kbs) issue(std::integral_constant<int, (C::STAGES > 3 ? 2 : 0)>{}, 2);
  };

  int64_t v = v_begin + slot;
  if (v < v_end) {
    setup(v);
    prologue();
  }
  if constexpr (!FC1) {
    if (a.fc.out) zero_unrouted_rows(a.fc, (int)a.hdr[kHdrTokens], a.top_k, a.n_rows);
  }
  for (; v < v_end; v += per_xcd) {
    float pf = 1.0f;
    v4f acc[C::NB][C::TBW];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int tb = 0; tb < C::TBW; ++tb) acc[nb][tb] = v4f{0.f, 0.f, 0.f, 0.f};

    // ---- K loop: STAGES-deep LDS ring -------------------------------------
    // acc holds sum_{j <= kb} P_j * F_j / F_kb for block products P_j; before
    // block kb's MFMAs it is rescaled by r_kb = F_{kb-1} / F_kb, and after the
    // loop multiplied by F_last.
    auto step = [&](auto stage, int kb) {
      constexpr int ST = decltype(stage)::value;
      const int ahead = min(C::STAGES - 2, kbs - 1 - kb);  // stages issued after this one
      if (C::STAGES >= 4 && ahead >= 2) wait_vmcnt<(C::STAGES >= 4 ? 2 : 0) * C::N_LD>();
      else if (C::STAGES >= 3 && ahead >= 1) wait_vmcnt<(C::STAGES >= 3 ? 1 : 0) * C::N_LD>();
      else wait_vmcnt<0>();
      // Every wave has its own DMA for this stage complete and its ratio
      // writes of the previous step done; the barrier makes that true for
      // all waves.  It also orders the previous stage's LDS reads (consumed
      // by MFMAs already) before the DMA issued next into it.  A plain
      // s_barrier: a fenced barrier would also drain the DMA of the stages
      // still in flight.
      wait_lgkmcnt0();
      barrier_nofence();
      if (kb + C::STAGES - 1 < kbs)
        issue(std::integral_constant<int, (ST + C::STAGES - 1) % C::STAGES>{}, kb + C::STAGES - 1);

      const lds_u8* As = ring(stage);
      const lds_u8* Bs = As + C::A_BYTES;
      const lds_f32* Ss = (const lds_f32*)(Bs + C::B_BYTES);
      const lds_u8* Ap = As + a_lane;
      const lds_u8* Bp0 = Bs + b_lane0;
      const lds_u8* Bp1 = Bs + b_lane1;
      typedef __attribute__((address_space(3))) const v2f lds_v2f;
      const lds_v2f* Rp = (const lds_v2f*)((const lds_f32*)&rsc[kb & 1][0][0] + 2 * t_lane);
      auto aoff = [](int nb) {  // byte offset of weight block nb of this wave
        return (nb < C::NB / 2 ? nb : 8 - C::NB / 2 + nb) * 2048;
      };
      if constexpr (C::NB > C::TBW) {
        // Hold the token fragments; weight fragments stream one block ahead.
        // The scheduling barrier keeps the compiler from hoisting every
        // block's LDS reads to the top (all of them live at once).
        v8i bq[C::TBW];
        v2f rr[C::TBW];
#pragma unroll
        for (int tb = 0; tb < C::TBW; ++tb) {
          bq[tb] = lds_frag2(Bp0 + tb * 2048, Bp1 + tb * 2048);
          rr[tb] = Rp[tb * 16];
        }
        v8i aq = lds_frag(Ap + aoff(0));
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          const v8i an = lds_frag(Ap + aoff(nb + 1 < C::NB ? nb + 1 : nb));
#pragma unroll
          for (int tb = 0; tb < C::TBW; ++tb)
            acc[nb][tb] = mfma_fp8(aq, bq[tb], acc[nb][tb] * (nb < C::NB / 2 ? rr[tb].x : rr[tb].y));
          __builtin_amdgcn_sched_barrier(0);
          aq = an;
        }
      } else {
        // Hold the weight fragments; token fragments stream one block ahead.
        v8i aq[C::NB];
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) aq[nb] = lds_frag(Ap + aoff(nb));
        v8i bq = lds_frag2(Bp0, Bp1);
        v2f rr = Rp[0];
#pragma unroll
        for (int tb = 0; tb < C::TBW; ++tb) {
          const int tn = tb + 1 < C::TBW ? tb + 1 : tb;
          const v8i bn = lds_frag2(Bp0 + tn * 2048, Bp1 + tn * 2048);
          const v2f rn = Rp[tn * 16];
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) acc[nb][tb] = mfma_fp8(aq[nb], bq, acc[nb][tb] * (nb < C::NB / 2 ? rr.x : rr.y));
          __builtin_amdgcn_sched_barrier(0);
          bq = bn;
          rr = rn;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // promotion threads: ratios of K-block kb + 1 (read by every wave at
      // the next step)
      if (prole) {
        const float swb_kb = wscl[pb * kMaxKBlocks + kb];
        if (kb == 0) pf = carry_scale(((const lds_f32*)sx0)[pt] * swb_kb, 1.0f);
        if (kb + 1 < kbs) {
          const float fn = carry_scale(Ss[pt] * wscl[pb * kMaxKBlocks + kb + 1], pf);
          rsc[(kb + 1) & 1][pt][pb] = pf * __builtin_amdgcn_rcpf(fn);
          pf = fn;
        }
      }
    };
    for (int kb = 0; kb < kbs; kb += C::STAGES) {
      step(std::integral_constant<int, 0>{}, kb);
      if (kb + 1 < kbs) step(std::integral_constant<int, 1>{}, kb + 1);
      if (C::STAGES > 2 && kb + 2 < kbs) step(std::integral_constant<int, (C::STAGES > 2 ? 2 : 0)>{}, kb + 2);
      if (C::STAGES > 3 && kb + 3 < kbs) step(std::integral_constant<int, (C::STAGES > 3 ? 3 : 0)>{}, kb + 3);
    }
    if (prole) fsc[pt][pb] = pf;
    __syncthreads();  // every wave is done with the ring (and fsc is visible) before the epilogue
    // this tile's epilogue coordinates; then the next tile's first loads
    const int ep_p0 = p0, ep_rows = rows_valid, ep_nt = nt;
    if (v + per_xcd < v_end) {
      setup(v + per_xcd);
      prologue();
    }
    // undo the running scale: acc = sum_kb F_kb * (block product)
#pragma unroll
    for (int tb = 0; tb < C::TBW; ++tb) {
      const v2f f = ((const __attribute__((address_space(3))) v2f*)((const lds_f32*)&fsc[0][0]))[t_lane + tb * 16];
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) acc[nb][tb] *= (nb < C::NB / 2 ? f.x : f.y);
    }

    // ---- epilogue -----------------------------------------------------------
    if (FC1 && a.gateup != nullptr) {
      // unfused FC1: FP32 gate and up rows, SwiGLU + requant run separately
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        const int col = (nb < C::NB / 2 ? 0 : a.inter) + ep_nt * 128 + wn * C::G + (nb % (C::NB / 2)) * 16 + 4 * (lane >> 4);
#pragma unroll
        for (int tb = 0; tb < C::TBW; ++tb) {
          const int t = wt * C::TW + tb * 16 + (lane & 15);
          if (t < ep_rows) *reinterpret_cast<v4f*>(a.gateup + (int64_t)(ep_p0 + t) * (2 * a.inter) + col) = acc[nb][tb];
        }
      }
    } else if (FC1) {
      // h = silu(gate) * up = g / (1 + 2^(-g log2 e)) * up on the hardware
      // exp2 and reciprocal; then the 1x128 amax, s = amax / 448 and the
      // codes of h * (1 / s).
      float* red = red_s;  // [WN][BT] partial amax
      float hv[C::TBW][C::NB / 2][4];
#pragma unroll
      for (int tb = 0; tb < C::TBW; ++tb) {
        float m = 0.f;
#pragma unroll
        for (int g = 0; g < C::NB / 2; ++g)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gt = acc[g][tb][i], up = acc[C::NB / 2 + g][tb][i];
            const float h = swiglu(gt, up);
            hv[tb][g][i] = h;
            m = fmaxf(m, fabsf(h));
          }
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (lane < 16) red[wn * BT + wt * C::TW + tb * 16 + lane] = m;
      }
      // LDS-only exchange: a fenced barrier would also wait for the next
      // tile's loads issued above
      wait_lgkmcnt0();
      barrier_nofence();
      const int ikb = a.inter / 128;
#pragma unroll
      for (int tb = 0; tb < C::TBW; ++tb) {
        const int t = wt * C::TW + tb * 16 + (lane & 15);
        float amax = 0.f;
#pragma unroll
        for (int w = 0; w < C::WN; ++w) amax = fmaxf(amax, red[w * BT + t]);
        const float s = amax / kE4m3Max;
        const float inv = requant_inv(amax, s);
        if (t < ep_rows) {
          uint8_t* dst = a.hq + (int64_t)(ep_p0 + t) * a.inter + ep_nt * 128 + wn * C::G + 4 * (lane >> 4);
#pragma unroll
          for (int g = 0; g < C::NB / 2; ++g) {
            int w = cvt2_e4m3(hv[tb][g][0] * inv, hv[tb][g][1] * inv, 0, false);
            w = cvt2_e4m3(hv[tb][g][2] * inv, hv[tb][g][3] * inv, w, true);
            *reinterpret_cast<uint32_t*>(dst + g * 16) = (uint32_t)w;
          }
          if (wn == 0 && (lane >> 4) == 0) a.hs[(int64_t)(ep_p0 + t) * ikb + ep_nt] = s;
        }
      }
    } else {
      const int n0 = ep_nt * kBN;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        const int n = (nb < C::NB / 2 ? wn * C::G + nb * 16 : 128 + wn * C::G + (nb - C::NB / 2) * 16) +
                      4 * (lane >> 4);
#pragma unroll
        for (int tb = 0; tb < C::TBW; ++tb) {
          const int t = wt * C::TW + tb * 16 + (lane & 15);
          if (t < ep_rows && n0 + n < a.n_rows) {
            u32x2 o;
            o[0] = f32_to_bf16_rne(acc[nb][tb][0]) | (f32_to_bf16_rne(acc[nb][tb][1]) << 16);
            o[1] = f32_to_bf16_rne(acc[nb][tb][2]) | (f32_to_bf16_rne(acc[nb][tb][3]) << 16);
            uint16_t* dst = a.y + (int64_t)(ep_p0 + t) * a.n_rows + n0 + n;
            if (a.fc.out)
              store_y_coherent(dst, o[0], o[1]);  // read by the workgroup that completes the token
            else
              *reinterpret_cast<u32x2*>(dst) = o;
          }
        }
      }
      if (a.fc.out)
        arrive_and_combine<kThreads>(a.fc, a.y, a.sorted_route, a.top_k, a.n_rows, a.n_tiles, ep_p0, ep_rows, ep_nt,
                                     (__attribute__((address_space(3))) int32_t*)cb_list,
                                     (__attribute__((address_space(3))) int32_t*)&cb_count);
    }
  }
}

template <int BT, bool FC1>
static int launch_one(const GemmArgs& a, void* stream) {
  hipLaunchKernelGGL((gemm_fp8_kernel<BT, FC1>), dim3(a.grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <bool FC1>
static int launch_bt(const GemmArgs& a, int block_m, void* stream) {
  switch (block_m) {
    case 16: return launch_one<16, FC1>(a, stream);
    case 32: return launch_one<32, FC1>(a, stream);
    case 64: return launch_one<64, FC1>(a, stream);
    case 128: return launch_one<128, FC1>(a, stream);
    case 256: return launch_one<256, FC1>(a, stream);
  }
  return -1;
}

int launch_fc1(const GemmArgs& a, int block_m, void* stream) { return launch_bt<true>(a, block_m, stream); }
int launch_fc2(const GemmArgs& a, int block_m, void* stream) { return launch_bt<false>(a, block_m, stream); }

template <int BT, bool FC1>
static int occ() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_fp8_kernel<BT, FC1>, kThreads, 0) != hipSuccess) return 1;
  return n > 0 ? n : 1;
}

int gemm_max_workgroups_per_cu(int which, int block_m) {
  const bool f1 = which == 1;
  switch (block_m) {
    case 16: return f1 ? occ<16, true>() : occ<16, false>();
    case 32: return f1 ? occ<32, true>() : occ<32, false>();
    case 64: return f1 ? occ<64, true>() : occ<64, false>();
    case 128: return f1 ? occ<128, true>() : occ<128, false>();
    default: return f1 ? occ<256, true>() : occ<256, false>();
  }
}

}  // namespace moe
