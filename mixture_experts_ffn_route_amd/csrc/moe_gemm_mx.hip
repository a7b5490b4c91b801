// MXFP8-weight x BF16-activation grouped GEMMs of the MoE layer on gfx950
// MX-scaled MFMA (the variant of "feat(moe_ep): MXFP8 x BF16 integration",
// flashinfer PR #4604, Description: e4m3 or e5m2 weights with one E8M0
// exponent per 32 K-elements, BF16 activations, BF16 h between the GEMMs).
//
// FC1: gu[p, n] = sum_k x[t, k] * w13[e, n, k] * 2^(s13[e, n, k/32] - 127)
//      h = bf16_RNE(silu(gate) * up)
// FC2: y[p, n]  = sum_k h[p, k] * w2[e, n, k] * 2^(s2[e, n, k/32] - 127)  -> bf16
//
// The scaled f8f6f4 MFMA takes FP8/FP6/FP4 operands only, so every BF16
// activation row is carried as two e4m3 terms with their own E8M0 exponent
// per 32 elements, hi = e4m3(x / 2^e_hi) and lo = e4m3((x - hi) / 2^e_lo)
// (made by the stage kernel for x and by the FC1 epilogue for h).  A K-block
// is then two scaled MFMAs into one FP32 accumulator; the hardware applies
// both the weight and the activation exponents, so no per-block VALU work
// remains.  hi + lo keeps 8 significant bits of each BF16 value; the
// remaining error is below 2^-9 relative per element.
//
// Structure as the FP8 kernel (moe_gemm_fp8.hip): swap-AB (weights are the
// MFMA row operand), 256 weight rows x BT tokens per workgroup tile, 8 waves,
// LDS-DMA ring with explicit waits, fragment-ordered LDS, persistent
// XCD-aware tile walk.  Per ring stage: 32 KB of weight codes, 1 KB of weight
// exponents, 2 x BT x 128 bytes of activation terms and BT x 16 bytes of
// activation exponents.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "moe_combine_dev.h"
#include "moe_device.h"
#include "moe_internal.h"
#include "moe_store_dev.h"

namespace moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kBN = 256;
constexpr int kKB = 128;
constexpr int kGroupM = 4;
constexpr int kLdsBytes = 160 * 1024;

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) const uint32_t lds_u32;

// Scaled MFMA: A = weights (row operand), B = activation term (column
// operand, always e4m3).  FA is the weight element type (0 e4m3, 1 e5m2).
// OA / OB pick the byte of the scale words: lane l's scale word supplies the
// exponent of row (or column) l%16 for 32-block l/16.
template <int FA, int OA, int OB>
__device__ __forceinline__ v4f mfma_mx(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, 0, OA, sa, OB, sb);
}

__device__ __forceinline__ v8i lds_frag(const lds_u8* p) {
  const u32x4 lo = *reinterpret_cast<lds_u32x4*>(p);
  const u32x4 hi = *reinterpret_cast<lds_u32x4*>(p + 1024);
  v8i r;
  r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
  r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
  return r;
}

// Token line layout in LDS: piece c (16 bytes) of token t of a 16-token
// area at position 8 t + (c ^ tok_swz(t)).  One DMA instruction then fills
// 8 whole 128-byte token lines (gathers of partial lines run at a fraction
// of the L2 rate), and the fragment reads of 16 consecutive lanes hit 16
// distinct 16-byte bank groups.
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

// LDS-DMA, explicit waits and a fence-free barrier, as in the FP8 kernel.
__device__ __forceinline__ uint32_t lds_addr(const lds_u8* p) { return (uint32_t)(uintptr_t)p; }
__device__ __forceinline__ void dma16(const uint8_t* src, const lds_u8* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds_addr(lds_wave_base)) : "memory", "m0");
}
// Weights of a tile that no other workgroup reads stream non-temporally
// (see the FP8 kernel).
__device__ __forceinline__ void dma16_nt(const uint8_t* src, const lds_u8* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :: "v"(src), "s"(lds_addr(lds_wave_base)) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const uint32_t* src, const lds_u8* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(lds_addr(lds_wave_base)) : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

template <int BT>
struct MxCfg {
  static constexpr int WN = BT >= 64 ? 2 : (BT == 32 ? 4 : 8);  // waves along weight rows
  static constexpr int WT = kWaves / WN;
  static constexpr int G = 128 / WN;          // rows of each 128-row half per wave
  static constexpr int NBH = G / 16;          // 16-row blocks per half per wave (1, 2 or 4)
  static constexpr int NB = 2 * NBH;
  static constexpr int TW = BT / WT;
  static constexpr int TBW = TW / 16;
  static constexpr int A_BYTES = kBN * kKB;   // weight codes
  static constexpr int AS_BYTES = 1024;       // weight exponents
  static constexpr int B_BYTES = 2 * BT * kKB;  // hi and lo activation terms
  static constexpr int BS_BYTES = ((BT * 16 + 255) / 256) * 256;  // activation exponent words
  static constexpr int STAGE = A_BYTES + AS_BYTES + B_BYTES + BS_BYTES;
  static constexpr int STAGES = (kLdsBytes / STAGE) > 4 ? 4 : (kLdsBytes / STAGE);
  static constexpr int B_PIECES = 2 * BT;     // 16-byte activation pieces per wave per stage
  static constexpr int B_INSTR = (B_PIECES + 63) / 64;
  static constexpr int B_LANES = B_PIECES < 64 ? B_PIECES : 64;
  static constexpr int BS_LANES = BT / 2;     // activation exponent words per wave per stage
  static constexpr int N_LD = 4 + 1 + B_INSTR + 1;
  static_assert(TBW >= 1 && NBH >= 1 && NBH <= 4 && STAGES >= 2, "tile shape");
  static_assert(BS_LANES <= 64 && (STAGES - 2) * N_LD < 64, "load shape");
};

template <int BT, bool FC1, int FA>
__global__ __launch_bounds__(kThreads, 1) void gemm_mx_kernel(MxGemmArgs a) {
  using C = MxCfg<BT>;
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[C::STAGES > 2 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t ring3[C::STAGES > 3 ? C::STAGE : 16];
  // FC1 epilogue: per-32-row block maxima of h (pass 1) and of h - hi (pass
  // 2), [16-row block][token]; outside the ring, which holds the next
  // tile's first stages by then
  __shared__ __attribute__((aligned(16))) float red_s[FC1 ? 2 * 8 * BT : 4];
  __shared__ int32_t cb_list[FC1 ? 1 : BT];  // FC2 fused combine: tokens this tile completes
  __shared__ int32_t cb_count;
  auto ring = [&](auto stage) -> lds_u8* {
    constexpr int S = decltype(stage)::value;
    if constexpr (S == 0) return (lds_u8*)ring0;
    else if constexpr (S == 1) return (lds_u8*)ring1;
    else if constexpr (S == 2) return (lds_u8*)ring2;
    else return (lds_u8*)ring3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % C::WN, wt = wave / C::WN;
  const int kbs = a.k_dim / kKB;
  const int kq = a.k_dim / 32;
  const int total_m = __builtin_amdgcn_readfirstlane((int)a.hdr[kHdrMTiles]);
  const int64_t total = (int64_t)total_m * a.n_tiles;
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int per_xcd = gridDim.x >> 3;
  const int64_t v_begin = total * xcd / 8, v_end = total * (xcd + 1) / 8;
  // Active slots of this XCD: the fewest that still finish its tiles in
  // ceil(tiles / slots) rounds, so that every active workgroup streams in
  // every round (with 112 tiles on 32 slots: 28 slots x 4 rounds rather
  // than 16 x 4 + 16 x 3, whose last round runs half the XCD's CUs).
  const int64_t rounds = (v_end - v_begin + per_xcd - 1) / per_xcd;
  const int stride = rounds > 0 ? (int)((v_end - v_begin + rounds - 1) / rounds) : per_xcd;
  const uint32_t a_lane = (uint32_t)(wn * C::NBH) * 2048u + (uint32_t)lane * 16u;
  // token fragment of lane (token tl, K-group q): pieces q and q + 4 of its
  // token line (the scaled MFMA's K order: bytes 16q.. and 64 + 16q..)
  const int tl = lane & 15, lq = lane >> 4;
  const uint32_t b_lo = (uint32_t)(wt * C::TBW) * 4096u + 16u * (uint32_t)(8 * tl + (lq ^ tok_swz(tl)));
  const uint32_t b_hi = (uint32_t)(wt * C::TBW) * 4096u + 16u * (uint32_t)(8 * tl + ((lq + 4) ^ tok_swz(tl)));
  const uint32_t bs_lane = (uint32_t)(wt * C::TBW * 64 + lane);
  // weight exponents: word group of the wave's first gate/first-half block,
  // and the byte of that block inside the word
  const int sa_grp = (wn * C::NBH) / 4;
  const int sa_shift = 8 * ((wn * C::NBH) % 4);

  // ---- tile state, set one tile ahead: the next tile's first stages are
  // issued before the current tile's epilogue, which hides their latency ----
  int e = 0, p0 = 0, rows_valid = 1, nt = 0;
  bool w_once = false;  // the tile's expert has a single row tile: no other workgroup reads its weights
  const uint8_t* a_src = a.w;
  const uint32_t* as_src = a.w_scale;
  const uint8_t* b_src[C::B_INSTR];
  const uint32_t* bs_src = a.a_scale;
  auto src_row = [&](int t) -> int64_t {
    const int p = p0 + min(t, rows_valid - 1);
    if (!FC1) return p;
    const int r = a.sorted_route[p];
    return r / a.top_k;
  };
  // Row tile of tile index v (token tiles grouped kGroupM deep, column tile
  // fastest within a group).
  auto row_tile = [&](int64_t v) -> int {
    const int64_t group = v / ((int64_t)kGroupM * a.n_tiles);
    const int64_t rem = v - group * kGroupM * a.n_tiles;
    const int g0 = (int)(group * kGroupM);
    return g0 + (int)(rem % min(kGroupM, total_m - g0));
  };
  // `rec` is the row tile's record (load_tile_rec), fetched ahead of time.
  auto setup = [&](int64_t v, tile_rec_t rec) {
    const int64_t group = v / ((int64_t)kGroupM * a.n_tiles);
    const int64_t rem = v - group * kGroupM * a.n_tiles;
    const int m0 = (int)(group * kGroupM);
    const int gm = min(kGroupM, total_m - m0);
    nt = (int)(rem / gm);
    e = __builtin_amdgcn_readfirstlane(rec[0]);
    p0 = __builtin_amdgcn_readfirstlane(rec[1]);
    rows_valid = __builtin_amdgcn_readfirstlane(rec[2]);
    w_once = __builtin_amdgcn_readfirstlane(rec[3]) != 0;
    const int64_t tile0 = ((int64_t)e * a.n_tiles + nt) * kbs;
    a_src = a.w + tile0 * C::A_BYTES + (wave * 4 * 64 + lane) * 16;
    as_src = a.w_scale + tile0 * 256 + wave * 32 + (lane < 32 ? lane : 0);
    // activation terms: 2 KB per (token block, term), 16-byte piece c of
    // token t at position 8 t + (c ^ tok_swz(t)), so that 8 consecutive
    // lanes read one whole 128-byte token line; piece pv of the wave is
    // position pv % 128 of area pv / 128
#pragma unroll
    for (int j = 0; j < C::B_INSTR; ++j) {
      const int pv = wave * C::B_PIECES + j * 64 + (lane < C::B_LANES ? lane : 0);
      const int area = pv >> 7, pos = pv & 127;
      const int tt = pos >> 3;
      const int t = (area >> 1) * 16 + tt;
      const int c = (pos & 7) ^ tok_swz(tt);
      b_src[j] = a.a + (area & 1) * a.a_plane + src_row(t) * a.k_dim + 16 * c;
    }
    // activation exponents: word U covers token block U/64, lane U%64 =
    // token (U%16) and 32-block (U%64)/16
    const int u = wave * C::BS_LANES + (lane < C::BS_LANES ? lane : 0);
    const int lp = u & 63;
    bs_src = a.a_scale + src_row((u >> 6) * 16 + (lp & 15)) * kq + (lp >> 4);
  };

  auto issue = [&](auto stage, int kb) {
    const lds_u8* As = ring(stage);
    const lds_u8* ASs = As + C::A_BYTES;
    const lds_u8* Bs = ASs + C::AS_BYTES;
    const lds_u8* BSs = Bs + C::B_BYTES;
    if (w_once) {
#pragma unroll
      for (int j = 0; j < 4; ++j) dma16_nt(a_src + (int64_t)kb * C::A_BYTES + j * 1024, As + (wave * 4 + j) * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) dma16(a_src + (int64_t)kb * C::A_BYTES + j * 1024, As + (wave * 4 + j) * 1024);
    }
    if (lane < 32) dma4(as_src + kb * 256, ASs + wave * 128);
#pragma unroll
    for (int j = 0; j < C::B_INSTR; ++j)
      if (lane < C::B_LANES) dma16(b_src[j] + kb * kKB, Bs + (wave * C::B_PIECES + j * 64) * 16);
    if (lane < C::BS_LANES) dma4(bs_src + kb * 4, BSs + wave * C::BS_LANES * 4);
  };
  auto prologue = [&]() {
    issue(std::integral_constant<int, 0>{}, 0);
    if (C::STAGES > 2 && 1 < kbs) issue(std::integral_constant<int, 1>{}, 1);
    if (C::STAGES > 3 && 2 < kbs) issue(std::integral_constant<int, (C::STAGES > 3 ? 2 : 0)>{}, 2);
  };

  // FC2's output stores stay in flight into the next tile's first steps, as
  // in the FP8 kernel: kEpiStores buffer stores per wave, issued after the
  // next tile's first STAGES - 1 stages, so the waits for those stages allow
  // for kEpiStores newer operations.  The tile's BF16 rows go out through
  // the ring's last stage, whole rows per store (two 512-byte rows per
  // instruction): BT / 16 stores per wave.  The first tile adds kEpiStores
  // stores that write nothing; the fused-combine epilogue waits for every
  // outstanding operation before it stores.
  constexpr bool kStoreOverlap = !FC1;
  constexpr int kEpiStores = BT / 16;
  static_assert(BT * 512 <= C::STAGE, "output staging");
  static_assert((C::STAGES - 2) * C::N_LD + kEpiStores < 64, "vmcnt range");

  if constexpr (!FC1) {
    if (a.fc.out) zero_unrouted_rows(a.fc, (int)a.hdr[kHdrTokens], a.top_k, a.n_rows);
  }
  int64_t v = slot < stride ? v_begin + slot : v_end;
  if (v < v_end) {
    setup(v, load_tile_rec(a.tiles, row_tile(v)));
    prologue();
    if constexpr (kStoreOverlap) {
      const st_u32x4 none = buffer_rsrc(a.y, 0u);
#pragma unroll
      for (int i = 0; i < kEpiStores; ++i) buffer_store_none(none);
    }
  }
  for (; v < v_end; v += stride) {
    // the next tile's record, in flight while this tile's first stage lands
    tile_rec_t rec_next = {0, 0, 1, 0};
    if (v + stride < v_end) rec_next = load_tile_rec(a.tiles, row_tile(v + stride));
    v4f acc[C::NB][C::TBW];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int tb = 0; tb < C::TBW; ++tb) acc[nb][tb] = v4f{0.f, 0.f, 0.f, 0.f};

    auto step = [&](auto stage, int kb) {
      constexpr int ST = decltype(stage)::value;
      const int ahead = min(C::STAGES - 2, kbs - 1 - kb);
      if (kStoreOverlap && ST <= C::STAGES - 2 && kb <= C::STAGES - 2) {
        // stage kb came from the prologue, before the previous epilogue's stores
        if (C::STAGES >= 4 && ahead >= 2) wait_vmcnt<(C::STAGES >= 4 ? 2 : 0) * C::N_LD + kEpiStores>();
        else if (C::STAGES >= 3 && ahead >= 1) wait_vmcnt<(C::STAGES >= 3 ? 1 : 0) * C::N_LD + kEpiStores>();
        else wait_vmcnt<kEpiStores>();
      } else {
        if (C::STAGES >= 4 && ahead >= 2) wait_vmcnt<(C::STAGES >= 4 ? 2 : 0) * C::N_LD>();
        else if (C::STAGES >= 3 && ahead >= 1) wait_vmcnt<(C::STAGES >= 3 ? 1 : 0) * C::N_LD>();
        else wait_vmcnt<0>();
      }
      barrier_nofence();
      if (kb + C::STAGES - 1 < kbs)
        issue(std::integral_constant<int, (ST + C::STAGES - 1) % C::STAGES>{}, kb + C::STAGES - 1);

      const lds_u8* As = ring(stage);
      const lds_u32* ASs = (const lds_u32*)(As + C::A_BYTES);
      const lds_u8* Bs = As + C::A_BYTES + C::AS_BYTES;
      const lds_u32* BSs = (const lds_u32*)(Bs + C::B_BYTES);
      const lds_u8* Ap = As + a_lane;
      v8i bh[C::TBW], bl[C::TBW];
      int sb[C::TBW];
#pragma unroll
      for (int tb = 0; tb < C::TBW; ++tb) {
        bh[tb] = lds_frag2(Bs + b_lo + tb * 4096, Bs + b_hi + tb * 4096);
        bl[tb] = lds_frag2(Bs + b_lo + tb * 4096 + 2048, Bs + b_hi + tb * 4096 + 2048);
        sb[tb] = (int)BSs[bs_lane + tb * 64];
      }
      const int sa_g = (int)(ASs[sa_grp * 64 + lane] >> sa_shift);
      const int sa_u = (int)(ASs[(2 + sa_grp) * 64 + lane] >> sa_shift);
      auto aoff = [](int nb) { return (nb < C::NBH ? nb : 8 - C::NBH + nb) * 2048; };
      v8i aq = lds_frag(Ap + aoff(0));
      static_for<0, C::NB>([&](auto nbc) {
        constexpr int nb = decltype(nbc)::value;
        constexpr int OA = nb % C::NBH;
        const v8i an = lds_frag(Ap + aoff(nb + 1 < C::NB ? nb + 1 : nb));
        const int sa = nb < C::NBH ? sa_g : sa_u;
#pragma unroll
        for (int tb = 0; tb < C::TBW; ++tb) {
          acc[nb][tb] = mfma_mx<FA, OA, 0>(aq, bh[tb], acc[nb][tb], sa, sb[tb]);
          acc[nb][tb] = mfma_mx<FA, OA, 1>(aq, bl[tb], acc[nb][tb], sa, sb[tb]);
        }
        __builtin_amdgcn_sched_barrier(0);
        aq = an;
      });
      // every LDS read of this stage is complete before the next barrier
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    };
    for (int kb = 0; kb < kbs; kb += C::STAGES) {
      step(std::integral_constant<int, 0>{}, kb);
      if (kb + 1 < kbs) step(std::integral_constant<int, 1>{}, kb + 1);
      if (C::STAGES > 2 && kb + 2 < kbs) step(std::integral_constant<int, (C::STAGES > 2 ? 2 : 0)>{}, kb + 2);
      if (C::STAGES > 3 && kb + 3 < kbs) step(std::integral_constant<int, (C::STAGES > 3 ? 3 : 0)>{}, kb + 3);
    }
    // Every wave is done reading the ring before the next tile's first
    // stages go into it.  LDS-only barrier: nothing of this tile is in
    // flight, and a fenced one would also wait for the previous tile's
    // output stores.
    barrier_nofence();
    const int ep_p0 = p0, ep_rows = rows_valid, ep_nt = nt;
    if (v + stride < v_end) {
      setup(v + stride, rec_next);
      prologue();
    }

    if (FC1) {
      // h = bf16(silu(g) * up), then the two-term split per 32 rows of h.
      // A lane holds 4 consecutive rows of a 16-row block for one token; a
      // 32-block is two row blocks, which may sit in different waves, so the
      // block maxima go through LDS: red[rb][t] (pass 1: |h|, pass 2: |h - hi|).
      // The exchanges wait on LDS only: a fenced barrier would also wait for
      // the next tile's stages issued above.
      float* red1 = red_s;
      float* red2 = red1 + 8 * BT;
      const int iq = a.inter / 32;
      float hv[C::TBW][C::NBH][4];
#pragma unroll
      for (int tb = 0; tb < C::TBW; ++tb)
#pragma unroll
        for (int g = 0; g < C::NBH; ++g) {
          float m = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gt = acc[g][tb][i], up = acc[C::NBH + g][tb][i];
            const float h = bf16_to_f32(f32_to_bf16_rne(gt / (1.0f + expf(-gt)) * up));
            hv[tb][g][i] = h;
            m = fmaxf(m, fabsf(h));
          }
          m = fmaxf(m, __shfl_xor(m, 16));
          m = fmaxf(m, __shfl_xor(m, 32));
          if (lane < 16) red1[(wn * C::NBH + g) * BT + wt * C::TW + tb * 16 + lane] = m;
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      barrier_nofence();
      uint32_t hi_codes[C::TBW][C::NBH];
      int ehi[C::TBW][C::NBH];
#pragma unroll
      for (int tb = 0; tb < C::TBW; ++tb)
#pragma unroll
        for (int g = 0; g < C::NBH; ++g) {
          const int t = wt * C::TW + tb * 16 + (lane & 15);
          const int rb = wn * C::NBH + g;
          const int r0 = rb & ~1;
          ehi[tb][g] = mx_block_exp(fmaxf(red1[r0 * BT + t], red1[(r0 + 1) * BT + t]));
          float r[4];
          hi_codes[tb][g] = mx_term4(hv[tb][g], ehi[tb][g], r);
          float m = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            hv[tb][g][i] = r[i];
            m = fmaxf(m, fabsf(r[i]));
          }
          m = fmaxf(m, __shfl_xor(m, 16));
          m = fmaxf(m, __shfl_xor(m, 32));
          if (lane < 16) red2[rb * BT + t] = m;
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      barrier_nofence();
#pragma unroll
      for (int tb = 0; tb < C::TBW; ++tb)
#pragma unroll
        for (int g = 0; g < C::NBH; ++g) {
          const int t = wt * C::TW + tb * 16 + (lane & 15);
          const int rb = wn * C::NBH + g;
          const int r0 = rb & ~1;
          const int elo = mx_block_exp(fmaxf(red2[r0 * BT + t], red2[(r0 + 1) * BT + t]));
          float unused[4];
          const uint32_t lo_codes = mx_term4(hv[tb][g], elo, unused);
          if (t < ep_rows) {
            const int64_t off = (int64_t)(ep_p0 + t) * a.inter + ep_nt * 128 + rb * 16 + 4 * (lane >> 4);
            *reinterpret_cast<uint32_t*>(a.hq + off) = hi_codes[tb][g];
            *reinterpret_cast<uint32_t*>(a.hq + a.h_plane + off) = lo_codes;
            if ((rb & 1) == 0 && (lane >> 4) == 0)
              a.hs[(int64_t)(ep_p0 + t) * iq + ep_nt * 4 + rb / 2] =
                  (uint32_t)(ehi[tb][g] + 127) | ((uint32_t)(elo + 127) << 8);
          }
        }
    } else {
      const int n0 = ep_nt * kBN;
      if (a.fc.out == nullptr) {
        // The tile's rows are transposed through the ring's last stage (free:
        // the next tile's prologue fills the others): a lane's MFMA outputs
        // are 4 columns of one row, so direct stores would write 32-byte
        // pieces of 16 rows.  LDS holds BT rows x 32 chunks of 16 bytes,
        // chunk c of row r at position c ^ (r & 31).  One buffer from the
        // tile's first row holds only its valid rows, so rows past ep_rows
        // fall past its end; with an odd number of 128-column blocks in H,
        // the last tile's second half (chunks 16..31) goes out of range.
        lds_u8* ys = ring(std::integral_constant<int, C::STAGES - 1>{});
        const bool hi_ok = n0 + 128 < a.n_rows;
        // an opaque copy of the lane index keeps the address terms from being
        // hoisted out of the tile loop (and held across the K loop)
        int ln;
        asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
        const int lq4 = 4 * (ln >> 4), lr = ln & 15;
#pragma unroll
        for (int tb = 0; tb < C::TBW; ++tb) {
          const int r = wt * C::TW + tb * 16 + lr;
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) {
            // first of this lane's 4 columns
            const int c = (nb < C::NBH ? wn * C::G + nb * 16 : 128 + wn * C::G + (nb - C::NBH) * 16) + lq4;
            u32x2 o;
            o[0] = bf16x2_rne(acc[nb][tb][0], acc[nb][tb][1]);
            o[1] = bf16x2_rne(acc[nb][tb][2], acc[nb][tb][3]);
            *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
                ys + r * 512 + (((c >> 3) ^ (r & 31)) << 4) + (c & 7) * 2) = o;
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        barrier_nofence();
        // whole rows out: wave w stores the row pairs w * BT / 16 ..
        const int rd_row = ln >> 5, rd_chunk = ln & 31;
        const uint32_t rd_col_off = (uint32_t)((n0 + rd_chunk * 8) * 2);
        const st_u32x4 rs = buffer_rsrc(a.y + (int64_t)ep_p0 * a.n_rows, (uint32_t)(ep_rows * a.n_rows * 2));
#pragma unroll
        for (int i = 0; i < BT / 16; ++i) {
          const int r = (wave * (BT / 16) + i) * 2 + rd_row;
          const u32x4 d = *reinterpret_cast<lds_u32x4*>(ys + r * 512 + ((rd_chunk ^ (r & 31)) << 4));
          const uint32_t voff = (rd_chunk < 16 || hi_ok) ? (uint32_t)(r * a.n_rows * 2) + rd_col_off : 0x7ffffff0u;
          buffer_store16(d, voff, rs);
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          const int n = (nb < C::NBH ? wn * C::G + nb * 16 : 128 + wn * C::G + (nb - C::NBH) * 16) + 4 * (lane >> 4);
#pragma unroll
          for (int tb = 0; tb < C::TBW; ++tb) {
            const int t = wt * C::TW + tb * 16 + (lane & 15);
            if (t < ep_rows && n0 + n < a.n_rows) {
              u32x2 o;
              o[0] = bf16x2_rne(acc[nb][tb][0], acc[nb][tb][1]);
              o[1] = bf16x2_rne(acc[nb][tb][2], acc[nb][tb][3]);
              store_y_coherent(a.y + (int64_t)(ep_p0 + t) * a.n_rows + n0 + n, o[0], o[1]);  // read by the workgroup that completes the token
            }
          }
        }
        // (its opening vmcnt(0) also completes the next tile's prologue
        // stages, so the next tile's first waits hold without more stores)
        arrive_and_combine<kThreads>(a.fc, a.y, a.sorted_route, a.top_k, a.n_rows, a.n_tiles, ep_p0, ep_rows, ep_nt,
                                     (__attribute__((address_space(3))) int32_t*)cb_list,
                                     (__attribute__((address_space(3))) int32_t*)&cb_count);
      }
    }
  }
}

#include "moe_gemm_mx_pp.inc"

// 128-token tiles without the fused combine run the ping-pong kernel.
template <int BT, bool FC1>
int launch_one(const MxGemmArgs& a, void* stream) {
  if constexpr (BT == 128) {
    if (a.fc.out == nullptr) {
      if (a.w_e5m2)
        hipLaunchKernelGGL((gemm_mx_pp_kernel<FC1, 1>), dim3(a.grid), dim3(kThreads), 0,
                           static_cast<hipStream_t>(stream), a);
      else
        hipLaunchKernelGGL((gemm_mx_pp_kernel<FC1, 0>), dim3(a.grid), dim3(kThreads), 0,
                           static_cast<hipStream_t>(stream), a);
      return hipGetLastError() == hipSuccess ? 0 : -1;
    }
  }
  if (a.w_e5m2)
    hipLaunchKernelGGL((gemm_mx_kernel<BT, FC1, 1>), dim3(a.grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       a);
  else
    hipLaunchKernelGGL((gemm_mx_kernel<BT, FC1, 0>), dim3(a.grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <bool FC1>
int launch_bt(const MxGemmArgs& a, int block_m, void* stream) {
  switch (block_m) {
    case 16: return launch_one<16, FC1>(a, stream);
    case 32: return launch_one<32, FC1>(a, stream);
    case 64: return launch_one<64, FC1>(a, stream);
    case 128: return launch_one<128, FC1>(a, stream);
  }
  return -1;
}

template <int BT, bool FC1>
int occ() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_mx_kernel<BT, FC1, 0>, kThreads, 0) != hipSuccess) return 1;
  if constexpr (BT == 128) {  // the grid serves either kernel: the smaller occupancy
    int m = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&m, gemm_mx_pp_kernel<FC1, 0>, kThreads, 0) != hipSuccess) return 1;
    n = m < n ? m : n;
  }
  return n > 0 ? n : 1;
}

}  // namespace

int launch_fc1_mx(const MxGemmArgs& a, int block_m, void* stream) { return launch_bt<true>(a, block_m, stream); }
int launch_fc2_mx(const MxGemmArgs& a, int block_m, void* stream) { return launch_bt<false>(a, block_m, stream); }

int gemm_mx_max_workgroups_per_cu(int which, int block_m) {
  const bool f1 = which == 1;
  switch (block_m) {
    case 16: return f1 ? occ<16, true>() : occ<16, false>();
    case 32: return f1 ? occ<32, true>() : occ<32, false>();
    case 64: return f1 ? occ<64, true>() : occ<64, false>();
    default: return f1 ? occ<128, true>() : occ<128, false>();
  }
}

}  // namespace moe
