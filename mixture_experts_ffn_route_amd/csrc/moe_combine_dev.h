// Weighted top-k combine, as device functions: the standalone combine kernel
// and the fused last-arriver combine at the end of the FC2 GEMMs run the
// same per-column arithmetic, so the two give identical bits.
//
// Combine: out[t, :] = bf16_RNE( sum_{k = 0..K-1, kept} w[t, k] * y[pos(t, k), :] ),
// FP32 fused multiply-adds in ascending slot order from +0 ("feat(moe_ep):
// add SM90 push FP8 mega-MoE backend for Hopper", flashinfer PR #4069,
// Description: owner-side FP32 route reduction).
//
// Fused form (the SM90 pull-style MegaMoE, flashinfer PR #4688, commit list,
// combine-dedup / grouped token-back bullet: the last FC2 row of a token's
// group reduces every member in FP32): each FC2 tile that stores the y columns
// [nt*256, nt*256 + 256) of a route row counts one arrival on the counter of
// (token, nt).  The arrival that completes the token's kept routes reduces
// the token's K rows over those columns.  Counters return to zero once their
// token is reduced, so they start every forward at zero without a reset pass.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

typedef uint32_t cb_u32x4 __attribute__((ext_vector_type(4)));

// FC2 rows that another workgroup reduces are stored and read at agent
// scope: the stores write through to the device-coherent level and the loads
// read from it, so no cache-wide writeback or invalidate is needed between
// them (see arrive_and_combine).
__device__ __forceinline__ void store_y_coherent(uint16_t* p, uint32_t lo, uint32_t hi) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), (uint64_t)lo | ((uint64_t)hi << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

template <bool kCoherent>
__device__ __forceinline__ cb_u32x4 load_y16(const uint16_t* p) {
  if constexpr (kCoherent) {
    const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
    const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return cb_u32x4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
  } else {
    // non-temporal: each y row piece is read once, and the standalone
    // combine's output is written once (18% less combine time at T=4096
    // than with the default cache policy)
    return __builtin_nontemporal_load(reinterpret_cast<const cb_u32x4*>(p));
  }
}

// Columns [c, c + 8) of token t, for K routes per token, given the token's
// route positions and weights.  Slots that are not kept contribute
// fmaf(0, 0, acc).  Every slot's row is loaded without a branch (a slot
// that is not kept reads row 0, which exists, and then counts as zero), so
// the rows take one round trip.
template <int K, bool kCoherent>
__device__ __forceinline__ void combine8_pw(const uint16_t* y, const int (&pos)[K], const float (&w_in)[K], int64_t t,
                                            int hidden, int c, uint16_t* out) {
  float w[K];
  cb_u32x4 raw[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const bool keep = pos[k] >= 0;
    w[k] = w_in[k];
    raw[k] = load_y16<kCoherent>(y + (int64_t)(keep ? pos[k] : 0) * hidden + c);
    if (!keep) {
      w[k] = 0.f;
      raw[k] = cb_u32x4{0u, 0u, 0u, 0u};
    }
  }
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(w[k], bf16_to_f32(raw[k][i] & 0xffffu), acc[2 * i]);
      acc[2 * i + 1] = fmaf(w[k], bf16_to_f32(raw[k][i] >> 16), acc[2 * i + 1]);
    }
  }
  cb_u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = bf16x2_rne(acc[2 * i], acc[2 * i + 1]);
  if constexpr (kCoherent)
    *reinterpret_cast<cb_u32x4*>(out + t * hidden + c) = o;
  else
    __builtin_nontemporal_store(o, reinterpret_cast<cb_u32x4*>(out + t * hidden + c));
}

template <int K, bool kCoherent>
__device__ __forceinline__ void combine8_k(const uint16_t* y, const int32_t* route_pos, const float* route_w,
                                           int64_t t, int hidden, int c, uint16_t* out) {
  int pos[K];
  float w[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    pos[k] = route_pos[t * K + k];
    w[k] = route_w[t * K + k];
  }
  combine8_pw<K, kCoherent>(y, pos, w, t, hidden, c, out);
}

// K in {1, 2, 4, 6, 8} (the layer configuration is validated to those).
template <bool kCoherent>
__device__ __forceinline__ void combine8(const uint16_t* y, const int32_t* route_pos, const float* route_w,
                                         int64_t t, int K, int hidden, int c, uint16_t* out) {
  switch (K) {
    case 1: combine8_k<1, kCoherent>(y, route_pos, route_w, t, hidden, c, out); break;
    case 2: combine8_k<2, kCoherent>(y, route_pos, route_w, t, hidden, c, out); break;
    case 4: combine8_k<4, kCoherent>(y, route_pos, route_w, t, hidden, c, out); break;
    case 6: combine8_k<6, kCoherent>(y, route_pos, route_w, t, hidden, c, out); break;
    default: combine8_k<8, kCoherent>(y, route_pos, route_w, t, hidden, c, out); break;
  }
}

// Kept routes of token t (K <= 8).  The loads are unconditional (slot index
// clamped to K - 1) so all of them are in flight at once.
__device__ __forceinline__ int kept_routes(const int32_t* route_pos, int64_t t, int K) {
  int v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = route_pos[t * K + (k < K ? k : K - 1)];
  int n = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) n += (k < K && v[k] >= 0) ? 1 : 0;
  return n;
}

// Tokens with no kept route get a +0 row (no FC2 tile arrives for them).
// Grid-strided over the staged tokens, one thread per token; such tokens are
// rare, so the thread writes the whole row itself.
__device__ __forceinline__ void zero_unrouted_rows(const FusedCombineArgs& f, int tokens, int K, int hidden) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < tokens; t += stride) {
    if (kept_routes(f.route_pos, t, K) != 0) continue;
    cb_u32x4* row = reinterpret_cast<cb_u32x4*>(f.out + t * hidden);
    for (int c = 0; c < hidden / 8; ++c) row[c] = cb_u32x4{0u, 0u, 0u, 0u};
  }
}

// End of one FC2 tile (sorted rows [p0, p0 + rows), output columns
// [nt*256, nt*256 + 256)), after every thread of the workgroup has issued
// its y stores with store_y_coherent.  Called by all NTHREADS threads;
// `list` is LDS room for `rows` token ids and `count` one LDS word.
//
// Ordering across workgroups (which may sit on other XCDs, each with its own
// L2): each wave waits until its write-through y stores are complete before
// the workgroup barrier, the arrivals are agent-scope atomics after it, and
// the workgroup that completes a token reads the routes' rows with
// agent-scope loads after its atomic has returned.
template <int NTHREADS>
__device__ __forceinline__ void arrive_and_combine(const FusedCombineArgs& f, const uint16_t* y, const int32_t* sorted_route,
                                                   int K, int hidden, int n_tiles, int p0, int rows, int nt,
                                                   __attribute__((address_space(3))) int32_t* list,
                                                   __attribute__((address_space(3))) int32_t* count) {
  const int tid = threadIdx.x;
  if (tid == 0) *count = 0;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid < rows) {
    const int r = sorted_route[p0 + tid];
    const int64_t t = r / K;
    const int kept = kept_routes(f.route_pos, t, K);
    int32_t* ctr = f.arrive + t * n_tiles + nt;
    const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == kept) {
      // last arrival of this forward: the counter is free for the next one
      __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int slot = __hip_atomic_fetch_add(count, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      list[slot] = (int32_t)t;
    }
  }
  __syncthreads();
  const int n = *count;
  if (n == 0) return;
  constexpr int kPerRow = 32;  // threads per token: 32 x 8 columns = one tile width
  const int c = nt * 256 + (tid % kPerRow) * 8;
  if (c >= hidden) return;
  for (int i = tid / kPerRow; i < n; i += NTHREADS / kPerRow)
    combine8<true>(y, f.route_pos, f.route_w, list[i], K, hidden, c, f.out);
}

}  // namespace moe
