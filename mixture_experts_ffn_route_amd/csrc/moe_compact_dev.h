// Device-side route compaction, run by the staging launch (route staging
// and counting, or the whole compaction for one workgroup) and by the
// scatter kernel.  See moe_compact.hip for the method.
#pragma once

#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kCompactThreads = 256;
constexpr int kCompactWaves = kCompactThreads / 64;
constexpr int kItems = kCompactChunk / kCompactThreads;  // routes per lane per block (a.chunk <= kCompactChunk)
static_assert(kCompactOneRoutes <= kCompactChunk && kCompactBlockRoutes <= kCompactChunk && kCompactBlockRoutes >= 8,
              "a compaction workgroup holds at most kCompactChunk routes and at least one token of 8");

__device__ __forceinline__ int id_bits(int num_experts) {
  int b = 0;
  while ((1 << b) < num_experts) ++b;
  return b;
}

// Lanes of this wave whose route has the same expert as this lane (valid lanes only).
__device__ __forceinline__ uint64_t peers_of(int e, bool valid, int nbits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

// The routes a wave walks in block blk (routes [blk * chunk, blk * chunk +
// chunk)): the block's routes split into kCompactWaves ascending contiguous
// ranges of whole 64-route items (at most kItems each), so a small batch
// spreads over every wave.  Sweep and scatter use the same split.  The last
// wave's items may reach past the block's routes (a chunk of K=6 routes per
// token is not a multiple of 256): `end` bounds them.
struct WaveRange {
  int64_t base;
  int64_t end;  // the block's last route + 1
  int items;
};
__device__ inline WaveRange wave_range(const CompactArgs& a, int blk, int wave) {
  const int64_t b0 = (int64_t)blk * a.chunk;
  const int64_t n = min((int64_t)a.routes - b0, (int64_t)a.chunk);
  const int items = (int)((n + 64 * kCompactWaves - 1) / (64 * kCompactWaves));
  return WaveRange{b0 + (int64_t)wave * items * 64, b0 + n, items};
}

// Walk this block's routes wave by wave.  hist[w*E + e] holds wave w's
// running count; rank[i] receives the count of same-expert routes before
// item i within this wave's range.  ids_lds: the block's staged expert ids
// in LDS, from its first route on (the staging launch keeps them there),
// else they are read from a.staged_idx.
__device__ inline void sweep(const CompactArgs& a, int blk, int* hist, int* rank, int* expert,
                             const int* ids_lds = nullptr) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nbits = id_bits(a.num_experts);
  const WaveRange wr = wave_range(a, blk, wave);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // All of this lane's expert ids first: the histogram updates below go
  // through a generic pointer, so a load placed after one of them would
  // wait for the previous item's load to return.
  int ids[kItems];
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    const int64_t r = wr.base + it * 64 + lane;
    ids[it] = -1;
    if (it < wr.items && r < wr.end) ids[it] = ids_lds ? ids_lds[r - (int64_t)blk * a.chunk] : a.staged_idx[r];
  }
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    if (it >= wr.items) break;
    const int e = ids[it];
    const bool valid = e >= 0;
    const uint64_t pm = peers_of(e, valid, nbits);
    const int below = __popcll(pm & lt);
    int run = 0;
    if (valid) run = hist[wave * a.num_experts + e];
    rank[it] = run + below;
    expert[it] = e;
    if (valid && below == 0) hist[wave * a.num_experts + e] = run + __popcll(pm);
  }
}

__device__ inline void clear_hist(int* hist, int n) {
  for (int i = threadIdx.x; i < n; i += kCompactThreads) hist[i] = 0;
}

// Exclusive prefix sum of v[0..n) in place (n <= 1024) by wave 0; returns the total.
__device__ inline int wave0_exclusive_scan(int* v, int n, int* total_out) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (n + 63) / 64;
    int s = 0;
    for (int i = 0; i < per; ++i) {
      const int j = lane * per + i;
      if (j < n) s += v[j];
    }
    int incl = s;
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    int run = incl - s;
    for (int i = 0; i < per; ++i) {
      const int j = lane * per + i;
      if (j < n) {
        const int c = v[j];
        v[j] = run;
        run += c;
      }
    }
    if (lane == 63) *total_out = incl;
  }
  __syncthreads();
  return *total_out;
}

// From full per-expert counts in `cnt` (LDS, E entries): kept counts/offsets,
// capacity flag, route total and the tile list.  `tmp` is LDS scratch of E+1.
__device__ inline void finish_counts(const CompactArgs& a, int* cnt, int* tmp, int* scalar) {
  const int E = a.num_experts;
  // full exclusive offsets -> tmp
  for (int e = threadIdx.x; e < E; e += kCompactThreads) tmp[e] = cnt[e];
  __syncthreads();
  const int total = wave0_exclusive_scan(tmp, E, scalar);
  const int cap = a.row_cap;
  for (int e = threadIdx.x; e < E; e += kCompactThreads) {
    const int lo = min(tmp[e], cap);
    const int hi = min(tmp[e] + cnt[e], cap);
    a.offsets[e] = lo;
    a.counts[e] = hi - lo;
  }
  if (threadIdx.x == 0) {
    a.offsets[E] = min(total, cap);
    a.hdr[kHdrRoutes] = (uint32_t)min(total, cap);
    if (total > cap) atomicOr(a.hdr + kHdrStatus, (uint32_t)MOE_DEV_CAPACITY);
  }
  __syncthreads();
  // tiles per expert (kept rows), scanned into cnt (reused)
  for (int e = threadIdx.x; e < E; e += kCompactThreads) {
    const int lo = min(tmp[e], cap), hi = min(tmp[e] + cnt[e], cap);
    cnt[e] = (hi - lo + a.block_m - 1) / a.block_m;
  }
  __syncthreads();
  // keep the full offsets in tmp; scan tiles in cnt
  const int ntiles = wave0_exclusive_scan(cnt, E, scalar + 1);
  for (int e = threadIdx.x; e < E; e += kCompactThreads) {
    const int lo = min(tmp[e], cap);
    const int kept_hi = (e + 1 < E) ? min(tmp[e + 1], cap) : min(total, cap);
    int m = cnt[e];
    for (int p = lo; p < kept_hi; p += a.block_m, ++m) {
      a.tiles[4 * m] = e;
      a.tiles[4 * m + 1] = p;
      a.tiles[4 * m + 2] = min(a.block_m, kept_hi - p);        // rows of this tile
      a.tiles[4 * m + 3] = kept_hi - lo <= a.block_m ? 1 : 0;  // the expert's only row tile
      if (a.ready) a.ready[m] = 0;
    }
  }
  if (threadIdx.x == 0) a.hdr[kHdrMTiles] = (uint32_t)ntiles;
}

// Positions from the per-wave running ranks; wave bases come from
// blk_base (this block's first position per expert) plus earlier waves.
__device__ inline void scatter(const CompactArgs& a, int blk, int* hist, const int* blk_start, const int* rank,
                        const int* expert) {
  const int E = a.num_experts;
  for (int e = threadIdx.x; e < E; e += kCompactThreads) {
    int run = blk_start[e];
    for (int w = 0; w < kCompactWaves; ++w) {
      const int c = hist[w * E + e];
      hist[w * E + e] = run;
      run += c;
    }
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const WaveRange wr = wave_range(a, blk, wave);
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    if (it >= wr.items) break;
    const int64_t r = wr.base + it * 64 + lane;
    if (r >= wr.end) continue;
    const int e = expert[it];
    int p = -1;
    if (e >= 0) {
      p = hist[wave * E + e] + rank[it];
      if (p < a.row_cap) {
        a.sorted_route[p] = (int)r;
      } else {
        p = -1;
      }
    }
    a.route_pos[r] = p;
  }
}

// Single-workgroup compaction (routes <= a.chunk): count, scan, scatter.
// `lds` holds compact_one_workgroup_lds(E) bytes; ids_lds as in sweep.
__device__ inline void compact_one_workgroup(const CompactArgs& a, int* lds, const int* ids_lds = nullptr) {
  const int E = a.num_experts;
  int* hist = lds;                        // [waves, E]
  int* cnt = hist + kCompactWaves * E;    // [E]
  int* tmp = cnt + E;                     // [E + 1]
  int* scalar = tmp + E + 1;              // [2]
  int rank[kItems], expert[kItems];
  clear_hist(hist, kCompactWaves * E);
  __syncthreads();
  sweep(a, 0, hist, rank, expert, ids_lds);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kCompactThreads) {
    int s = 0;
    for (int w = 0; w < kCompactWaves; ++w) s += hist[w * E + e];
    cnt[e] = s;
  }
  __syncthreads();
  finish_counts(a, cnt, tmp, scalar);
  __syncthreads();
  scatter(a, 0, hist, tmp, rank, expert);  // tmp holds the full exclusive offsets
}

__host__ __device__ inline size_t compact_one_workgroup_lds(int num_experts) {
  return (size_t)(kCompactWaves * num_experts + num_experts + num_experts + 1 + 3) * 4;
}

// Values one compaction workgroup hands to another within a launch: stored
// write-through and loaded from the device-coherent level (agent scope), so
// that no cache-wide writeback or invalidate is needed between them.
__device__ __forceinline__ void store_agent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_agent(int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Compaction over several workgroups, all but the scatter (which needs
// every workgroup's bases, so it is a launch of its own): workgroup blk
// counts its routes per expert and publishes the counts and its route rows'
// status bits.  The workgroup whose arrival completes the count writes the
// header (tokens, every workgroup's status bits), turns the counts into
// offsets, per-workgroup bases and the tile list, and returns the arrival
// counter to zero.
//
// Ordering: each wave waits until its write-through stores are complete
// before the workgroup barrier, the arrival is an agent-scope atomic after
// it, and the completing workgroup loads the counts at agent scope after its
// atomic has returned.  No workgroup waits for another.
__device__ inline void count_and_arrive(const CompactArgs& a, int blk, int* lds, int* ids_lds,
                                        uint32_t status, int32_t tokens) {
  const int E = a.num_experts;
  int* hist = lds;                        // [waves, E]
  int* cnt = hist + kCompactWaves * E;    // [E]
  int* tmp = cnt + E;                     // [E + 1]
  int* scalar = tmp + E + 1;              // [3]
  int rank[kItems], expert[kItems];
  clear_hist(hist, kCompactWaves * E);
  __syncthreads();
  sweep(a, blk, hist, rank, expert, ids_lds);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kCompactThreads) {
    int s = 0;
    for (int w = 0; w < kCompactWaves; ++w) s += hist[w * E + e];
    store_agent(a.blk_base + (int64_t)blk * E + e, s);
  }
  if (threadIdx.x == 0) store_agent(reinterpret_cast<int32_t*>(a.blk_status) + blk, (int32_t)status);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    scalar[2] = __hip_atomic_fetch_add(a.arrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.blocks - 1;
  __syncthreads();
  if (!scalar[2]) return;
  // The last arrival: header, then the scan over workgroups.  P threads
  // share each expert (P = 256 / E for E <= 128, else 1), each over a
  // contiguous range of workgroups, loading 8 of them per round trip; their
  // partial sums get a per-expert prefix in LDS (with P = 1 the sum is the
  // expert's total).  The threads of expert 0 also OR the workgroups' status
  // bits.  LDS: the partial sums go to the ids area (E * P <= 256 ints, and
  // a.chunk >= 1020) and the status word to the histogram, both free by now.
  constexpr int kBatch = 8;
  const int P = E <= kCompactThreads / 2 ? kCompactThreads / E : 1;
  const int bp = (a.blocks + P - 1) / P;  // workgroups per part
  int* part = ids_lds;                    // [E * P] when P > 1
  uint32_t* status_or = reinterpret_cast<uint32_t*>(hist);
  if (threadIdx.x == 0) *status_or = 0u;
  __syncthreads();
  for (int idx = threadIdx.x; idx < E * P; idx += kCompactThreads) {
    const int e = idx / P, b_lo = (idx - e * P) * bp, b_hi = min(b_lo + bp, a.blocks);
    int sum = 0;
    uint32_t st = 0;
    for (int b0 = b_lo; b0 < b_hi; b0 += kBatch) {
      int c[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) c[j] = b0 + j < b_hi ? load_agent(a.blk_base + (int64_t)(b0 + j) * E + e) : 0;
      if (e == 0) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
          st |= b0 + j < b_hi ? (uint32_t)load_agent(reinterpret_cast<int32_t*>(a.blk_status) + b0 + j) : 0u;
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) sum += c[j];
    }
    if (P > 1)
      part[idx] = sum;
    else
      cnt[e] = sum;
    if (st) atomicOr(status_or, st);
  }
  __syncthreads();
  if (threadIdx.x < 64)
    a.hdr[threadIdx.x] = threadIdx.x == kHdrStatus ? *status_or : threadIdx.x == kHdrTokens ? (uint32_t)tokens : 0u;
  for (int e = threadIdx.x; P > 1 && e < E; e += kCompactThreads) {  // totals; part[] becomes exclusive
    int run = 0;
    for (int p = 0; p < P; ++p) {
      const int v = part[e * P + p];
      part[e * P + p] = run;
      run += v;
    }
    cnt[e] = run;
  }
  __syncthreads();
  finish_counts(a, cnt, tmp, scalar);
  __syncthreads();
  // each workgroup's first position per expert: the expert's offset plus the
  // counts of the workgroups before it
  for (int idx = threadIdx.x; idx < E * P; idx += kCompactThreads) {
    const int e = idx / P, b_lo = (idx - e * P) * bp, b_hi = min(b_lo + bp, a.blocks);
    int run = tmp[e] + (P > 1 ? part[idx] : 0);
    for (int b0 = b_lo; b0 < b_hi; b0 += kBatch) {
      int c[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) c[j] = b0 + j < b_hi ? load_agent(a.blk_base + (int64_t)(b0 + j) * E + e) : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (b0 + j < b_hi) a.blk_base[(int64_t)(b0 + j) * E + e] = run;
        run += c[j];
      }
    }
  }
  if (threadIdx.x == 0) store_agent(a.arrive, 0);  // as the arrivals do, at the device-coherent level
}

}  // namespace moe
