// Forward preparation: activation quantisation to e4m3 with 1x128 scales and
// route staging with the routing checker, after "perf(moe_ep): fuse Rubin
// MegaMoE forward preparation" (flashinfer PR #6398: fused input quantisation
// + route staging; checker for expert-id bounds, duplicate routes and finite
// scores; masked slots may carry NaN/inf and are staged as zero without
// touching the caller's tensors).
#include <hip/hip_runtime.h>

#include "moe_compact_dev.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// One 8-lane group per 1x128 block; each lane owns 16 consecutive columns.
//   s = amax / 448 (IEEE float division), q = RNE_sat(x / s), s == 0 -> q = 0
// (the codes of the IEEE quotient x / s; see below for how it is formed).
// With a prequantised input (x_scale != null) codes and scales are copied.
constexpr int kQuantLanes = 8;  // lanes per 1x128 block
__device__ inline void quant_1x128(const StageArgs& a, int64_t g, int64_t groups, int copies) {
  const int64_t grp = g / kQuantLanes;
  if (grp >= groups) return;
  const int ql = threadIdx.x & (kQuantLanes - 1);
  const int kbs = a.hidden >> 7;
  const int64_t row = grp / kbs;
  const int kb = (int)(grp - row * kbs);
  const int64_t col = (int64_t)kb * 128 + ql * 16;
  uint4 codes;
  float s;
  if (a.x_scale == nullptr) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + row * a.hidden + col);
    const uint4 r0 = src[0], r1 = src[1];
    const uint32_t words[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    float v[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = bf16_to_f32(words[i] & 0xffffu);
      v[2 * i + 1] = bf16_to_f32(words[i] >> 16);
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
    m = group_max<kQuantLanes>(m);
    s = m / kE4m3Max;
    if (s == 0.0f) {
      codes = make_uint4(0u, 0u, 0u, 0u);
    } else {
      // x / s without an IEEE division per element: inv = fl32(1/s) once,
      // then q0 = fl32(x * inv), r = fma(-q0, s, x) and q = fma(r, inv, q0)
      // (a reciprocal with one correction step), given the sign of x (the
      // sums give +0 for x = -0, whose quotient is -0, code 0x80).  For every
      // bf16 x with |x| <= amax and every block with s >= 2^-90 this gives
      // the e4m3 code of the IEEE quotient, checked exhaustively; below that
      // (amax under ~3.6e-25) the remainder can underflow, so such blocks
      // divide.
      float q[16];
      if (s >= 0x1p-90f) {
        const float inv = 1.0f / s;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float q0 = v[i] * inv;
          q[i] = copysignf(fmaf(fmaf(-q0, s, v[i]), inv, q0), v[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = v[i] / s;
      }
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int c = cvt2_e4m3(q[4 * j], q[4 * j + 1], 0, false);
        w[j] = (uint32_t)cvt2_e4m3(q[4 * j + 2], q[4 * j + 3], c, true);
      }
      codes = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
    codes = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.x) + row * a.hidden + col);
    s = a.x_scale[row * kbs + kb];
  }
  for (int c = 0; c < copies; ++c) {
    const int64_t dst = row * copies + c;
    *reinterpret_cast<uint4*>(a.xq + dst * a.hidden + col) = codes;
    if (ql == 0) a.xs[dst * kbs + kb] = s;
  }
}

// MXFP8 variant: BF16 rows are kept (not quantised) as the sum of two e4m3
// terms, each with its own E8M0 exponent per 32 columns, so the scaled MFMA
// can consume them: hi = e4m3(x / 2^e_hi), lo = e4m3((x - hi * 2^e_hi) / 2^e_lo).
// Four lanes per 32-column block, eight columns each.  Writes the hi codes
// to plane 0, the lo codes to plane 1 (x_plane bytes further) and one word
// (e_hi + 127) | (e_lo + 127) << 8 per block.
__device__ inline void split_mx(const StageArgs& a, int64_t g, int64_t groups) {
  const int64_t grp = g >> 2;
  if (grp >= groups) return;
  const int q = a.hidden >> 5;
  const int64_t row = grp / q;
  const int blk = (int)(grp - row * q);
  const int64_t col = (int64_t)blk * 32 + (threadIdx.x & 3) * 8;
  const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + row * a.hidden + col);
  float v[8];
  v[0] = bf16_to_f32(raw.x & 0xffffu); v[1] = bf16_to_f32(raw.x >> 16);
  v[2] = bf16_to_f32(raw.y & 0xffffu); v[3] = bf16_to_f32(raw.y >> 16);
  v[4] = bf16_to_f32(raw.z & 0xffffu); v[5] = bf16_to_f32(raw.z >> 16);
  v[6] = bf16_to_f32(raw.w & 0xffffu); v[7] = bf16_to_f32(raw.w >> 16);
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  const int e_hi = mx_block_exp(group_max<4>(m));
  float r[8];
  const uint32_t h0 = mx_term4(v, e_hi, r), h1 = mx_term4(v + 4, e_hi, r + 4);
  float mr = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) mr = fmaxf(mr, fabsf(r[i]));
  const int e_lo = mx_block_exp(group_max<4>(mr));
  float unused[8];
  const uint32_t l0 = mx_term4(r, e_lo, unused), l1 = mx_term4(r + 4, e_lo, unused + 4);
  uint8_t* dst = a.xq + row * a.hidden + col;
  *reinterpret_cast<uint2*>(dst) = make_uint2(h0, h1);
  *reinterpret_cast<uint2*>(dst + a.x_plane) = make_uint2(l0, l1);
  if ((threadIdx.x & 3) == 0) a.xs_mx[row * q + blk] = (uint32_t)(e_hi + 127) | ((uint32_t)(e_lo + 127) << 8);
}

// One thread per token slot row in [0, max_rows).  Live rows are checked and
// masked; rows past the live count are staged as masked.  ids_lds (live rows
// only, from token t0 on): a copy of the staged expert ids for the
// compaction of the same workgroup.  Status bits go to the workgroup's LDS
// word `status`.
__device__ inline void stage_route_row(const StageArgs& a, int t, int* ids_lds, int t0, uint32_t* status) {
  const int K = a.top_k;
  uint32_t bits = 0;
  int ids[8];
  float ws[8];
  bool act[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    ids[k] = -1;
    ws[k] = 0.0f;
    act[k] = false;
  }
  if (t < a.tokens) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {  // all loads first
      if (k < K) {
        ids[k] = a.topk_idx[(int64_t)t * K + k];
        ws[k] = a.topk_w[(int64_t)t * K + k];
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k >= K) continue;
      const int e = ids[k];
      if (e == -1) continue;
      if (e < -1 || e >= a.num_experts) {
        bits |= MOE_DEV_BAD_EXPERT;
        continue;
      }
      act[k] = true;
    }
    if (a.flags & MOE_FLAG_CHECK_ROUTES) {
#pragma unroll
      for (int k = 1; k < 8; ++k) {
        if (k >= K || !act[k]) continue;
#pragma unroll
        for (int j = 0; j < k; ++j) {
          if (act[j] && ids[j] == ids[k]) {  // the lowest slot of an id stays active
            act[k] = false;
            bits |= MOE_DEV_DUPLICATE;
            break;
          }
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (act[k] && !isfinite(ws[k])) {
          act[k] = false;
          bits |= MOE_DEV_NONFINITE;
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < K) {
      a.staged_idx[(int64_t)t * K + k] = act[k] ? ids[k] : -1;
      a.staged_w[(int64_t)t * K + k] = act[k] ? ws[k] : 0.0f;
      if (ids_lds && t < a.tokens) ids_lds[(t - t0) * K + k] = act[k] ? ids[k] : -1;
    }
  }
  if (bits) atomicOr(status, bits);
}

// The staging launch.  Workgroups [0, c.blocks) take the route rows, one
// chunk of whole tokens each, and compact them: the whole compaction when
// c.blocks == 1, else the counting (compact_scatter_kernel finishes in the
// next launch).  They come first so that they run beside the quantisation
// workgroups [c.blocks, ...), which are most of the grid.  The header is
// written by the compaction (after every status bit of the launch is known);
// nothing else in the launch touches it.
__global__ __launch_bounds__(256) void stage_kernel(StageArgs a, CompactArgs c, int64_t groups, int copies) {
  extern __shared__ int lds[];
  if ((int)blockIdx.x >= c.blocks) {
    const int64_t g = (int64_t)(blockIdx.x - c.blocks) * 256 + threadIdx.x;
    if (a.act_format == MOE_ACT_BF16)
      split_mx(a, g, groups);
    else
      quant_1x128(a, g, groups, copies);
    return;
  }
  const int blk = blockIdx.x;
  int* ids_lds = lds + compact_one_workgroup_lds(c.num_experts) / 4;  // [c.chunk]
  uint32_t* status = reinterpret_cast<uint32_t*>(ids_lds + c.chunk);
  if (threadIdx.x == 0) *status = 0u;
  __syncthreads();
  const int tc = c.chunk / a.top_k;
  const int t0 = blk * tc, t1 = min(t0 + tc, a.tokens);
  for (int t = t0 + (int)threadIdx.x; t < t1; t += 256) stage_route_row(a, t, ids_lds, t0, status);
  for (int t = a.tokens + blk * 256 + (int)threadIdx.x; t < a.max_rows; t += c.blocks * 256)
    stage_route_row(a, t, nullptr, 0, status);  // rows past the live count
  __syncthreads();
  if (c.blocks == 1) {
    if (threadIdx.x < 64)
      a.hdr[threadIdx.x] = threadIdx.x == kHdrTokens ? (uint32_t)a.tokens : threadIdx.x == kHdrStatus ? *status : 0u;
    __syncthreads();
    compact_one_workgroup(c, lds, ids_lds);
  } else {
    count_and_arrive(c, blk, lds, ids_lds, *status, a.tokens);
  }
}

static void quant_grid(const StageArgs& a, int64_t* groups, int* blocks, int* copies) {
  if (a.act_format == MOE_ACT_BF16) {
    *groups = (int64_t)a.tokens * (a.hidden / 32);
    *blocks = (int)((*groups * 4 + 255) / 256);
  } else {
    *groups = (int64_t)a.tokens * (a.hidden / 128);
    *blocks = (int)((*groups * kQuantLanes + 255) / 256);
  }
  *copies = (a.flags & MOE_FLAG_PER_ROUTE_STAGING) ? a.top_k : 1;
}

int launch_stage(const StageArgs& a, const CompactArgs& c, void* stream) {
  int64_t groups;
  int qblocks, copies;
  quant_grid(a, &groups, &qblocks, &copies);
  const size_t lds = compact_one_workgroup_lds(c.num_experts) + (size_t)c.chunk * 4 + 4;
  hipLaunchKernelGGL(stage_kernel, dim3(c.blocks + qblocks), dim3(256), lds, static_cast<hipStream_t>(stream), a, c,
                     groups, copies);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
