// Entry points of include/moe.h: handle lifecycle, staging, forward, status,
// regions and optional per-kernel event timing.
#include <hip/hip_runtime.h>
#include <string.h>

#include <new>
#include <vector>

#include "moe_internal.h"

namespace moe {
const char* last_error();
void clear_error();
}  // namespace moe

struct EventPair {
  hipEvent_t start, stop;
  int kind;
};

struct moe_layer {
  moe_config_t cfg;
  moe_weights_t w;
  moe::Tactic tac;
  moe::Layout L;
  uint8_t* ws;
  int32_t max_rows;
  int32_t expected_m;
  float capacity_factor;
  int32_t staged_tokens;
  bool compacted;  // the staging launch also scattered the routes (one compaction workgroup)
  void* out;
  int32_t grid_fc1, grid_fc2;
  int32_t stream_fc1, stream_fc2;  // register-ring depth of the streaming kernel per GEMM (0: LDS-ring kernel)
  int32_t grid_persist;  // MOE_FLAG_PERSISTENT_FFN: cooperative grid of the FC1->FC2 launch
  // profiling: event pairs around the launches of the classes in prof_mask
  uint32_t prof_mask;
  // Where the per-call regions (everything but the create-time weight tiles)
  // live: the workspace, or the static scratch during
  // moe_layer_forward_noalloc.
  uint8_t* cur_base;
  const moe::Layout* cur_L;
  int32_t cur_max_rows;
  std::vector<EventPair> pending;
  std::vector<hipEvent_t> pool;
  double ms[MOE_KERNEL_COUNT];
  int64_t launches[MOE_KERNEL_COUNT];
};

namespace {

bool is_weight_region(int r) {
  return r == MOE_REGION_W13T || r == MOE_REGION_W2T || r == MOE_REGION_W13S || r == MOE_REGION_W2S;
}

// A region of the call in progress: the create-time weight tiles are always
// the workspace's; the others come from the current per-call layout.
template <typename T>
T* region(moe_layer* l, int r) {
  if (is_weight_region(r)) return reinterpret_cast<T*>(l->ws + l->L.off[r]);
  return reinterpret_cast<T*>(l->cur_base + l->cur_L->off[r]);
}

hipEvent_t take_event(moe_layer* l) {
  if (!l->pool.empty()) {
    hipEvent_t e = l->pool.back();
    l->pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Records a start event if profiling; returns the pending index or -1.
int prof_begin(moe_layer* l, int kind, hipStream_t s) {
  if (!(l->prof_mask & (1u << kind))) return -1;
  EventPair p{take_event(l), take_event(l), kind};
  if (!p.start || !p.stop) return -1;
  (void)hipEventRecord(p.start, s);
  l->pending.push_back(p);
  return (int)l->pending.size() - 1;
}

void prof_end(moe_layer* l, int idx, hipStream_t s) {
  if (idx >= 0) (void)hipEventRecord(l->pending[idx].stop, s);
}

// Compaction arguments for the T tokens currently staged.
moe::CompactArgs compact_args(moe_layer* l, int32_t T) {
  moe::CompactArgs ca;
  const int32_t routes = T * l->cfg.top_k;
  ca.staged_idx = region<int32_t>(l, MOE_REGION_STAGED_IDX);
  ca.routes = routes;
  ca.num_experts = l->cfg.num_experts;
  ca.row_cap = (int32_t)l->cur_L->row_cap;
  ca.block_m = l->tac.block_m;
  ca.blocks = moe::compact_blocks_for(T, l->cfg.top_k);
  ca.chunk = moe::compact_chunk_routes(T, l->cfg.top_k);
  ca.hdr = region<uint32_t>(l, MOE_REGION_STATUS);
  // internal region: bases [compact_blocks, E], status [compact_blocks], arrival counter
  ca.blk_base = region<int32_t>(l, moe::kRegionBlkBase);
  ca.blk_status = reinterpret_cast<uint32_t*>(ca.blk_base + l->cur_L->compact_blocks * l->cfg.num_experts);
  ca.arrive = ca.blk_base + l->cur_L->compact_blocks * (l->cfg.num_experts + 1);
  ca.counts = region<int32_t>(l, MOE_REGION_COUNTS);
  ca.offsets = region<int32_t>(l, MOE_REGION_OFFSETS);
  ca.sorted_route = region<int32_t>(l, MOE_REGION_SORTED_ROUTE);
  ca.route_pos = region<int32_t>(l, MOE_REGION_ROUTE_POS);
  ca.tiles = region<int32_t>(l, MOE_REGION_TILES);
  ca.ready = (l->cfg.flags & MOE_FLAG_PERSISTENT_FFN) ? region<int32_t>(l, MOE_REGION_READY) : nullptr;
  return ca;
}

// Operands of the last-arriver combine fused into FC2 (MOE_FLAG_FUSED_COMBINE),
// or none.
moe::FusedCombineArgs fused_combine_args(moe_layer* l) {
  moe::FusedCombineArgs f;
  memset(&f, 0, sizeof(f));
  if (!(l->cfg.flags & MOE_FLAG_FUSED_COMBINE)) return f;
  f.out = static_cast<uint16_t*>(l->out);
  f.route_pos = region<int32_t>(l, MOE_REGION_ROUTE_POS);
  f.route_w = region<float>(l, MOE_REGION_STAGED_W);
  f.arrive = region<int32_t>(l, MOE_REGION_ARRIVE);
  return f;
}

moe_status_t hip_fail(const char* what) {
  hipError_t e = hipGetLastError();
  return moe::fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Weighted top-k combine of the FC2 rows into the bound output tensor.
moe_status_t combine(moe_layer* l, int32_t T, hipStream_t s, void* stream) {
  moe::CombineArgs cb;
  cb.y = region<uint16_t>(l, MOE_REGION_Y);
  cb.route_pos = region<int32_t>(l, MOE_REGION_ROUTE_POS);
  cb.staged_w = region<float>(l, MOE_REGION_STAGED_W);
  cb.tokens = T;
  cb.top_k = l->cfg.top_k;
  cb.hidden = l->cfg.hidden;
  cb.out = static_cast<uint16_t*>(l->out);
  const int p = prof_begin(l, MOE_KERNEL_COMBINE, s);
  if (moe::launch_combine(cb, stream) != 0) return hip_fail("combine launch");
  prof_end(l, p, s);
  return MOE_OK;
}

}  // namespace

extern "C" moe_status_t moe_layer_create(const moe_config_t* cfg, int32_t expected_m, int32_t max_rows,
                                         float capacity_factor, const moe_weights_t* w, void* workspace,
                                         size_t ws_bytes, void* stream, moe_layer_t** out) {
  moe::clear_error();
  moe_status_t s = moe::validate_config(cfg, expected_m, max_rows, capacity_factor);
  if (s != MOE_OK) return s;
  if (!out) return moe::fail(MOE_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!w || !w->w13 || !w->w13_scale || !w->w2 || !w->w2_scale)
    return moe::fail(MOE_ERR_INVALID_ARG, "weights or a weight pointer is NULL");
  if (((uintptr_t)w->w13 | (uintptr_t)w->w2) & 15)
    return moe::fail(MOE_ERR_INVALID_ARG, "weight codes must be 16-byte aligned");
  if (((uintptr_t)w->w13_scale | (uintptr_t)w->w2_scale) & 3)
    return moe::fail(MOE_ERR_INVALID_ARG, "weight scales must be 4-byte aligned");
  if (!workspace || ((uintptr_t)workspace & 255))
    return moe::fail(MOE_ERR_INVALID_ARG, "workspace must be non-NULL and 256-byte aligned");
  moe::Tactic t = moe::choose_tactic(*cfg, expected_m);
  moe::Layout L = moe::compute_layout(*cfg, t, max_rows, capacity_factor);
  s = moe::validate_layout(*cfg, L);
  if (s != MOE_OK) return s;
  if (ws_bytes < L.total)
    return moe::fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < required %zu", ws_bytes, L.total);

  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hip_fail("hipGetDevice");
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hip_fail("hipDeviceGetAttribute");
  moe_layer* l = new (std::nothrow) moe_layer();
  if (!l) return moe::fail(MOE_ERR_INVALID_ARG, "out of host memory");
  l->cfg = *cfg;
  l->w = *w;
  l->tac = t;
  l->L = L;
  l->ws = static_cast<uint8_t*>(workspace);
  l->max_rows = max_rows;
  l->expected_m = expected_m;
  l->capacity_factor = capacity_factor;
  l->staged_tokens = -1;
  l->compacted = false;
  l->out = nullptr;
  const bool mx = moe::is_mx(cfg->weight_format);
  // the streaming kernel serves the plain two-launch FP8 path (the variants
  // with a gate/up output, the fused combine or one persistent launch run the
  // LDS-ring kernel): FC2 by default, FC1 on request
  const bool stream_ok = !mx && !(cfg->flags & (MOE_FLAG_UNFUSED_FC1 | MOE_FLAG_FUSED_COMBINE |
                                                MOE_FLAG_PERSISTENT_FFN | MOE_FLAG_NO_STREAM));
  l->stream_fc1 = stream_ok && (cfg->flags & MOE_FLAG_STREAM_FC1)
                      ? moe::gemm_stream_depth(t.block_m, cfg->hidden / 128, cfg->intermediate / 128)
                      : 0;
  l->stream_fc2 = stream_ok ? moe::gemm_stream_depth(t.block_m, cfg->intermediate / 128, (cfg->hidden + 255) / 256) : 0;
  auto grid = [&](int which) {
    int g = cus * (mx ? moe::gemm_mx_max_workgroups_per_cu(which, t.block_m)
                      : moe::gemm_max_workgroups_per_cu(which, t.block_m, which == 1 ? l->stream_fc1 : l->stream_fc2));
    g = (g / 8) * 8;
    return g < 8 ? 8 : g;
  };
  l->grid_fc1 = grid(1);
  l->grid_fc2 = grid(2);
  l->grid_persist = 0;
  if (cfg->flags & MOE_FLAG_PERSISTENT_FFN) {
    // every workgroup must be resident at once (cooperative launch)
    const int g = (cus * moe::gemm_persist_max_workgroups_per_cu(t.block_m) / 8) * 8;
    l->grid_persist = g < 8 ? 8 : g;
  }
  // weight codes -> kernel tile order, stream-ordered before any forward
  uint8_t* w13t = l->ws + L.off[MOE_REGION_W13T];
  uint8_t* w2t = l->ws + L.off[MOE_REGION_W2T];
  const int E = cfg->num_experts, H = cfg->hidden, I = cfg->intermediate;
  const int order = mx ? moe::kTileOrderMx : moe::kTileOrder16;
  bool ok = moe::launch_tile_weights(static_cast<const uint8_t*>(w->w13), w13t, E, 2 * I, H, I / 128, I, true, order,
                                     stream) == 0 &&
            moe::launch_tile_weights(static_cast<const uint8_t*>(w->w2), w2t, E, H, I, (H + 255) / 256, I, false,
                                     order, stream) == 0;
  if (ok && mx)
    ok = moe::launch_tile_mx_scales(static_cast<const uint8_t*>(w->w13_scale),
                                    reinterpret_cast<uint32_t*>(l->ws + L.off[MOE_REGION_W13S]), E, 2 * I, H, I / 128,
                                    I, true, stream) == 0 &&
         moe::launch_tile_mx_scales(static_cast<const uint8_t*>(w->w2_scale),
                                    reinterpret_cast<uint32_t*>(l->ws + L.off[MOE_REGION_W2S]), E, H, I,
                                    (H + 255) / 256, I, false, stream) == 0;
  // the compaction's arrival counter starts at zero (each staging leaves it so)
  if (ok)
    ok = moe::launch_fill_zero(reinterpret_cast<uint32_t*>(l->ws + L.off[moe::kRegionBlkBase]),
                               (int64_t)(L.size[moe::kRegionBlkBase] / 4), stream) == 0;
  // arrival counters of the fused combine start at zero (each forward leaves them so)
  if (ok && (cfg->flags & MOE_FLAG_FUSED_COMBINE))
    ok = moe::launch_fill_zero(reinterpret_cast<uint32_t*>(l->ws + L.off[MOE_REGION_ARRIVE]),
                               (int64_t)(L.size[MOE_REGION_ARRIVE] / 4), stream) == 0;
  if (!ok) {
    delete l;
    return hip_fail("weight transform launch");
  }
  l->prof_mask = 0;
  l->cur_base = l->ws;
  l->cur_L = &l->L;
  l->cur_max_rows = max_rows;
  memset(l->ms, 0, sizeof(l->ms));
  memset(l->launches, 0, sizeof(l->launches));
  *out = l;
  return MOE_OK;
}

namespace {

moe_status_t stage_impl(moe_layer_t* l, const void* x, const float* x_scale, const int32_t* topk_idx,
                        const float* topk_w, int32_t num_tokens, void* out_bf16, void* stream) {
  if (!l) return moe::fail(MOE_ERR_INVALID_ARG, "layer is NULL");
  if (num_tokens < 0) return moe::fail(MOE_ERR_INVALID_ARG, "num_tokens %d < 0", num_tokens);
  if (num_tokens > l->max_rows)
    return moe::fail(MOE_ERR_CAPACITY, "num_tokens %d exceeds max_rows %d", num_tokens, l->max_rows);
  if (num_tokens > 0) {
    if (!x || !topk_idx || !topk_w || !out_bf16)
      return moe::fail(MOE_ERR_INVALID_ARG, "x, topk_idx, topk_w and out must be non-NULL");
    if (((uintptr_t)x | (uintptr_t)out_bf16) & 15)
      return moe::fail(MOE_ERR_INVALID_ARG, "x and out must be 16-byte aligned");
    if (((uintptr_t)topk_idx | (uintptr_t)topk_w | (uintptr_t)x_scale) & 3)
      return moe::fail(MOE_ERR_INVALID_ARG, "topk_idx, topk_w and x_scale must be 4-byte aligned");
  }
  if (x_scale && l->cfg.act_format != MOE_ACT_E4M3_1X128)
    return moe::fail(MOE_ERR_INVALID_ARG, "x_scale is only meaningful for E4M3_1X128 activations");
  hipStream_t s = static_cast<hipStream_t>(stream);
  moe::StageArgs a;
  a.x = x;
  a.x_scale = x_scale;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.tokens = num_tokens;
  a.max_rows = l->cur_max_rows;
  a.hidden = l->cfg.hidden;
  a.top_k = l->cfg.top_k;
  a.num_experts = l->cfg.num_experts;
  a.flags = l->cfg.flags;
  a.act_format = l->cfg.act_format;
  a.hdr = region<uint32_t>(l, MOE_REGION_STATUS);
  a.staged_idx = region<int32_t>(l, MOE_REGION_STAGED_IDX);
  a.staged_w = region<float>(l, MOE_REGION_STAGED_W);
  a.xq = region<uint8_t>(l, MOE_REGION_XQ);
  a.xs = region<float>(l, MOE_REGION_XS);
  a.x_plane = (int64_t)l->cur_L->rows_x * l->cfg.hidden;
  a.xs_mx = region<uint32_t>(l, MOE_REGION_XS);
  // One launch stages and compacts; a compaction over several workgroups
  // leaves its scatter to the forward.
  const moe::CompactArgs ca = compact_args(l, num_tokens);
  const int p = prof_begin(l, MOE_KERNEL_STAGE, s);
  if (moe::launch_stage(a, ca, stream) != 0) return hip_fail("stage launch");
  prof_end(l, p, s);
  l->compacted = ca.blocks == 1;
  l->staged_tokens = num_tokens;
  l->out = out_bf16;
  return MOE_OK;
}

moe_status_t forward_impl(moe_layer_t* l, void* stream) {
  if (!l) return moe::fail(MOE_ERR_INVALID_ARG, "layer is NULL");
  if (l->staged_tokens < 0) return moe::fail(MOE_ERR_STATE, "moe_stage_inputs has not been called");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const moe_config_t& c = l->cfg;
  const int32_t T = l->staged_tokens;

  const moe::CompactArgs ca = compact_args(l, T);
  int p = -1;
  if (!l->compacted) {
    p = prof_begin(l, MOE_KERNEL_COMPACT, s);
    if (moe::launch_compact_scatter(ca, stream) != 0) return hip_fail("compact launch");
    prof_end(l, p, s);
  }

  if (moe::is_mx(c.weight_format)) {
    moe::MxGemmArgs m1;
    memset(&m1, 0, sizeof(m1));
    m1.a = region<uint8_t>(l, MOE_REGION_XQ);
    m1.a_plane = (int64_t)l->cur_L->rows_x * c.hidden;
    m1.a_scale = region<uint32_t>(l, MOE_REGION_XS);
    m1.a_mode = 1;
    m1.sorted_route = ca.sorted_route;
    m1.top_k = c.top_k;
    m1.w = region<uint8_t>(l, MOE_REGION_W13T);
    m1.w_scale = region<uint32_t>(l, MOE_REGION_W13S);
    m1.n_rows = 2 * c.intermediate;
    m1.k_dim = c.hidden;
    m1.inter = c.intermediate;
    m1.n_tiles = c.intermediate / 128;
    m1.tiles = ca.tiles;
    m1.offsets = ca.offsets;
    m1.hdr = ca.hdr;
    m1.hq = region<uint8_t>(l, MOE_REGION_HQ);
    m1.h_plane = l->cur_L->row_cap * c.intermediate;
    m1.hs = region<uint32_t>(l, MOE_REGION_HS);
    m1.grid = l->grid_fc1;
    m1.w_e5m2 = c.weight_format == MOE_WEIGHT_MXFP8_E5M2;
    p = prof_begin(l, MOE_KERNEL_FC1, s);
    if (moe::launch_fc1_mx(m1, l->tac.block_m, stream) != 0) return hip_fail("fc1 launch");
    prof_end(l, p, s);

    moe::MxGemmArgs m2;
    memset(&m2, 0, sizeof(m2));
    m2.a = m1.hq;
    m2.a_plane = m1.h_plane;
    m2.a_scale = m1.hs;
    m2.a_mode = 0;
    m2.sorted_route = ca.sorted_route;
    m2.top_k = c.top_k;
    m2.w = region<uint8_t>(l, MOE_REGION_W2T);
    m2.w_scale = region<uint32_t>(l, MOE_REGION_W2S);
    m2.n_rows = c.hidden;
    m2.k_dim = c.intermediate;
    m2.inter = c.intermediate;
    m2.n_tiles = (c.hidden + 255) / 256;
    m2.tiles = ca.tiles;
    m2.offsets = ca.offsets;
    m2.hdr = ca.hdr;
    m2.y = region<uint16_t>(l, MOE_REGION_Y);
    m2.grid = l->grid_fc2;
    m2.w_e5m2 = m1.w_e5m2;
    m2.fc = fused_combine_args(l);
    p = prof_begin(l, MOE_KERNEL_FC2, s);
    if (moe::launch_fc2_mx(m2, l->tac.block_m, stream) != 0) return hip_fail("fc2 launch");
    prof_end(l, p, s);
    return m2.fc.out ? MOE_OK : combine(l, T, s, stream);
  }

  moe::GemmArgs g1;
  memset(&g1, 0, sizeof(g1));
  g1.a = region<uint8_t>(l, MOE_REGION_XQ);
  g1.a_scale = region<float>(l, MOE_REGION_XS);
  g1.a_mode = (c.flags & MOE_FLAG_PER_ROUTE_STAGING) ? 2 : 1;
  g1.sorted_route = ca.sorted_route;
  g1.top_k = c.top_k;
  g1.w = region<uint8_t>(l, MOE_REGION_W13T);
  g1.w_scale = static_cast<const float*>(l->w.w13_scale);
  g1.n_rows = 2 * c.intermediate;
  g1.k_dim = c.hidden;
  g1.inter = c.intermediate;
  g1.n_tiles = c.intermediate / 128;
  g1.tiles = ca.tiles;
  g1.offsets = ca.offsets;
  g1.hdr = ca.hdr;
  g1.hq = region<uint8_t>(l, MOE_REGION_HQ);
  g1.hs = region<float>(l, MOE_REGION_HS);
  g1.grid = l->grid_fc1;
  g1.stream_depth = l->stream_fc1;
  const bool unfused = (c.flags & MOE_FLAG_UNFUSED_FC1) != 0;
  g1.gateup = unfused ? region<float>(l, MOE_REGION_GATEUP) : nullptr;
  g1.gateup_bf16 = (c.flags & MOE_FLAG_BF16_GATEUP) != 0;
  const bool persistent = (c.flags & MOE_FLAG_PERSISTENT_FFN) != 0;
  if (!persistent) {
    p = prof_begin(l, MOE_KERNEL_FC1, s);
    if (moe::launch_fc1(g1, l->tac.block_m, stream) != 0) return hip_fail("fc1 launch");
    if (unfused && moe::launch_swiglu_quant(g1.gateup, g1.gateup_bf16 != 0, (int32_t)l->cur_L->row_cap,
                                            c.intermediate, g1.hdr, g1.hq, g1.hs, stream) != 0)
      return hip_fail("swiglu launch");
    prof_end(l, p, s);
  }

  moe::GemmArgs g2;
  memset(&g2, 0, sizeof(g2));
  g2.a = g1.hq;
  g2.a_scale = g1.hs;
  g2.a_mode = 0;
  g2.sorted_route = ca.sorted_route;
  g2.top_k = c.top_k;
  g2.w = region<uint8_t>(l, MOE_REGION_W2T);
  g2.w_scale = static_cast<const float*>(l->w.w2_scale);
  g2.n_rows = c.hidden;
  g2.k_dim = c.intermediate;
  g2.inter = c.intermediate;
  g2.n_tiles = (c.hidden + 255) / 256;
  g2.tiles = ca.tiles;
  g2.offsets = ca.offsets;
  g2.hdr = ca.hdr;
  g2.y = region<uint16_t>(l, MOE_REGION_Y);
  g2.grid = l->grid_fc2;
  g2.stream_depth = l->stream_fc2;
  g2.fc = fused_combine_args(l);
  if (persistent) {
    // FC1 and FC2 in one launch, timed as the FC1 class (FC2 has no launch)
    moe::PersistArgs q;
    q.ready = region<int32_t>(l, MOE_REGION_READY);
    q.need = c.intermediate / 128;
    q.status = region<uint32_t>(l, MOE_REGION_STATUS) + moe::kHdrStatus;
    g1.grid = g2.grid = l->grid_persist;
    p = prof_begin(l, MOE_KERNEL_FC1, s);
    if (moe::launch_fc1_fc2(g1, g2, q, l->tac.block_m, l->grid_persist, stream) != 0)
      return hip_fail("persistent fc1+fc2 launch");
    prof_end(l, p, s);
    return g2.fc.out ? MOE_OK : combine(l, T, s, stream);
  }
  p = prof_begin(l, MOE_KERNEL_FC2, s);
  if (moe::launch_fc2(g2, l->tac.block_m, stream) != 0) return hip_fail("fc2 launch");
  prof_end(l, p, s);

  return g2.fc.out ? MOE_OK : combine(l, T, s, stream);
}

}  // namespace

extern "C" moe_status_t moe_stage_inputs(moe_layer_t* l, const void* x, const float* x_scale,
                                         const int32_t* topk_idx, const float* topk_w, int32_t num_tokens,
                                         void* out_bf16, void* stream) {
  moe::clear_error();
  return stage_impl(l, x, x_scale, topk_idx, topk_w, num_tokens, out_bf16, stream);
}

extern "C" moe_status_t moe_layer_forward(moe_layer_t* l, void* stream) {
  moe::clear_error();
  return forward_impl(l, stream);
}

// Stage + forward with every per-call region in the library's static device
// scratch (moe_noalloc.hip) instead of the workspace: no device memory is
// allocated, and the handle's own staged batch is left as it was.
extern "C" moe_status_t moe_layer_forward_noalloc(moe_layer_t* l, const void* x, const float* x_scale,
                                                  const int32_t* topk_idx, const float* topk_w,
                                                  int32_t num_tokens, void* out_bf16, uint32_t* status_bits,
                                                  void* stream) {
  moe::clear_error();
  if (!l) return moe::fail(MOE_ERR_INVALID_ARG, "layer is NULL");
  if (num_tokens < 0) return moe::fail(MOE_ERR_INVALID_ARG, "num_tokens %d < 0", num_tokens);
  if (num_tokens > l->max_rows)
    return moe::fail(MOE_ERR_CAPACITY, "num_tokens %d exceeds max_rows %d", num_tokens, l->max_rows);
  if ((uintptr_t)status_bits & 3) return moe::fail(MOE_ERR_INVALID_ARG, "status_bits must be 4-byte aligned");
  uint8_t* base = nullptr;
  size_t cap = 0;
  if (moe::noalloc_scratch(&base, &cap) != 0) return hip_fail("device scratch address");
  // rows as in the call; route rows held as the layer holds them (never
  // more than the call's routes), so routes drop exactly as they would in
  // the workspace
  const moe::Layout S = moe::compute_scratch_layout(l->cfg, l->tac, num_tokens, l->L.row_cap);
  if (S.total > cap)
    return moe::fail(MOE_ERR_CAPACITY,
                     "num_tokens %d needs %zu bytes of per-call regions; the no-allocation forward holds %zu",
                     num_tokens, S.total, cap);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The scratch keeps the last call's contents (of any layer on this
  // device): what must start at zero is cleared by a fill kernel.
  if (moe::launch_fill_zero(reinterpret_cast<uint32_t*>(base + S.off[moe::kRegionBlkBase]),
                            (int64_t)(S.size[moe::kRegionBlkBase] / 4), stream) != 0)
    return hip_fail("scratch clear");
  if ((l->cfg.flags & MOE_FLAG_FUSED_COMBINE) &&
      moe::launch_fill_zero(reinterpret_cast<uint32_t*>(base + S.off[MOE_REGION_ARRIVE]),
                            (int64_t)(S.size[MOE_REGION_ARRIVE] / 4), stream) != 0)
    return hip_fail("scratch clear");
  // run on the scratch, then put the handle back as it was
  const int32_t staged = l->staged_tokens;
  const bool compacted = l->compacted;
  void* out = l->out;
  const uint32_t prof = l->prof_mask;
  l->cur_base = base;
  l->cur_L = &S;
  l->cur_max_rows = num_tokens > 0 ? num_tokens : 1;
  l->prof_mask = 0;  // event records would create events
  moe_status_t st = stage_impl(l, x, x_scale, topk_idx, topk_w, num_tokens, out_bf16, stream);
  if (st == MOE_OK) st = forward_impl(l, stream);
  if (st == MOE_OK && status_bits &&
      hipMemcpyAsync(status_bits, base + S.off[MOE_REGION_STATUS] + 4 * moe::kHdrStatus, 4,
                     hipMemcpyDeviceToDevice, s) != hipSuccess)
    st = hip_fail("status copy");
  l->cur_base = l->ws;
  l->cur_L = &l->L;
  l->cur_max_rows = l->max_rows;
  l->prof_mask = prof;
  l->staged_tokens = staged;
  l->compacted = compacted;
  l->out = out;
  return st;
}

extern "C" moe_status_t moe_read_status(moe_layer_t* l, void* stream, uint32_t* bits) {
  moe::clear_error();
  if (!l || !bits) return moe::fail(MOE_ERR_INVALID_ARG, "layer and bits must be non-NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  if (hipMemcpyAsync(&v, region<uint32_t>(l, MOE_REGION_STATUS), sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess)
    return hip_fail("hipMemcpyAsync");
  if (hipStreamSynchronize(s) != hipSuccess) return hip_fail("hipStreamSynchronize");
  *bits = v;
  return MOE_OK;
}

extern "C" moe_status_t moe_layer_region(moe_layer_t* l, int32_t r, void** dptr, size_t* bytes) {
  moe::clear_error();
  if (!l || !dptr || !bytes) return moe::fail(MOE_ERR_INVALID_ARG, "NULL argument");
  if (r < 0 || r > MOE_REGION_READY) return moe::fail(MOE_ERR_INVALID_ARG, "unknown region %d", r);
  *dptr = l->ws + l->L.off[r];
  *bytes = l->L.size[r];
  return MOE_OK;
}

extern "C" moe_status_t moe_layer_tactic(const moe_layer_t* l, moe_tactic_t* t) {
  moe::clear_error();
  if (!l || !t) return moe::fail(MOE_ERR_INVALID_ARG, "NULL argument");
  t->token_bucket = l->tac.bucket;
  t->block_m = l->tac.block_m;
  t->block_n = l->tac.block_n;
  t->grid_fc1 = l->grid_fc1;
  t->grid_fc2 = l->grid_fc2;
  t->row_cap = (int32_t)l->L.row_cap;
  t->max_m_tiles = (int32_t)l->L.max_m_tiles;
  t->tile_order = moe::is_mx(l->cfg.weight_format) ? moe::kTileOrderMx : moe::kTileOrder16;
  t->stream_depth_fc1 = l->stream_fc1;
  t->stream_depth_fc2 = l->stream_fc2;
  return MOE_OK;
}

extern "C" moe_status_t moe_profile_enable(moe_layer_t* l, uint32_t kernel_mask) {
  moe::clear_error();
  if (!l) return moe::fail(MOE_ERR_INVALID_ARG, "layer is NULL");
  if (kernel_mask & ~MOE_PROFILE_ALL) return moe::fail(MOE_ERR_INVALID_ARG, "unknown kernel classes 0x%x", kernel_mask);
  l->prof_mask = kernel_mask;
  memset(l->ms, 0, sizeof(l->ms));
  memset(l->launches, 0, sizeof(l->launches));
  return MOE_OK;
}

extern "C" moe_status_t moe_profile_read(moe_layer_t* l, double* ms_total, int64_t* launches) {
  moe::clear_error();
  if (!l || !ms_total || !launches) return moe::fail(MOE_ERR_INVALID_ARG, "NULL argument");
  for (EventPair& p : l->pending) {
    if (hipEventSynchronize(p.stop) != hipSuccess) return hip_fail("hipEventSynchronize");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess) return hip_fail("hipEventElapsedTime");
    l->ms[p.kind] += ms;
    l->launches[p.kind] += 1;
    l->pool.push_back(p.start);
    l->pool.push_back(p.stop);
  }
  l->pending.clear();
  for (int k = 0; k < MOE_KERNEL_COUNT; ++k) {
    ms_total[k] = l->ms[k];
    launches[k] = l->launches[k];
  }
  return MOE_OK;
}

extern "C" moe_status_t moe_layer_destroy(moe_layer_t* l) {
  moe::clear_error();
  if (!l) return MOE_OK;
  for (EventPair& p : l->pending) {
    (void)hipEventSynchronize(p.stop);
    (void)hipEventDestroy(p.start);
    (void)hipEventDestroy(p.stop);
  }
  for (hipEvent_t e : l->pool) (void)hipEventDestroy(e);
  delete l;
  return MOE_OK;
}
