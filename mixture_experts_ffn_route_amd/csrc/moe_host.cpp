// Host-side logic with no HIP dependency: argument validation, the token
// bucket and tile tactic table, and the workspace layout.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "moe_internal.h"

namespace moe {

static thread_local char g_last_error[512];

moe_status_t fail(moe_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

const char* last_error() { return g_last_error; }
void clear_error() { g_last_error[0] = 0; }

// Clamped ceil power of two in [8, 32768]: the token bucket of the SM90
// pull-style MegaMoE heuristics (flashinfer PR #4688, heuristic-config test).
int32_t token_bucket(int32_t tokens) {
  if (tokens <= 0) return -1;
  if (tokens >= 32768) return 32768;
  int32_t b = 8;
  while (b < tokens) b <<= 1;
  return b;
}

static bool valid_top_k(int k) { return k == 1 || k == 2 || k == 4 || k == 6 || k == 8; }

moe_status_t validate_config(const moe_config_t* cfg, int32_t expected_m, int32_t max_rows,
                             float capacity_factor) {
  if (!cfg) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  if (cfg->hidden <= 0 || cfg->intermediate <= 0)
    return fail(MOE_ERR_INVALID_ARG, "hidden (%d) and intermediate (%d) must be positive", cfg->hidden,
                cfg->intermediate);
  if (cfg->hidden % 128 || cfg->intermediate % 128)
    return fail(MOE_ERR_UNSUPPORTED, "hidden (%d) and intermediate (%d) must be multiples of 128",
                cfg->hidden, cfg->intermediate);
  if (cfg->hidden > 16384 || cfg->intermediate > 16384)
    return fail(MOE_ERR_UNSUPPORTED, "hidden/intermediate above 16384 are not supported");
  if (cfg->num_experts < 1 || cfg->num_experts > kMaxExperts)
    return fail(MOE_ERR_UNSUPPORTED, "num_experts %d outside [1, %d]", cfg->num_experts, kMaxExperts);
  if (!valid_top_k(cfg->top_k))
    return fail(MOE_ERR_UNSUPPORTED, "top_k %d not in {1, 2, 4, 6, 8}", cfg->top_k);
  if (cfg->top_k > cfg->num_experts)
    return fail(MOE_ERR_INVALID_ARG, "top_k %d exceeds num_experts %d", cfg->top_k, cfg->num_experts);
  if (cfg->flags & ~(uint32_t)(MOE_FLAG_CHECK_ROUTES | MOE_FLAG_PER_ROUTE_STAGING | MOE_FLAG_UNFUSED_FC1 |
                               MOE_FLAG_FUSED_COMBINE | MOE_FLAG_PERSISTENT_FFN | MOE_FLAG_BF16_GATEUP |
                               MOE_FLAG_NO_STREAM | MOE_FLAG_STREAM_FC1))
    return fail(MOE_ERR_INVALID_ARG, "unknown flag bits 0x%x", cfg->flags);
  if ((cfg->flags & MOE_FLAG_STREAM_FC1) && (cfg->flags & MOE_FLAG_NO_STREAM))
    return fail(MOE_ERR_INVALID_ARG, "MOE_FLAG_STREAM_FC1 and MOE_FLAG_NO_STREAM exclude each other");
  if ((cfg->flags & MOE_FLAG_BF16_GATEUP) && !(cfg->flags & MOE_FLAG_UNFUSED_FC1))
    return fail(MOE_ERR_INVALID_ARG, "MOE_FLAG_BF16_GATEUP selects the unfused FC1's gate/up type; it needs MOE_FLAG_UNFUSED_FC1");
  if (cfg->weight_format == MOE_WEIGHT_E4M3_BLOCK128) {
    if (cfg->act_format != MOE_ACT_E4M3_1X128)
      return fail(MOE_ERR_UNSUPPORTED, "E4M3_BLOCK128 weights need E4M3_1X128 activations");
    if ((cfg->flags & MOE_FLAG_UNFUSED_FC1) && (cfg->flags & MOE_FLAG_PERSISTENT_FFN))
      return fail(MOE_ERR_UNSUPPORTED, "the unfused FC1 runs as separate launches; it has no persistent form");
  } else if (is_mx(cfg->weight_format)) {
    if (cfg->act_format != MOE_ACT_BF16)
      return fail(MOE_ERR_UNSUPPORTED, "MXFP8 weights need BF16 activations");
    if (cfg->flags & (MOE_FLAG_PER_ROUTE_STAGING | MOE_FLAG_UNFUSED_FC1 | MOE_FLAG_PERSISTENT_FFN))
      return fail(MOE_ERR_UNSUPPORTED,
                  "per-route staging, the unfused FC1 and the persistent FC1->FC2 are only provided for the FP8 path");
  } else {
    return fail(MOE_ERR_INVALID_ARG, "unknown weight_format %d", cfg->weight_format);
  }
  if (expected_m < 1) return fail(MOE_ERR_INVALID_ARG, "expected_m %d must be >= 1", expected_m);
  if (max_rows < 1) return fail(MOE_ERR_INVALID_ARG, "max_rows %d must be >= 1", max_rows);
  if ((int64_t)max_rows * cfg->top_k > (int64_t)1 << 30)
    return fail(MOE_ERR_UNSUPPORTED, "max_rows * top_k above 2^30");
  if (!(capacity_factor > 0.0f) || !isfinite(capacity_factor))
    return fail(MOE_ERR_INVALID_ARG, "capacity_factor must be finite and > 0");
  return MOE_OK;
}

// Tile tactic from the expected rows per expert: the token tile (block_m)
// is the token bucket, clamped to [16, 256].  Weights always come in 256-row
// tiles (FC1: 128 gate + 128 up rows of one 128-wide block of h; FC2: two
// 128-row blocks of H).
// The MXFP8 variant stages two activation terms per K-block, so its token
// tile stops at 128 (two ring stages of 67 KB).
Tactic choose_tactic(const moe_config_t& cfg, int32_t expected_m) {
  Tactic t;
  t.bucket = token_bucket(expected_m);
  t.block_n = 256;
  // 256-token tiles run the ping-pong FP8 kernel, which has no gate/up
  // output, fused combine or persistent form: those variants (and the MX
  // path, whose stage holds two activation terms) stop at 128.
  const bool cap128 = is_mx(cfg.weight_format) ||
                      (cfg.flags & (MOE_FLAG_UNFUSED_FC1 | MOE_FLAG_FUSED_COMBINE | MOE_FLAG_PERSISTENT_FFN));
  const int cap = cap128 ? 128 : 256;
  t.block_m = t.bucket <= 16 ? 16 : (t.bucket >= cap ? cap : t.bucket);
  // 192-token ping-pong tiles where they pad an expert's expected rows at
  // least 1/8 less than 256-token tiles (129-192 rows: one tile of 192, not
  // of 256; 257-384: two of 192, not two of 256); the 256-token kernel does
  // more per token, so near-equal padding keeps it.
  if (t.block_m == 256) {
    const int64_t m = expected_m;
    const int64_t pad192 = (m + 191) / 192 * 192, pad256 = (m + 255) / 256 * 256;
    if (pad192 * 8 < pad256 * 7) t.block_m = 192;
  }
  t.stages = t.block_m >= 256 ? 2 : (t.block_m >= 64 ? 3 : 4);
  if (is_mx(cfg.weight_format)) t.stages = t.block_m >= 128 ? 2 : (t.block_m >= 32 ? 3 : 4);
  return t;
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// The FP8 GEMMs gather token rows from the staged activations (FC1) and the
// FC1 output (FC2) as 32-bit byte offsets from the buffer's base, kept
// below 2^31 so that they read the same as signed or unsigned.
moe_status_t validate_layout(const moe_config_t& cfg, const Layout& L) {
  const size_t lim = (size_t)1 << 31;
  if (cfg.weight_format == MOE_WEIGHT_E4M3_BLOCK128 &&
      (L.size[MOE_REGION_XQ] >= lim || L.size[MOE_REGION_HQ] >= lim))
    return fail(MOE_ERR_UNSUPPORTED, "staged activations (%zu bytes) and FC1 output (%zu bytes) must each be under 2 GiB",
                L.size[MOE_REGION_XQ], L.size[MOE_REGION_HQ]);
  return MOE_OK;
}

// Regions for max_rows tokens holding row_cap route rows; the create-time
// weight tiles are sized only with `weights`.
static Layout layout_for(const moe_config_t& cfg, const Tactic& t, int32_t max_rows, int64_t row_cap, bool weights) {
  Layout L;
  memset(&L, 0, sizeof(L));
  const int64_t K = cfg.top_k, H = cfg.hidden, I = cfg.intermediate, E = cfg.num_experts;
  const bool mx = cfg.act_format == MOE_ACT_BF16;  // MXFP8 weights x BF16 activations
  L.route_slots = (int64_t)max_rows * K;
  L.rows_x = (cfg.flags & MOE_FLAG_PER_ROUTE_STAGING) ? L.route_slots : max_rows;
  L.row_cap = row_cap < 1 ? 1 : row_cap;
  L.max_m_tiles = (L.row_cap + t.block_m - 1) / t.block_m + E;
  L.compact_blocks = compact_blocks_for(max_rows, cfg.top_k);

  L.size[MOE_REGION_STATUS] = 256;
  L.size[MOE_REGION_STAGED_IDX] = L.route_slots * 4;
  L.size[MOE_REGION_STAGED_W] = L.route_slots * 4;
  L.size[MOE_REGION_XQ] = L.rows_x * H * (mx ? 2 : 1);  // MX: hi-term and lo-term planes
  L.size[MOE_REGION_XS] = mx ? L.rows_x * (H / 32) * 4 : L.rows_x * (H / 128) * 4;
  L.size[MOE_REGION_COUNTS] = E * 4;
  L.size[MOE_REGION_OFFSETS] = (E + 1) * 4;
  L.size[MOE_REGION_SORTED_ROUTE] = L.row_cap * 4;
  L.size[MOE_REGION_ROUTE_POS] = L.route_slots * 4;
  L.size[MOE_REGION_HQ] = L.row_cap * I * (mx ? 2 : 1);
  L.size[MOE_REGION_HS] = mx ? L.row_cap * (I / 32) * 4 : L.row_cap * (I / 128) * 4;
  L.size[MOE_REGION_Y] = L.row_cap * H * 2;
  L.size[MOE_REGION_TILES] = L.max_m_tiles * 4 * 4;
  // create-time tiled copies of the e4m3 weights (FC2 padded to 256-row tiles)
  if (weights) {
    L.size[MOE_REGION_W13T] = E * (2 * I) * H;
    L.size[MOE_REGION_W2T] = E * ((H + 255) / 256 * 256) * I;
    // MX: one 1 KB exponent tile per 32 KB code tile
    L.size[MOE_REGION_W13S] = mx ? L.size[MOE_REGION_W13T] / 32 : 0;
    L.size[MOE_REGION_W2S] = mx ? L.size[MOE_REGION_W2T] / 32 : 0;
  }
  L.size[MOE_REGION_GATEUP] =
      (cfg.flags & MOE_FLAG_UNFUSED_FC1) ? L.row_cap * 2 * I * ((cfg.flags & MOE_FLAG_BF16_GATEUP) ? 2 : 4) : 0;
  L.size[MOE_REGION_READY] = (cfg.flags & MOE_FLAG_PERSISTENT_FFN) ? L.max_m_tiles * 4 : 0;
  L.size[MOE_REGION_ARRIVE] = (cfg.flags & MOE_FLAG_FUSED_COMBINE) ? (int64_t)max_rows * ((H + 255) / 256) * 4 : 0;
  // compaction: per-(workgroup, expert) bases, per-workgroup status bits, the arrival counter
  L.size[kRegionBlkBase] = (L.compact_blocks * (E + 1) + 1) * 4;
  size_t off = 0;
  for (int r = 0; r < kNumRegions; ++r) {
    L.off[r] = off;
    off += align256(L.size[r]);
  }
  L.total = off;
  return L;
}

Layout compute_layout(const moe_config_t& cfg, const Tactic& t, int32_t max_rows, float capacity_factor) {
  const int64_t slots = (int64_t)max_rows * cfg.top_k;
  const double cap = ceil((double)capacity_factor * (double)slots);
  return layout_for(cfg, t, max_rows, cap >= (double)slots ? slots : (int64_t)cap, true);
}

Layout compute_scratch_layout(const moe_config_t& cfg, const Tactic& t, int32_t tokens, int64_t layer_row_cap) {
  const int32_t rows = tokens > 0 ? tokens : 1;
  const int64_t slots = (int64_t)rows * cfg.top_k;
  return layout_for(cfg, t, rows, layer_row_cap < slots ? layer_row_cap : slots, false);
}

}  // namespace moe

extern "C" int32_t moe_token_bucket(int32_t tokens) { return moe::token_bucket(tokens); }

extern "C" const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_CAPACITY: return "MOE_ERR_CAPACITY";
    case MOE_ERR_STATE: return "MOE_ERR_STATE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

extern "C" const char* moe_last_error(void) { return moe::last_error(); }

extern "C" moe_status_t moe_workspace_query(const moe_config_t* cfg, int32_t expected_m, int32_t max_rows,
                                            float capacity_factor, size_t* ws_bytes) {
  moe::clear_error();
  moe_status_t s = moe::validate_config(cfg, expected_m, max_rows, capacity_factor);
  if (s != MOE_OK) return s;
  if (!ws_bytes) return moe::fail(MOE_ERR_INVALID_ARG, "ws_bytes is NULL");
  moe::Tactic t = moe::choose_tactic(*cfg, expected_m);
  const moe::Layout L = moe::compute_layout(*cfg, t, max_rows, capacity_factor);
  s = moe::validate_layout(*cfg, L);
  if (s != MOE_OK) return s;
  *ws_bytes = L.total;
  return MOE_OK;
}
