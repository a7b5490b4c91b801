// Internal declarations shared by the host side and the kernel launchers.
// Nothing here is part of the public ABI (include/moe.h).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kCompactChunk = 4096;        // bound on the routes per compaction workgroup (256 lanes x 16)
constexpr int kCompactOneRoutes = 2048;    // batches up to this many routes compact in one workgroup
constexpr int kCompactBlockRoutes = 1024;  // beyond that, about this many routes per workgroup
constexpr int kNumRegions = 21;
constexpr int kRegionBlkBase = 20;   // internal: per-(compaction block, expert) bases

// Words of the device header (MOE_REGION_STATUS).
enum HeaderWord : int {
  kHdrStatus = 0,      // MOE_DEV_* bits
  kHdrTokens = 1,      // tokens staged
  kHdrRoutes = 2,      // routes kept after compaction (R)
  kHdrMTiles = 3,      // (expert, row-tile) pairs in the tile list
};

struct Tactic {
  int32_t bucket;
  int32_t block_m;
  int32_t block_n;
  int32_t stages;
};

struct Layout {
  int64_t rows_x;       // staged activation rows (max_rows, or max_rows*K per-route)
  int64_t route_slots;  // max_rows * K
  int64_t row_cap;      // route rows held by h/y
  int64_t max_m_tiles;  // bound on the tile list length
  int64_t compact_blocks;  // compaction workgroups at max_rows tokens
  size_t off[kNumRegions];
  size_t size[kNumRegions];
  size_t total;
};

// Host-only logic (moe_host.cpp, no HIP dependency).
int32_t token_bucket(int32_t tokens);
// Tokens per compaction workgroup when there are several: whole tokens,
// at most kCompactBlockRoutes routes.
inline int32_t compact_chunk_tokens(int32_t top_k) { return kCompactBlockRoutes / top_k; }
// Compaction workgroups for `tokens` staged tokens: one (which also writes
// the header when no token is staged) up to kCompactOneRoutes routes.
inline int32_t compact_blocks_for(int64_t tokens, int32_t top_k) {
  if (tokens * top_k <= kCompactOneRoutes) return 1;
  const int64_t tc = compact_chunk_tokens(top_k);
  return (int32_t)((tokens + tc - 1) / tc);
}
// Routes per compaction workgroup (the whole batch for one workgroup).
inline int32_t compact_chunk_routes(int64_t tokens, int32_t top_k) {
  if (tokens * top_k <= kCompactOneRoutes) return tokens > 0 ? (int32_t)(tokens * top_k) : top_k;
  return compact_chunk_tokens(top_k) * top_k;
}
// Limits that depend on the layout (call after compute_layout).
moe_status_t validate_layout(const moe_config_t& cfg, const Layout& L);
moe_status_t validate_config(const moe_config_t* cfg, int32_t expected_m, int32_t max_rows,
                             float capacity_factor);
Tactic choose_tactic(const moe_config_t& cfg, int32_t expected_m);
Layout compute_layout(const moe_config_t& cfg, const Tactic& t, int32_t max_rows, float capacity_factor);
// The per-call regions of one call of `tokens` tokens (no weight tiles),
// holding min(layer_row_cap, tokens * K) route rows: routes drop exactly as
// in the layer's workspace.
Layout compute_scratch_layout(const moe_config_t& cfg, const Tactic& t, int32_t tokens, int64_t layer_row_cap);
// Device address and size of the library's static scratch on the current
// device (moe_noalloc.hip); 0 on success.
int noalloc_scratch(uint8_t** base, size_t* bytes);
moe_status_t fail(moe_status_t s, const char* fmt, ...);
void clear_error();

// ---------------------------------------------------------------------------
// Kernel launchers (moe_*.hip).  All take a hipStream_t as void*.
// ---------------------------------------------------------------------------

struct StageArgs {
  const void* x;          // bf16 [T, H] or e4m3 [T, H]
  const float* x_scale;   // null for bf16 input
  const int32_t* topk_idx;
  const float* topk_w;
  int32_t tokens, max_rows, hidden, top_k, num_experts;
  uint32_t flags;
  int32_t act_format;
  // workspace
  uint32_t* hdr;
  int32_t* staged_idx;
  float* staged_w;
  uint8_t* xq;            // e4m3 rows; MX variant: hi-term plane then lo-term plane
  float* xs;              // 1x128 float32 scales (FP8 path)
  int64_t x_plane;        // MX variant: bytes from the hi-term plane to the lo-term plane
  uint32_t* xs_mx;        // MX variant: packed E8M0 exponents [rows, H/32] (byte 0 hi, byte 1 lo)
};
struct CompactArgs;
// One launch stages the batch: the first c.blocks workgroups stage and check
// the route rows and compact them (the whole compaction when c.blocks == 1,
// else everything but the scatter), the others quantise (or split) x.
int launch_stage(const StageArgs& a, const CompactArgs& c, void* stream);

struct CompactArgs {
  const int32_t* staged_idx;
  int32_t routes;          // T*K
  int32_t num_experts;
  int32_t row_cap;
  int32_t block_m;
  int32_t blocks;          // compaction workgroups
  int32_t chunk;           // routes per workgroup (whole tokens, <= kCompactChunk): compact_chunk_routes
  uint32_t* hdr;
  int32_t* blk_base;       // [blocks, E]
  uint32_t* blk_status;    // [blocks] MOE_DEV_* bits of each workgroup's route rows
  int32_t* arrive;         // one word, zero between launches: compaction workgroups done counting
  int32_t* counts;         // [E]
  int32_t* offsets;        // [E+1]
  int32_t* sorted_route;   // [row_cap]
  int32_t* route_pos;      // [routes]
  int32_t* tiles;          // [max_m_tiles, 4] (expert, first sorted row, rows, only-tile flag)
  int32_t* ready;          // [max_m_tiles] persistent FC1->FC2 counters, zeroed per listed tile (or null)
};
// Scatter of a compaction split over several workgroups (after launch_stage).
int launch_compact_scatter(const CompactArgs& a, void* stream);

// Operands of the last-arriver combine fused into FC2 (moe_combine_dev.h).
struct FusedCombineArgs {
  uint16_t* out;             // bf16 [T, H]; null: FC2 stores y only
  const int32_t* route_pos;  // [T*K]
  const float* route_w;      // [T*K] staged weights
  int32_t* arrive;           // [max_rows, ceil(H/256)] arrival counters, zero between forwards
};

struct GemmArgs {
  // A operand: activation rows
  const uint8_t* a;        // e4m3 rows
  const float* a_scale;    // [rows, K/128]
  int32_t a_mode;          // 0: sorted position p; 1: token = route/K; 2: route id
  const int32_t* sorted_route;
  int32_t top_k;
  // B operand: expert weights tiled by moe_weights.hip ([E, n_tiles, K/128] x 32 KB)
  const uint8_t* w;
  const float* w_scale;    // [E, N/128, K/128]
  int32_t n_rows;          // N (2I for FC1, H for FC2)
  int32_t k_dim;           // K (H for FC1, I for FC2)
  int32_t inter;           // I (FC1 gate/up split)
  int32_t n_tiles;         // output column tiles
  // tiles
  const int32_t* tiles;    // [m] = (expert, first sorted row, rows, 1 if the expert's only row tile)
  const int32_t* offsets;  // kept offsets [E+1]
  const uint32_t* hdr;
  // outputs
  uint8_t* hq;  float* hs; // FC1: e4m3 [R, I], scales [R, I/128]
  uint16_t* y;             // FC2: bf16 [R, H]
  float* gateup;           // FC1, unfused: gate/up rows [R, 2I] instead of the fused epilogue
  int32_t gateup_bf16;     //   ... stored as bfloat16 bits (RNE) instead of FP32
  int32_t grid;
  FusedCombineArgs fc;     // FC2: last-arriver combine into the output (fc.out null: none)
  int32_t stream_depth;    // 64-token tiles: K-blocks in flight of the streaming kernel (0: LDS-ring kernel)
};
int launch_fc1(const GemmArgs& a, int block_m, void* stream);

// FC1 then FC2 in one persistent cooperative launch (MOE_FLAG_PERSISTENT_FFN).
// FC1 row tile m counts its finished column tiles in ready[m]; an FC2 tile
// of row tile m starts once ready[m] == need.  A wait longer than the spin
// bound sets MOE_DEV_WAIT_TIMEOUT in *status and goes on.
struct PersistArgs {
  int32_t* ready;    // [max_m_tiles], zeroed by the compaction for the tiles it lists
  int32_t need;      // FC1 column tiles per row tile (I / 128)
  uint32_t* status;  // device status word (MOE_DEV_* bits)
};
int launch_fc1_fc2(const GemmArgs& a1, const GemmArgs& a2, const PersistArgs& q, int block_m, int grid, void* stream);
int gemm_persist_max_workgroups_per_cu(int block_m);
// Unfused FC1 second half: SwiGLU + 1x128 requant of the FP32 gate/up rows.
int launch_swiglu_quant(const void* gateup, bool bf16, int32_t row_cap, int32_t inter, const uint32_t* hdr,
                        uint8_t* hq, float* hs, void* stream);
int launch_fc2(const GemmArgs& a, int block_m, void* stream);
// K-blocks in flight per workgroup of the streaming FP8 kernel for a GEMM
// with `kbs` K-blocks and `n_tiles` column tiles at token tile block_m, or 0
// where the LDS-ring kernel runs.
int gemm_stream_depth(int block_m, int kbs, int n_tiles);
int gemm_max_workgroups_per_cu(int which, int block_m, int stream_depth);

// MXFP8-weight x BF16-activation GEMMs (moe_gemm_mx.hip).  Activations are
// held as two e4m3 terms with their own E8M0 exponent per 32 K-elements.
struct MxGemmArgs {
  const uint8_t* a;          // hi-term rows; the lo-term rows are a_plane bytes further
  int64_t a_plane;
  const uint32_t* a_scale;   // [rows, K/32] packed E8M0 (byte 0 hi term, byte 1 lo term)
  int32_t a_mode;            // 0: sorted position p; 1: token = route/K
  const int32_t* sorted_route;
  int32_t top_k;
  const uint8_t* w;          // e4m3 weight tiles, MX operand order ([E, n_tiles, K/128] x 32 KB)
  const uint32_t* w_scale;   // E8M0 weight scale tiles ([E, n_tiles, K/128] x 256 words)
  int32_t n_rows, k_dim, inter, n_tiles;
  const int32_t* tiles;    // [m] = (expert, first sorted row, rows, 1 if the expert's only row tile)
  const int32_t* offsets;
  const uint32_t* hdr;
  uint8_t* hq;               // FC1: hi-term rows [R, I]; lo-term rows h_plane bytes further
  int64_t h_plane;
  uint32_t* hs;              // FC1: packed E8M0 [R, I/32]
  uint16_t* y;               // FC2: bf16 [R, H]
  int32_t grid;
  int32_t w_e5m2;            // weight element type: 0 e4m3, 1 e5m2
  FusedCombineArgs fc;       // FC2: last-arriver combine into the output (fc.out null: none)
};
int launch_fc1_mx(const MxGemmArgs& a, int block_m, void* stream);
int launch_fc2_mx(const MxGemmArgs& a, int block_m, void* stream);
int gemm_mx_max_workgroups_per_cu(int which, int block_m);

struct CombineArgs {
  const uint16_t* y;
  const int32_t* route_pos;
  const float* staged_w;
  int32_t tokens, top_k, hidden;
  uint16_t* out;
};
int launch_combine(const CombineArgs& a, void* stream);
// Zero-fill of 32-bit words (the arrival counters at create).
int launch_fill_zero(uint32_t* p, int64_t words, void* stream);

// MXFP8 weight formats (either element type, E8M0 scales per 32).
inline bool is_mx(int weight_format) {
  return weight_format == MOE_WEIGHT_MXFP8_E4M3 || weight_format == MOE_WEIGHT_MXFP8_E5M2;
}

// Weight tile orders (moe_weights.hip): 16x16x128 fragments (FP8 path) and
// the MX-scaled operand order (MXFP8 path).
enum TileOrder : int { kTileOrder16 = 0, kTileOrderMx = 1 };
int launch_tile_weights(const uint8_t* src, uint8_t* dst, int experts, int n_rows, int k_dim, int n_tiles,
                        int inter, bool fc1, int order, void* stream);
int launch_tile_mx_scales(const uint8_t* src, uint32_t* dst, int experts, int n_rows, int k_dim, int n_tiles,
                          int inter, bool fc1, void* stream);

}  // namespace moe
