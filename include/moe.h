/*
 * moe.h -- C ABI of the MI355X (gfx950) MegaMoE per-rank layer forward.
 *
 * One GPU's share of an expert-parallel MoE layer: the rows "received" from
 * peers are a plain device buffer, and the layer runs
 *
 *   stage (quantise x to e4m3 1x128, check + mask routes)
 *   -> compact (per-expert row lists)
 *   -> FC1 (FP8 block-scale grouped GEMM) with fused SwiGLU + 1x128 requant
 *   -> FC2 (FP8 block-scale grouped GEMM)
 *   -> owner-side FP32 weighted top-k combine to a BF16 output.
 *
 * Optional forms of the same arithmetic (cfg->flags): the unfused FC1, the
 * combine fused into FC2, and FC1 + FC2 in one persistent launch.
 *
 * This is the forward pipeline in the Description of "feat(moe_ep): add SM90
 * push FP8 mega-MoE backend for Hopper" (flashinfer PR #4069) with its
 * cross-GPU steps (tags, acks, peer dispatch, prefix waits) removed, the
 * staging contract of "perf(moe_ep): fuse Rubin MegaMoE forward preparation"
 * (PR #6398) and the BF16-activation x MXFP8-weight variant of
 * "feat(moe_ep): MXFP8 x BF16 integration" (PR #4604).
 *
 * Conventions for every entry point:
 *  - Device pointers are HIP device memory owned by the caller; the library
 *    never allocates or frees device memory.  Host pointers are marked.
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *    Every launch is stream-ordered; no entry point except moe_read_status
 *    synchronises with the host.
 *  - A negative moe_status_t is returned by synchronous host validation
 *    before anything is launched; moe_last_error() then describes it.
 *  - Problems found on the device (bad routes, capacity overflow) never
 *    abort: the offending routes are masked and a bit is set in the device
 *    status word, read with moe_read_status().  Every wait inside a kernel
 *    is bounded; one that gives up sets MOE_DEV_WAIT_TIMEOUT instead of
 *    hanging.
 *  - Calls on one layer handle are not thread-safe; distinct handles with
 *    distinct workspaces are independent.  The launches of one handle must
 *    also not overlap on the device (issue them on one stream, or order the
 *    streams): its workspace holds the staged batch between calls and a
 *    counter the staging launch leaves at zero for the next one.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,        /* null/misaligned pointer, bad size or value */
  MOE_ERR_UNSUPPORTED = -2,        /* valid but unsupported configuration */
  MOE_ERR_WORKSPACE_TOO_SMALL = -3,
  MOE_ERR_CAPACITY = -4,           /* num_tokens > max_rows */
  MOE_ERR_STATE = -5,              /* call out of order (forward before stage) */
  MOE_ERR_HIP = -6                 /* a HIP runtime call failed */
} moe_status_t;

/* Weight storage formats. */
enum {
  /* e4m3 (OCP, max 448) codes with one float32 scale per 128x128 block --
   * the DeepSeek-style FP8 block scaling listed in the Limitations of PR #4069. */
  MOE_WEIGHT_E4M3_BLOCK128 = 0,
  /* e4m3 codes with one E8M0 exponent per 32 consecutive K elements (OCP MX)
   * -- the MXFP8 weights of PR #4604. */
  MOE_WEIGHT_MXFP8_E4M3 = 1,
  /* e5m2 (OCP, max 57344) codes with one E8M0 exponent per 32 consecutive K
   * elements -- the other MXFP8 element type of PR #4604. */
  MOE_WEIGHT_MXFP8_E5M2 = 2
};

/* Activation formats (what moe_stage_inputs receives and FC1 consumes). */
enum {
  MOE_ACT_E4M3_1X128 = 0,  /* e4m3 rows with one float32 scale per 128 columns */
  /* bfloat16 rows (MXFP8 variant).  The gfx950 scaled MFMA takes FP8/FP6/FP4
   * operands only, so each row is carried as two e4m3 terms with their own
   * E8M0 exponent per 32 columns, hi = e4m3(x/2^a) and lo = e4m3((x - hi)/2^b);
   * hi + lo keeps 8 significant bits, within 2^-9 of x relatively.  h between
   * the GEMMs is rounded to bfloat16 (PR #4604, Description) and split the
   * same way. */
  MOE_ACT_BF16 = 1
};

/* cfg->flags */
enum {
  /* Value checks of the routing checker of PR #6398: duplicate experts within
   * a token and non-finite weights on active routes.  Off: the caller
   * guarantees valid routing; expert-id bounds are still enforced and masked
   * scores still zeroed. */
  MOE_FLAG_CHECK_ROUTES = 1u,
  /* Stage one activation row per route instead of one per token.  Exists to
   * show the deduplicated layout gives identical results (PR #4069,
   * Description, deduplicated dispatch bullet); costs K times the rows. */
  MOE_FLAG_PER_ROUTE_STAGING = 2u,
  /* Unfused FC1 (E4M3_BLOCK128 weights only): the FC1 GEMM stores its FP32
   * gate/up output in MOE_REGION_GATEUP and a separate kernel applies SwiGLU
   * and the 1x128 requantisation.  A debug and cross-check path for the fused
   * epilogue (PR #4069, Description: the fused FC1 reproduces the unfused
   * path); it gives the same bits and costs a 2I x 4-byte row per route. */
  MOE_FLAG_UNFUSED_FC1 = 4u,
  /* Fused last-arriver combine: FC2 still stores the un-weighted rows in
   * MOE_REGION_Y, and the FC2 tile that stores the last kept route of a
   * token over a 256-column slice reduces that token's routes over the slice
   * into the output, with the standalone combine's FP32 arithmetic (same
   * bits), so no combine launch follows FC2 (SM90 pull-style MegaMoE,
   * flashinfer PR #4688, commit list: grouped token-back, where the last FC2
   * row of a token's group reduces every member in FP32).  Uses the arrival
   * counters of MOE_REGION_ARRIVE, zeroed at create and returned to zero by
   * every forward.  The y rows are then stored write-through so that a tile
   * on another XCD can read them; on MI355X this costs more than the
   * separate combine launch it saves, so the flag is off by default. */
  MOE_FLAG_FUSED_COMBINE = 8u,
  /* Persistent FC1->FC2 (E4M3_BLOCK128 weights only): one cooperative launch
   * runs every FC1 tile and then every FC2 tile of each workgroup, and an
   * FC2 tile starts as soon as all FC1 column tiles of its row tile have
   * stored their rows (per-row-tile readiness counters in MOE_REGION_READY),
   * instead of after the whole FC1 launch (SM90 pull-style MegaMoE,
   * flashinfer PR #4688: persistent kernel with fc1_done readiness flags).
   * Same arithmetic, same bits.  The h rows are then stored write-through so
   * that a tile on another XCD can read them. */
  MOE_FLAG_PERSISTENT_FFN = 16u,
  /* With MOE_FLAG_UNFUSED_FC1 only: the FC1 GEMM rounds its gate/up output
   * to bfloat16 (round to nearest even) and stores that in
   * MOE_REGION_GATEUP; SwiGLU and the requantisation then read the BF16
   * values.  This is the unfused path's own BF16 gate/up buffer (PR #4069,
   * Description: the unfused FC1 stores a BF16 gate/up buffer before the
   * SwiGLU, and stays the maintained reference), so h differs from the fused
   * epilogue's by that rounding.  Costs a 2I x 2-byte row per route. */
  MOE_FLAG_BF16_GATEUP = 32u,
  /* Run FC2 at 64-token tiles on the LDS-ring GEMM kernel instead of the
   * streaming kernel.  The streaming kernel (FP8 path without UNFUSED_FC1,
   * FUSED_COMBINE or PERSISTENT_FFN, where the GEMM's K-blocks and column
   * tiles come in pairs) computes two 256-row weight tiles against one
   * 64-token tile per workgroup and loads the weights straight into a
   * register ring two K-blocks deep.  Same arithmetic, same bits; a
   * cross-check and comparison path. */
  MOE_FLAG_NO_STREAM = 64u,
  /* Run FC1 at 64-token tiles on the streaming kernel too, with
   * non-temporal weight loads.  Faster when every expert gets about one
   * token tile (balanced routing); slower when some experts get many tiles,
   * whose weights several workgroups then read from HBM again.  Excludes
   * MOE_FLAG_NO_STREAM. */
  MOE_FLAG_STREAM_FC1 = 128u
};

/* Device status bits (moe_read_status). */
enum {
  MOE_DEV_BAD_EXPERT = 1u,   /* an expert id outside [-1, E) was masked */
  MOE_DEV_DUPLICATE = 2u,    /* a repeated expert within a token was masked (lowest slot kept) */
  MOE_DEV_NONFINITE = 4u,    /* an active route with a NaN/inf weight was masked */
  MOE_DEV_CAPACITY = 8u,     /* routes beyond the row capacity were dropped */
  MOE_DEV_WAIT_TIMEOUT = 16u /* MOE_FLAG_PERSISTENT_FFN: an FC2 tile gave up waiting for its FC1 rows
                                (never expected; the output is then not valid) */
};

typedef struct {
  int32_t hidden;         /* H, multiple of 128, <= 16384 */
  int32_t intermediate;   /* I, multiple of 128, <= 16384 (FC1 produces 2I: gate rows then up rows) */
  int32_t num_experts;    /* E local experts, 1..1024 */
  int32_t top_k;          /* K in {1, 2, 4, 6, 8} (Limitations of PR #4069) */
  int32_t weight_format;  /* MOE_WEIGHT_* */
  int32_t act_format;     /* MOE_ACT_*: E4M3_1X128 with E4M3_BLOCK128 weights, BF16 with MXFP8 */
  uint32_t flags;         /* MOE_FLAG_* */
} moe_config_t;

/* Static expert weights, device memory, row-major, K contiguous:
 *   w13       e4m3 [E, 2I, H]   rows 0..I-1 gate, rows I..2I-1 up
 *   w2        e4m3 [E, H, I]
 *   E4M3_BLOCK128: w13_scale float32 [E, 2I/128, H/128], w2_scale float32 [E, H/128, I/128]
 *   MXFP8_E4M3 / MXFP8_E5M2: w13_scale uint8 [E, 2I, H/32], w2_scale uint8 [E, H, I/32]
 * The caller keeps them alive and unchanged while the layer handle exists. */
typedef struct {
  const void* w13;
  const void* w13_scale;
  const void* w2;
  const void* w2_scale;
} moe_weights_t;

/* Tile tactic the library chose (informational). */
typedef struct {
  int32_t token_bucket;  /* clamped ceil-power-of-two of expected_m, in [8, 32768] */
  int32_t block_m;       /* rows per GEMM tile */
  int32_t block_n;       /* weight rows per GEMM tile */
  int32_t grid_fc1;      /* persistent workgroups launched for FC1 */
  int32_t grid_fc2;
  int32_t row_cap;       /* route rows the workspace holds */
  int32_t max_m_tiles;   /* bound on (expert, row-tile) pairs */
  int32_t tile_order;    /* weight tile order in MOE_REGION_W13T/W2T: 0 16x16x128 fragments,
                            1 MX-scaled operand order */
  int32_t stream_depth_fc1;  /* K-blocks in flight per workgroup in the streaming FC1 kernel
                                (0: the LDS-ring kernel runs) */
  int32_t stream_depth_fc2;  /* the same for FC2 */
} moe_tactic_t;

/* Workspace regions exposed for inspection (moe_layer_region). */
enum {
  MOE_REGION_STATUS = 0,        /* uint32 [8]: status bits, staged tokens, kept routes, m-tiles */
  MOE_REGION_STAGED_IDX = 1,    /* int32 [max_rows*K]   expert per route, -1 masked */
  MOE_REGION_STAGED_W = 2,      /* float32 [max_rows*K] weight per route, 0 masked */
  MOE_REGION_XQ = 3,            /* e4m3 [rows_x, H]; MOE_ACT_BF16: [2][rows_x, H] hi-term then lo-term codes */
  MOE_REGION_XS = 4,            /* float32 [rows_x, H/128]; MOE_ACT_BF16: uint32 [rows_x, H/32] E8M0 pairs */
  MOE_REGION_COUNTS = 5,        /* int32 [E]   kept routes per expert */
  MOE_REGION_OFFSETS = 6,       /* int32 [E+1] exclusive prefix of counts */
  MOE_REGION_SORTED_ROUTE = 7,  /* int32 [row_cap] route ids t*K+k, expert-major, ascending in expert */
  MOE_REGION_ROUTE_POS = 8,     /* int32 [max_rows*K] inverse of sorted_route, -1 if not kept */
  MOE_REGION_HQ = 9,            /* FC1 output rows: e4m3 [row_cap, I]; MXFP8: [2][row_cap, I] hi/lo-term codes */
  MOE_REGION_HS = 10,           /* float32 [row_cap, I/128]; MXFP8: uint32 [row_cap, I/32] E8M0 pairs */
  MOE_REGION_Y = 11,            /* bf16 [row_cap, H] un-weighted FC2 rows */
  MOE_REGION_TILES = 12,        /* int32 [max_m_tiles, 4] (expert, first sorted row, rows, 1 if the expert's only tile) */
  MOE_REGION_W13T = 13,         /* e4m3 w13 tiled at create: [E, I/128, H/128] tiles of 32 KB */
  MOE_REGION_W2T = 14,          /* e4m3 w2 tiled at create: [E, ceil(H/256), I/128] tiles of 32 KB */
  MOE_REGION_W13S = 15,         /* MXFP8: w13 E8M0 tiled at create, 1 KB per w13 tile (empty for FP8) */
  MOE_REGION_W2S = 16,          /* MXFP8: w2 E8M0 tiled at create, 1 KB per w2 tile (empty for FP8) */
  MOE_REGION_GATEUP = 17,       /* MOE_FLAG_UNFUSED_FC1: float32 [row_cap, 2I] gate then up columns (bfloat16 bits
                                 * with MOE_FLAG_BF16_GATEUP; else empty) */
  MOE_REGION_ARRIVE = 18,       /* MOE_FLAG_FUSED_COMBINE: int32 [max_rows, ceil(H/256)] arrival counters,
                                   zero between forwards (else empty) */
  MOE_REGION_READY = 19         /* MOE_FLAG_PERSISTENT_FFN: int32 [max_m_tiles] finished FC1 column tiles
                                   per row tile, zeroed by the compaction (else empty) */
};

/* Kernel classes timed by the optional profiler. */
enum {
  MOE_KERNEL_STAGE = 0,    /* the staging launch: quantisation, route staging, compaction counts */
  MOE_KERNEL_COMPACT = 1,  /* the compaction's scatter, when it is a launch of its own */
  MOE_KERNEL_FC1 = 2,
  MOE_KERNEL_FC2 = 3,
  MOE_KERNEL_COMBINE = 4,
  MOE_KERNEL_COUNT = 5
};

typedef struct moe_layer moe_layer_t;

/* Size of the device workspace a layer needs.  Host only, launches nothing.
 *  expected_m      expected rows per expert; picks the tile tactic only.
 *  max_rows        token capacity per call (bounds memory).
 *  capacity_factor route rows held = ceil(capacity_factor * max_rows * K),
 *                  capped at max_rows*K; 1.0 never drops a route.
 *  ws_bytes        [host out] bytes, a multiple of 256.
 * MOE_ERR_UNSUPPORTED when, with E4M3_BLOCK128 weights, the staged
 * activations (max_rows * H bytes, max_rows * K * H with per-route staging)
 * or the FC1 output (route rows held * I bytes) reach 2 GiB: the FP8 GEMMs
 * address them with 31-bit offsets.
 * The split between tactic (expected_m) and memory bound (max_rows,
 * capacity_factor) is the workspace contract of PR #4069 ("Contracts
 * introduced by this PR": capacity_factor bounds the GEMM and scale buffers;
 * the query takes explicit expected_m and max_rows). */
moe_status_t moe_workspace_query(const moe_config_t* cfg, int32_t expected_m, int32_t max_rows,
                                 float capacity_factor, size_t* ws_bytes);

/* Bind the static weights and the workspace (PR #4069, Contracts: the
 * construction of the stateful variant binds transformed static weights).
 *  cfg, w          [host in] copied.
 *  workspace       device, 256-byte aligned, ws_bytes >= moe_workspace_query().
 *  stream          the weight transform is launched on it.
 *  out             [host out] new handle (host memory owned by the library).
 * Launches one transform per weight tensor that copies the e4m3 codes into
 * the workspace in the kernels' tile order (MOE_REGION_W13T / W2T).
 * E4M3_BLOCK128: the float32 scale tensors are read in place, so the caller
 * keeps them alive and unchanged while the handle exists.  MXFP8_E4M3: the
 * E8M0 tensors are tiled too (MOE_REGION_W13S / W2S).  Every tensor copied
 * into the workspace may be released once the stream has passed the create
 * call. */
moe_status_t moe_layer_create(const moe_config_t* cfg, int32_t expected_m, int32_t max_rows,
                              float capacity_factor, const moe_weights_t* w, void* workspace,
                              size_t ws_bytes, void* stream, moe_layer_t** out);

/* Stage one batch of received rows and bind the output tensor
 * (PR #4069, Contracts: stage_inputs pre-binds the caller's output tensor;
 * PR #6398: fused input quantisation + route staging + routing checker).
 *  x          device. act_format E4M3_1X128: either bfloat16 [T, H] with
 *             x_scale == NULL (quantised here: s = amax/448 per 1x128 block,
 *             q = RNE_sat(x/s)), or e4m3 [T, H] with x_scale float32
 *             [T, H/128] (copied).  act_format BF16: bfloat16 [T, H], x_scale NULL.
 *  topk_idx   device int32 [T, K]: expert per slot, -1 = masked slot.
 *  topk_w     device float32 [T, K]: routing weight (ignored for masked slots).
 *  num_tokens T, 0 <= T <= max_rows (else MOE_ERR_CAPACITY).
 *  out_bf16   device bfloat16 [T, H], written by the next moe_layer_forward.
 * The caller's tensors are never modified.  Rows [T, max_rows) of the staged
 * routes are masked.  The same launch counts the staged routes per expert
 * and builds the row-tile list; for batches of up to 2048 routes it also
 * finishes the compaction (the per-route positions). */
moe_status_t moe_stage_inputs(moe_layer_t* layer, const void* x, const float* x_scale,
                              const int32_t* topk_idx, const float* topk_w, int32_t num_tokens,
                              void* out_bf16, void* stream);

/* Run the rest of the compaction (the per-route positions, for batches over
 * 2048 routes) -> FC1(+SwiGLU+requant) -> FC2 -> combine on the staged batch
 * (with MOE_FLAG_FUSED_COMBINE the combine runs inside FC2).
 * Stream-ordered, no host synchronisation (PR #4069, Description: no
 * host-side synchronization in the steady-state forward). */
moe_status_t moe_layer_forward(moe_layer_t* layer, void* stream);

/* Stage + forward of one batch without allocating: for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid it).  Same arguments and results as
 * moe_stage_inputs followed by moe_layer_forward, on the same kernels, except
 * that every per-call region (staged rows and routes, compaction, FC1
 * output, FC2 rows, tile list, status header) lives in a static device
 * scratch of 64 MiB per device that the library holds until the process
 * ends; the layer's workspace supplies only its create-time weight tiles
 * and is not written.
 *  status_bits  device uint32, may be NULL: receives the call's MOE_DEV_*
 *               bits (moe_read_status does not see them).
 * The handle's own staged batch (moe_stage_inputs) is left as it was.
 * MOE_ERR_CAPACITY when num_tokens > max_rows or when the call's regions do
 * not fit in the scratch (about 139 KB per token at H=7168, I=2048, K=8:
 * some 480 tokens); nothing is launched then.  Calls no hipMalloc, hipFree
 * or allocating routine (the first call on a device looks up the scratch's
 * address).  Every call on a device shares that device's scratch, and it
 * keeps the last call's contents: calls that overlap on one device (on
 * different streams, or from different threads) race. */
moe_status_t moe_layer_forward_noalloc(moe_layer_t* layer, const void* x, const float* x_scale,
                                       const int32_t* topk_idx, const float* topk_w, int32_t num_tokens,
                                       void* out_bf16, uint32_t* status_bits, void* stream);

/* Synchronise `stream` and return the device status bits (MOE_DEV_*)
 * accumulated since the last moe_stage_inputs.  bits: [host out]. */
moe_status_t moe_read_status(moe_layer_t* layer, void* stream, uint32_t* bits);

/* Device pointer and size of a workspace region (MOE_REGION_*). */
moe_status_t moe_layer_region(moe_layer_t* layer, int32_t region, void** dptr, size_t* bytes);

/* The tactic chosen at create time. tactic: [host out]. */
moe_status_t moe_layer_tactic(const moe_layer_t* layer, moe_tactic_t* tactic);

/* Optional per-kernel timing with HIP events recorded around the launches
 * of the selected kernel classes on the launch stream.  kernel_mask: bit
 * (1 << MOE_KERNEL_*) per class to time, MOE_PROFILE_ALL for all of them,
 * 0 to stop; a non-zero mask starts (and resets) accumulation.  Each event
 * pair costs a few microseconds of stream time, so time only the classes
 * needed.  moe_profile_read synchronises, then returns, per MOE_KERNEL_*
 * class, the summed milliseconds and the number of launches timed (host
 * arrays of MOE_KERNEL_COUNT). */
#define MOE_PROFILE_ALL ((1u << MOE_KERNEL_COUNT) - 1u)
moe_status_t moe_profile_enable(moe_layer_t* layer, uint32_t kernel_mask);
moe_status_t moe_profile_read(moe_layer_t* layer, double* ms_total, int64_t* launches);

/* Cycle counters of the 256-token FP8 GEMM kernel's slots, for measuring
 * where its K loop spends time; not for production use.  Only a library
 * built with slot timers (build.py --slot-timers, which compiles the
 * counter reads into the kernel) records them; any other build returns
 * MOE_ERR_UNSUPPORTED and writes nothing.  out: host array of `count`
 * (>= MOE_SLOT_TIMER_WORDS) uint64, laid out [GEMM: FC1, FC2][wave group:
 * 0, 1][word]: words 0-6 the summed cycles of load-slot DMA issue, load-slot
 * LDS reads and records, load-slot barrier wait, MFMA-slot issue, wait for
 * the wave's own loads, MFMA-slot barrier wait, tile epilogue; word 7 the
 * number of K-blocks; summed over waves and launches since the previous
 * call, which then clears them.  Synchronises the device. */
#define MOE_SLOT_TIMER_WORDS 32
moe_status_t moe_debug_slot_timers(uint64_t* out, int32_t count);

/* Release the handle (host memory only; the workspace stays the caller's).
 * Destroying NULL is a no-op. */
moe_status_t moe_layer_destroy(moe_layer_t* layer);

/* Token bucket of the tactic table: clamped ceil power of two in
 * [8, 32768] (test "token bucket uses clamped ceil power of two" of the SM90
 * pull-style MegaMoE, flashinfer PR #4688).  Returns -1 for tokens <= 0. */
int32_t moe_token_bucket(int32_t tokens);

/* Static string for a status code; thread-local description of the last
 * error of this thread (empty if none). */
const char* moe_status_string(moe_status_t status);
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
