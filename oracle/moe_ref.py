"""Float64 reference of the MegaMoE per-rank layer forward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``): never imported by the
library.

Steps, in the order of the forward pipeline listed in the Description of
"feat(moe_ep): add SM90 push FP8 mega-MoE backend for Hopper" (PR #4069), with
the cross-GPU transport steps removed (rows "received" from peers are a plain
input here):

1. ``stage_quantize_1x128`` / ``stage_routes`` -- input quantisation and route
   staging with the routing checker ("perf(moe_ep): fuse Rubin MegaMoE forward
   preparation", PR #6398, Description and the follow-up commit on masked
   routes).
2. ``compact`` -- per-expert row lists (PR #4069 pipeline step "compact").
3. ``fc1_swiglu_requant`` -- FP8 block-scale FC1, SwiGLU, 1x128 e4m3
   requantisation (PR #4069 pipeline step "FC1 with fused SwiGLU + 1x128
   quantization"; the fused epilogue reaches the same result as the unfused
   path, so this is the plain definition).
4. ``fc2`` -- FP8 block-scale FC2 (PR #4069 pipeline step "FC2").
5. ``combine`` -- weighted top-k reduction on the owner, one BF16 row per token
   (PR #4069 bullet "Grouped combine performs FP32 route reduction on the
   owner rank"); carried out in float64 and rounded once.
6. ``forward_mx`` -- BF16 activations x MXFP8 weights, BF16 output
   ("feat(moe_ep): MXFP8 x BF16 integration", PR #4604, Description).

Readings where the pages are silent (each is also listed with its reason in
the design notes of the repository):

* W13 rows: the first I rows are the gate projection, the next I the up
  projection; h = silu(gate) * up with silu(z) = z * sigmoid(z).
* Every scale is amax/448 stored as float32; a block with amax == 0 gets
  scale 0 and all-zero codes.
* Gate/up and FC2 outputs stay unrounded (float64) unless ``bf16_gateup``.
* Invalid routes (expert id outside [-1, E), a repeated expert within a token
  -- the lowest slot is kept --, a non-finite weight on an active route) set a
  status bit and are treated as masked.  Expert -1 is masked silently, its
  weight ignored even if NaN/inf.
* Within an expert, rows are in ascending route id r = t*K + k.
* With a row capacity, routes whose expert-major sorted position is at or
  beyond the capacity are dropped and flagged.
* Combine: sum over the valid slots in ascending k, one rounding to bfloat16.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against values the formats' definitions fix, library routines, brute-force
loops, exact rational arithmetic or closed forms (see ``PIN_STATUS``).
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .formats import (
    bf16_bits_to_f64,
    bf16_rne_bits,
    e4m3_decode,
    e5m2_decode,
    e4m3_encode_rne_sat,
    e8m0_decode,
)

STATUS_BAD_EXPERT = 1
STATUS_DUPLICATE = 2
STATUS_NONFINITE = 4
STATUS_CAPACITY = 8

PIN_STATUS = {
    # value: "pinned: <what fixes it> [<test module>::<test>, ...]"; the tests
    # named in brackets must exist (checked by test_every_oracle_function_has_a_pin)
    "formats.e4m3_decode": "pinned: exhaustive vs OCP bit-field values and torch.float8_e4m3fn "
                           "[test_oracle_formats::test_e4m3_decode_exhaustive_vs_torch, "
                           "test_oracle_formats::test_e4m3_decode_spec_values]",
    "formats.e5m2_decode": "pinned: exhaustive vs OCP bit-field values and torch.float8_e5m2 "
                           "[test_oracle_formats::test_e5m2_decode_exhaustive_vs_torch, "
                           "test_oracle_formats::test_e5m2_decode_spec_values]",
    "formats.bf16_bits_to_f64": "pinned: round trips of the bfloat16 rounding tests (exact widening) "
                                "[test_oracle_formats::test_bf16_rne_float32_inputs_vs_torch]",
    "formats.e8m0_decode": "pinned: exhaustive vs torch.float8_e8m0fnu "
                           "[test_oracle_formats::test_e8m0_decode_exhaustive_vs_torch]",
    "formats.e4m3_encode_rne_sat": "pinned: all midpoints +-1 ulp and random values vs torch cast "
                                   "[test_oracle_formats::test_e4m3_encode_midpoints_vs_torch, "
                                   "test_oracle_formats::test_e4m3_encode_float64_near_midpoints_vs_exact]",
    "formats.bf16_rne_bits": "pinned: vs torch bfloat16 cast (float32 inputs) and exact fractions "
                             "[test_oracle_formats::test_bf16_rne_float32_inputs_vs_torch, "
                             "test_oracle_formats::test_bf16_rne_float64_single_rounding]",
    "dequant_block128": "pinned: exact-rational FC1 and one-hot FC1/FC2 closed forms recompute it "
                        "[test_oracle_layer::test_fc1_exact_rational_tiny, test_oracle_layer::test_fc2_one_hot_closed_form]",
    "dequant_rows_1x128": "pinned: exact-rational FC1 recomputes it from the codes and scales "
                          "[test_oracle_layer::test_fc1_exact_rational_tiny]",
    "dequant_mx": "pinned: one-hot MX closed forms and per-route loops, e4m3 and e5m2 elements "
                  "[test_oracle_layer::test_forward_mx_one_hot_and_loop, "
                  "test_oracle_branches::test_forward_mx_e5m2_one_hot, "
                  "test_oracle_branches::test_mx_e5m2_pins_catch_element_type_mistakes]",
    "silu": "pinned: one-hot SwiGLU closed form g/(1+exp(-g))*u "
            "[test_oracle_layer::test_fc1_swiglu_one_hot_closed_form]",
    "requant_1x128": "pinned: requantisation invariants (scale = amax/448, a code at 448, error bound) "
                     "[test_oracle_layer::test_fc1_swiglu_one_hot_closed_form]",
    "fc1_gateup": "pinned: exact rational (fractions) on the tiny shape, one-hot closed form "
                  "[test_oracle_layer::test_fc1_exact_rational_tiny, test_oracle_layer::test_fc2_and_fc1_brute_force_loops]",
    "stage_quantize_1x128": "pinned: torch-cast cross-check, amax->448 invariant, error bound "
                            "[test_oracle_stage_compact::test_stage_quant_matches_torch_cast_and_invariants]",
    "stage_routes": "pinned: brute-force loops and masked-route semantics "
                    "[test_oracle_stage_compact::test_stage_routes_vs_brute_force, "
                    "test_oracle_stage_compact::test_masked_routes_accept_nonfinite_weights]",
    "compact": "pinned: brute-force loops [test_oracle_stage_compact::test_compact_vs_brute_force, "
               "test_oracle_stage_compact::test_compact_capacity_drops_tail_in_sorted_order]",
    "fc1_swiglu_requant": "pinned: exact rational FC1, one-hot closed forms, requant invariants "
                          "[test_oracle_layer::test_fc1_swiglu_one_hot_closed_form]",
    "fc1_swiglu_requant[bf16_gateup=True]": "pinned: one-hot closed form requant(silu(bf16(g)) * bf16(u)), "
                                            "misplaced rounding caught "
                                            "[test_oracle_branches::test_forward_fp8_bf16_gateup_one_hot, "
                                            "test_oracle_branches::test_bf16_gateup_pin_catches_misplaced_rounding]",
    "fc2": "pinned: brute-force loops, one-hot closed form "
           "[test_oracle_layer::test_fc2_and_fc1_brute_force_loops, test_oracle_layer::test_fc2_one_hot_closed_form]",
    "combine": "pinned: K=1 identity, power-of-two scaling, all-masked token, masked NaN "
               "[test_oracle_layer::test_combine_identities, test_oracle_layer::test_masked_nan_weights_do_not_change_output]",
    "forward_fp8": "pinned: pure-Python per-route loop on tiny shapes; dedup == per-route "
                   "[test_oracle_layer::test_forward_fp8_vs_per_route_loop, test_oracle_layer::test_dedup_equals_per_route_staging]",
    "forward_fp8[bf16_gateup=True]": "pinned: one-hot closed form through the whole layer "
                                     "[test_oracle_branches::test_forward_fp8_bf16_gateup_one_hot]",
    "forward_mx": "pinned: one-hot closed forms and pure-Python loop on tiny shapes "
                  "[test_oracle_layer::test_forward_mx_one_hot_and_loop]",
    "forward_mx[elem=e5m2]": "pinned: one-hot e5m2 W13/W2 closed forms with bit-field decode, per-route loop, "
                             "element-type mistakes caught "
                             "[test_oracle_branches::test_forward_mx_e5m2_one_hot, "
                             "test_oracle_branches::test_forward_mx_e5m2_per_route_loop, "
                             "test_oracle_branches::test_mx_e5m2_pins_catch_element_type_mistakes]",
}


# ----------------------------------------------------------------------------
# dequantisation helpers
# ----------------------------------------------------------------------------

def dequant_block128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """e4m3 codes [N, K] with one float32 scale per 128x128 block -> float64."""
    n, k = codes.shape
    s = np.repeat(np.repeat(np.asarray(scales, np.float64), 128, axis=0), 128, axis=1)
    return e4m3_decode(codes) * s[:n, :k]


def dequant_rows_1x128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """e4m3 codes [R, K] with one float32 scale per row per 128 columns."""
    s = np.repeat(np.asarray(scales, np.float64), 128, axis=1)
    return e4m3_decode(codes) * s


def dequant_mx(codes: np.ndarray, e8m0: np.ndarray, elem: str = "e4m3") -> np.ndarray:
    """MXFP8 codes [N, K] (elem "e4m3" or "e5m2") with one E8M0 scale per 32
    consecutive K elements."""
    s = np.repeat(e8m0_decode(e8m0), 32, axis=1)
    dec = e5m2_decode if elem == "e5m2" else e4m3_decode
    return dec(codes) * s


def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z); exp overflow for very negative z gives the limit -0."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


# ----------------------------------------------------------------------------
# 1. staging
# ----------------------------------------------------------------------------

def stage_quantize_1x128(x_bf16_bits: np.ndarray):
    """BF16 activations -> e4m3 codes + one float32 scale per row per 128 columns.

    For each 1x128 block: amax = max |x| (exact in float32), s = fl32(amax/448)
    (IEEE float32 division), q = RNE_sat_e4m3(fl32(x / s)); s == 0 -> q = 0.
    """
    x = bf16_bits_to_f64(x_bf16_bits).astype(np.float32)
    t, h = x.shape
    blk = x.reshape(t, h // 128, 128)
    amax = np.abs(blk).max(axis=2)
    s = (amax / np.float32(448.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (blk / s[:, :, None]).astype(np.float32)
    codes = e4m3_encode_rne_sat(v.astype(np.float64))
    codes = np.where((s == 0)[:, :, None], np.uint8(0), codes)
    return codes.reshape(t, h).astype(np.uint8), s


def stage_routes(topk_idx: np.ndarray, topk_w: np.ndarray, num_experts: int,
                 check_routes: bool = True):
    """Validate and mask routes.  Returns (idx int32 [T*K], w float32 [T*K], status).

    Masked slots get idx -1 and weight 0.  With ``check_routes`` false only the
    expert-id range is enforced (so no route can address a missing expert);
    duplicates and non-finite weights pass through.
    """
    idx = np.asarray(topk_idx, np.int64)
    w = np.asarray(topk_w, np.float32)
    t, k = idx.shape
    status = 0
    masked = idx == -1
    bad = (idx < -1) | (idx >= num_experts)
    if bad.any():
        status |= STATUS_BAD_EXPERT
    active = ~masked & ~bad
    if check_routes:
        dup = np.zeros_like(active)
        for j in range(1, k):
            for i in range(j):
                dup[:, j] |= active[:, j] & active[:, i] & (idx[:, j] == idx[:, i])
        if dup.any():
            status |= STATUS_DUPLICATE
        active &= ~dup
        nonfinite = active & ~np.isfinite(w)
        if nonfinite.any():
            status |= STATUS_NONFINITE
        active &= ~nonfinite
    out_idx = np.where(active, idx, -1).astype(np.int32).reshape(-1)
    out_w = np.where(active, w, np.float32(0.0)).astype(np.float32).reshape(-1)
    return out_idx, out_w, status


# ----------------------------------------------------------------------------
# 2. compaction
# ----------------------------------------------------------------------------

@dataclass
class Compaction:
    counts: np.ndarray  # int32 [E]
    offsets: np.ndarray  # int32 [E + 1]
    sorted_route: np.ndarray  # int32 [R]   route ids, expert-major, ascending within expert
    route_pos: np.ndarray  # int32 [T*K] position in sorted_route, -1 if not kept
    status: int


def compact(staged_idx: np.ndarray, num_experts: int, row_cap: Optional[int] = None) -> Compaction:
    idx = np.asarray(staged_idx, np.int64)
    valid = np.nonzero(idx >= 0)[0]
    order = valid[np.argsort(idx[valid], kind="stable")]
    status = 0
    if row_cap is not None and order.size > row_cap:
        order = order[:row_cap]
        status |= STATUS_CAPACITY
    counts = np.bincount(idx[order], minlength=num_experts).astype(np.int32)
    offsets = np.zeros(num_experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    route_pos = np.full(idx.size, -1, np.int32)
    route_pos[order] = np.arange(order.size, dtype=np.int32)
    return Compaction(counts, offsets, order.astype(np.int32), route_pos, status)


# ----------------------------------------------------------------------------
# 3-5. FC1 + SwiGLU + requant, FC2, combine
# ----------------------------------------------------------------------------

def requant_1x128(h: np.ndarray):
    """float64 h [R, I] -> e4m3 codes + float32 scales [R, I/128].

    s = fl32(amax / 448) with amax taken in float64; s == 0 -> zero codes;
    otherwise q = RNE_sat_e4m3(h / s).
    """
    r, n = h.shape
    blk = h.reshape(r, n // 128, 128)
    amax = np.abs(blk).max(axis=2) if r else np.zeros((0, n // 128))
    s = (amax / 448.0).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = blk / s.astype(np.float64)[:, :, None]
    codes = e4m3_encode_rne_sat(v)
    codes = np.where((s == 0)[:, :, None], np.uint8(0), codes)
    return codes.reshape(r, n).astype(np.uint8), s


def fc1_gateup(x_rows: np.ndarray, w13_codes: np.ndarray, w13_scale: np.ndarray) -> np.ndarray:
    """One expert: GU = X @ dequant(W13)^T, float64 [n, 2I]."""
    return x_rows @ dequant_block128(w13_codes, w13_scale).T


def fc1_swiglu_requant(x_rows: np.ndarray, w13_codes: np.ndarray, w13_scale: np.ndarray,
                       bf16_gateup: bool = False):
    """One expert: float64 activation rows [n, H] -> (h float64, codes, scales).

    GU = X @ W13^T over dequantised operands; gate = GU[:, :I], up = GU[:, I:];
    h = silu(gate) * up; then 1x128 requantisation.
    """
    gu = fc1_gateup(x_rows, w13_codes, w13_scale)
    if bf16_gateup:
        gu = bf16_bits_to_f64(bf16_rne_bits(gu))
    i = gu.shape[1] // 2
    h = silu(gu[:, :i]) * gu[:, i:]
    codes, scales = requant_1x128(h)
    return h, codes, scales


def fc2(h_rows: np.ndarray, w2_codes: np.ndarray, w2_scale: np.ndarray) -> np.ndarray:
    """One expert: float64 rows [n, I] @ dequant(W2)^T -> float64 [n, H]."""
    return h_rows @ dequant_block128(w2_codes, w2_scale).T


def combine(y: np.ndarray, route_pos: np.ndarray, staged_w: np.ndarray, tokens: int, top_k: int,
            token_ids: Optional[np.ndarray] = None) -> np.ndarray:
    """out[t] = bf16( sum_{k valid} w[t,k] * y[route_pos[t*K+k]] ), float64 sum.

    ``y`` is indexed by sorted position (rows absent from ``y`` are never
    read).  Returns uint16 bf16 bits [len(token_ids), H].
    """
    if token_ids is None:
        token_ids = np.arange(tokens)
    hdim = y.shape[1]
    acc = np.zeros((len(token_ids), hdim), np.float64)
    for j, t in enumerate(token_ids):
        for k in range(top_k):
            p = route_pos[t * top_k + k]
            if p >= 0:
                acc[j] += np.float64(staged_w[t * top_k + k]) * y[p]
    return bf16_rne_bits(acc)


@dataclass
class ForwardResult:
    out_bits: np.ndarray  # uint16 [len(tokens), H]
    token_ids: np.ndarray
    staged_idx: np.ndarray
    staged_w: np.ndarray
    status: int
    comp: Compaction
    xq: Optional[np.ndarray] = None
    xs: Optional[np.ndarray] = None
    hq: Optional[dict] = None  # sorted position -> codes [I]
    hs: Optional[dict] = None  # sorted position -> scales [I/128]
    y: Optional[dict] = None  # sorted position -> float64 [H]


def _rows_for_tokens(comp: Compaction, top_k: int, token_ids: Optional[np.ndarray]):
    """Sorted positions needed for the requested tokens (all positions if None)."""
    if token_ids is None:
        return np.arange(comp.sorted_route.size)
    want = np.zeros(comp.sorted_route.size, bool)
    for t in token_ids:
        for k in range(top_k):
            p = comp.route_pos[t * top_k + k]
            if p >= 0:
                want[p] = True
    return np.nonzero(want)[0]


def forward_fp8(x_bf16_bits, topk_idx, topk_w, w13, w13_scale, w2, w2_scale, *,
                row_cap: Optional[int] = None, check_routes: bool = True,
                token_ids: Optional[np.ndarray] = None, per_route_staging: bool = False,
                bf16_gateup: bool = False, prequant=None) -> ForwardResult:
    """FP8 e4m3 block-scale layer forward (steps 1-5).

    ``token_ids`` restricts FC1/FC2/combine to the routes of those tokens
    (each output row depends only on its own token's routes); compaction is
    always global.  ``prequant=(codes, scales)`` supplies already-quantised
    rows instead of quantising BF16 ``x_bf16_bits``.  ``per_route_staging``
    stages one copy of the token row per route before FC1 instead of one row
    per token (the deduplicated layout); the result is identical.
    """
    tokens, top_k = np.asarray(topk_idx).shape
    num_experts = w13.shape[0]
    if prequant is None:
        xq, xs = stage_quantize_1x128(x_bf16_bits)
    else:
        xq, xs = prequant
    sidx, sw, status = stage_routes(topk_idx, topk_w, num_experts, check_routes)
    comp = compact(sidx, num_experts, row_cap)
    status |= comp.status
    if per_route_staging:
        rq = np.repeat(xq, top_k, axis=0)  # row r = t*K + k holds token t
        rs = np.repeat(xs, top_k, axis=0)
    positions = _rows_for_tokens(comp, top_k, token_ids)
    hq, hs, yd = {}, {}, {}
    for e in range(num_experts):
        lo, hi = comp.offsets[e], comp.offsets[e + 1]
        pos = positions[(positions >= lo) & (positions < hi)]
        if pos.size == 0:
            continue
        routes = comp.sorted_route[pos]
        if per_route_staging:
            xr = dequant_rows_1x128(rq[routes], rs[routes])
        else:
            toks = routes // top_k
            xr = dequant_rows_1x128(xq[toks], xs[toks])
        _, codes, scales = fc1_swiglu_requant(xr, w13[e], w13_scale[e], bf16_gateup)
        hd = dequant_rows_1x128(codes, scales)
        ye = fc2(hd, w2[e], w2_scale[e])
        for j, p in enumerate(pos):
            hq[int(p)], hs[int(p)], yd[int(p)] = codes[j], scales[j], ye[j]
    tid = np.arange(tokens) if token_ids is None else np.asarray(token_ids)
    out = _combine_dict(yd, comp.route_pos, sw, top_k, tid, w2.shape[1])
    return ForwardResult(out, tid, sidx, sw, status, comp, xq, xs, hq, hs, yd)


def _combine_dict(yd: dict, route_pos, staged_w, top_k, token_ids, hdim):
    acc = np.zeros((len(token_ids), hdim), np.float64)
    for j, t in enumerate(token_ids):
        for k in range(top_k):
            p = int(route_pos[t * top_k + k])
            if p >= 0:
                acc[j] += np.float64(staged_w[t * top_k + k]) * yd[p]
    return bf16_rne_bits(acc)


def forward_mx(x_bf16_bits, topk_idx, topk_w, w13, w13_e8m0, w2, w2_e8m0, *,
               row_cap: Optional[int] = None, check_routes: bool = True,
               token_ids: Optional[np.ndarray] = None, elem: str = "e4m3") -> ForwardResult:
    """BF16 activations x MXFP8 (e4m3 or e5m2 codes + E8M0 per 32 along K) weights.

    Same pipeline as ``forward_fp8`` except: activations are used as exact
    BF16 values (no quantisation), weights are decoded with their E8M0
    scales, and h is rounded once to BF16 (RNE) instead of the 1x128 e4m3
    requantisation.
    """
    tokens, top_k = np.asarray(topk_idx).shape
    num_experts = w13.shape[0]
    x = bf16_bits_to_f64(x_bf16_bits)
    sidx, sw, status = stage_routes(topk_idx, topk_w, num_experts, check_routes)
    comp = compact(sidx, num_experts, row_cap)
    status |= comp.status
    positions = _rows_for_tokens(comp, top_k, token_ids)
    hb, yd = {}, {}
    for e in range(num_experts):
        lo, hi = comp.offsets[e], comp.offsets[e + 1]
        pos = positions[(positions >= lo) & (positions < hi)]
        if pos.size == 0:
            continue
        toks = comp.sorted_route[pos] // top_k
        w = dequant_mx(w13[e], w13_e8m0[e], elem)
        gu = x[toks] @ w.T
        i = w.shape[0] // 2
        h = silu(gu[:, :i]) * gu[:, i:]
        hbits = bf16_rne_bits(h)
        ye = bf16_bits_to_f64(hbits) @ dequant_mx(w2[e], w2_e8m0[e], elem).T
        for j, p in enumerate(pos):
            hb[int(p)], yd[int(p)] = hbits[j], ye[j]
    tid = np.arange(tokens) if token_ids is None else np.asarray(token_ids)
    out = _combine_dict(yd, comp.route_pos, sw, top_k, tid, w2.shape[1])
    return ForwardResult(out, tid, sidx, sw, status, comp, hq=hb, y=yd)
