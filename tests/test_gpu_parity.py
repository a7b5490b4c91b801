"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Bit-exact: staged e4m3 codes and scales, staged routes, status bits,
per-expert counts, offsets, sorted route ids and their inverse.  Within the
output tolerance of ``parity_util``: the BF16 layer output.  Shapes span
several tiles and ragged tails; the full-size workloads are checked on a
sample of tokens the oracle recomputes one by one.
"""

import numpy as np
import pytest
import torch

from oracle import moe_ref as M
from synthetic import CONFIGS, MoEShape, make_layer_inputs, make_routing
from tests.parity_util import assert_output_close, gemm_error_bound

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mixture_experts_ffn_route_amd import _lib as L
    from mixture_experts_ffn_route_amd.harness import make_layer, run_forward, to_device


def _np(t):
    return t.detach().cpu().numpy()


def _bits(out):
    return _np(out.view(torch.int16)).view(np.uint16)


def _gpu_run(inp, shape, **kw):
    dev = to_device(inp)
    layer = make_layer(shape, dev, **kw)
    out = run_forward(layer, dev)
    torch.cuda.synchronize()
    return layer, dev, out


def _check_compaction(layer, res, shape, T):
    E, K = shape.experts, shape.top_k
    counts = _np(layer.region("counts", torch.int32, (E,)))
    offsets = _np(layer.region("offsets", torch.int32, (E + 1,)))
    R = int(res.comp.offsets[-1])
    sorted_route = _np(layer.region("sorted_route", torch.int32))[:R]
    route_pos = _np(layer.region("route_pos", torch.int32))[:T * K]
    assert np.array_equal(counts, res.comp.counts)
    assert np.array_equal(offsets, res.comp.offsets)
    assert np.array_equal(sorted_route, res.comp.sorted_route)
    assert np.array_equal(route_pos, res.comp.route_pos)


def _check_stage(layer, res, shape, T):
    H, K = shape.hidden, shape.top_k
    xq = _np(layer.region("xq", torch.uint8))[:T * H].reshape(T, H)
    xs = _np(layer.region("xs", torch.float32))[:T * (H // 128)].reshape(T, H // 128)
    assert np.array_equal(xq, res.xq), "stage e4m3 codes differ"
    assert np.array_equal(xs.view(np.uint32), res.xs.view(np.uint32)), "stage scales differ"
    sidx = _np(layer.region("staged_idx", torch.int32))[:T * K]
    sw = _np(layer.region("staged_w", torch.float32))[:T * K]
    assert np.array_equal(sidx, res.staged_idx)
    assert np.array_equal(sw.view(np.uint32), res.staged_w.view(np.uint32))


def _check_requant(layer, res, shape):
    I = shape.intermediate
    R = int(res.comp.offsets[-1])
    if R == 0:
        return
    hq = _np(layer.region("hq", torch.uint8))[:R * I].reshape(R, I)
    hs = _np(layer.region("hs", torch.float32))[:R * (I // 128)].reshape(R, I // 128)
    want_q = np.stack([res.hq[p] for p in range(R)])
    want_s = np.stack([res.hs[p] for p in range(R)])
    same = np.mean(hq == want_q)
    assert same >= 0.99, f"only {same:.4f} of FC1 e4m3 codes agree"
    assert np.allclose(hs, want_s, rtol=2e-3, atol=0), "FC1 requant scales differ"
    assert np.all((hq & 0x7F) != 0x7F), "NaN code in FC1 output"


@pytest.mark.parametrize("cfg,masked", [("tiny", 0.0), ("tiny", 0.25), ("small", 0.0), ("small", 0.1)])
def test_layer_parity(cfg, masked):
    shape = CONFIGS[cfg]
    inp = make_layer_inputs(shape, seed=0, masked_fraction=masked)
    layer, dev, out = _gpu_run(inp, shape)
    res = M.forward_fp8(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale)
    assert layer.status() == res.status == 0
    _check_stage(layer, res, shape, shape.tokens)
    _check_compaction(layer, res, shape, shape.tokens)
    _check_requant(layer, res, shape)
    assert_output_close(_bits(out), res.out_bits, f"{cfg} masked={masked}")


@pytest.mark.parametrize("tokens", [0, 1, 37, 301])
def test_ragged_token_counts(tokens):
    shape = MoEShape(512, 2048, 768, 32, 6, "topk")
    inp = make_layer_inputs(shape, seed=3)
    dev = to_device(inp)
    layer = make_layer(shape, dev, expected_m=48, max_rows=512)
    out = run_forward(layer, dev, tokens=tokens)
    torch.cuda.synchronize()
    res = M.forward_fp8(inp.x_bf16[:tokens], inp.topk_idx[:tokens], inp.topk_w[:tokens], inp.w13, inp.w13_scale,
                        inp.w2, inp.w2_scale)
    # rows past the live count are staged as masked
    sidx = _np(layer.region("staged_idx", torch.int32))
    assert np.all(sidx[tokens * 6:512 * 6] == -1)
    _check_compaction(layer, res, shape, tokens)
    if tokens:
        assert_output_close(_bits(out), res.out_bits, f"T={tokens}")


def test_multi_workgroup_compaction_repeated():
    """Route compaction over several workgroups (whole tokens each, at most
    4096 routes: 682 tokens per workgroup at K=6) in consecutive stagings
    whose workgroup count changes (4, 2, 2, 1, 4).  The last workgroup to
    finish counting writes the header and the tile list and returns the
    arrival counter to zero; a counter left elsewhere would leave the next
    staging without its scan."""
    shape = MoEShape(2100, 256, 128, 16, 6, "topk")
    inp = make_layer_inputs(shape, seed=41, masked_fraction=0.2)
    dev = to_device(inp)
    layer = make_layer(shape, dev, max_rows=2100)
    for T in (2100, 700, 683, 1, 2100):
        out = run_forward(layer, dev, tokens=T)
        torch.cuda.synchronize()
        res = M.forward_fp8(inp.x_bf16[:T], inp.topk_idx[:T], inp.topk_w[:T], inp.w13, inp.w13_scale, inp.w2,
                            inp.w2_scale)
        _check_compaction(layer, res, shape, T)
        assert layer.status() == res.status, T
        sidx = _np(layer.region("staged_idx", torch.int32))
        assert np.all(sidx[T * 6:2100 * 6] == -1)
        assert_output_close(_bits(out), res.out_bits, f"T={T}")


def test_stage_codes_at_tiny_magnitudes():
    """The quantiser forms x / s from a reciprocal with one correction step
    for blocks with s >= 2^-90 and divides below that.  Rows scaled across
    that bound, and down to subnormal bf16, stage bit for bit as the oracle's
    IEEE quotient."""
    from oracle.formats import bf16_bits_to_f64, bf16_rne_bits
    shape = CONFIGS["small"]
    inp = make_layer_inputs(shape, seed=43)
    x = bf16_bits_to_f64(inp.x_bf16)
    scales = [1e-26, 3e-26, 1e-25, 4e-25, 1e-22, 1e-30, 1e-36, 1e-38, 3e-39]
    for i, f in enumerate(scales):
        x[i::len(scales) + 3] *= f  # a spread of rows at each magnitude, the rest as drawn
    inp.x_bf16 = bf16_rne_bits(x)
    layer, dev, out = _gpu_run(inp, shape)
    res = M.forward_fp8(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale)
    amax = np.abs(bf16_bits_to_f64(inp.x_bf16)).reshape(shape.tokens, -1, 128).max(axis=2)
    s = (amax / 448.0).astype(np.float32)
    assert np.any((s > 0) & (s < 2.0 ** -90)) and np.any((s >= 2.0 ** -90) & (s < 2.0 ** -80))
    _check_stage(layer, res, shape, shape.tokens)
    # the layer output of those rows: every block-scale product of the tiny
    # rows lies far below 2^-100 (their outputs are +0 or subnormal)
    _check_compaction(layer, res, shape, shape.tokens)
    assert_output_close(_bits(out), res.out_bits, "tiny magnitudes")


@pytest.mark.parametrize("expected_m", [None, 16, 4096])
def test_block_scales_across_the_float32_range(expected_m):
    """Block scales that differ by up to 2^120 within one output's sum, for
    both GEMMs, against the oracle.

    FC1: activation rows whose 1x128 blocks are scaled by 2^-40..2^20, rows
    with one block 2^-80 below the others (a scale product near 2^-100),
    rows with zero blocks and whole rows at 1e-26 (every product below
    2^-100).  FC2: the W13 block scales of some 128-column blocks of h are
    divided by 2^60 or 2^70, so those h blocks sit 2^120 to 2^140 below the
    rest of their row (h scales near or below the float32 normal range).
    Checked at the 16-, 128- and 256-token tiles."""
    from oracle.formats import bf16_bits_to_f64, bf16_rne_bits
    shape = CONFIGS["small"]
    T, H = shape.tokens, shape.hidden
    inp = make_layer_inputs(shape, seed=47)
    rng = np.random.default_rng(47)
    x = bf16_bits_to_f64(inp.x_bf16).reshape(T, H // 128, 128)
    x[0::5] *= np.exp2(rng.integers(-40, 21, (len(range(0, T, 5)), H // 128, 1)))
    x[1::5, 7] *= 2.0 ** -80
    x[2::5, ::3] = 0.0
    x[3::10] *= 1e-26
    inp.x_bf16 = bf16_rne_bits(x.reshape(T, H))
    s13 = inp.w13_scale.copy()
    ib = shape.intermediate // 128
    s13[:, 1, :] *= np.float32(2.0 ** -60)            # gate rows of h block 1
    s13[:, ib + 1, :] *= np.float32(2.0 ** -60)       # up rows of h block 1
    s13[:, 4, :] *= np.float32(2.0 ** -70)
    s13[:, ib + 4, :] *= np.float32(2.0 ** -70)
    inp.w13_scale = s13
    layer, dev, out = _gpu_run(inp, shape, expected_m=expected_m)
    res = M.forward_fp8(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale)
    assert layer.status() == 0
    _check_stage(layer, res, shape, T)
    assert_output_close(_bits(out), res.out_bits, f"wide block-scale range, expected_m={expected_m}")
    # the h blocks scaled down carry scales 2^120+ below their neighbours
    hs = np.stack([res.hs[p] for p in range(int(res.comp.offsets[-1]))])
    live = hs[:, 0] > 0
    assert np.all(hs[live, 1] < hs[live, 0] * 2.0 ** -100)


@pytest.mark.parametrize("pair", [(8, 48), (2, 24), (96, 4096), (128, 200), (8, 4096)])
def test_tactics_agree_bit_exact(pair):
    """Every token tile (16 to 256 tokens) computes the same bits: each
    output's arithmetic is tile-independent."""
    shape = CONFIGS["small"]
    inp = make_layer_inputs(shape, seed=1)
    dev = to_device(inp)
    outs = []
    for em in pair:
        layer = make_layer(shape, dev, expected_m=em)
        outs.append(_bits(run_forward(layer, dev)))
    assert np.array_equal(outs[0], outs[1])


def test_dedup_equals_per_route_staging_on_gpu():
    shape = CONFIGS["small"]
    inp = make_layer_inputs(shape, seed=2)
    dev = to_device(inp)
    a = _bits(run_forward(make_layer(shape, dev), dev))
    b = _bits(run_forward(make_layer(shape, dev, flags=L.MOE_FLAG_CHECK_ROUTES | L.MOE_FLAG_PER_ROUTE_STAGING),
                          dev))
    assert np.array_equal(a, b)


def test_deterministic_and_reusable():
    shape = CONFIGS["small"]
    inp = make_layer_inputs(shape, seed=4)
    dev = to_device(inp)
    layer = make_layer(shape, dev)
    a = _bits(run_forward(layer, dev))
    # poison the intermediate buffers; a second forward must not read stale data
    layer.region("y", torch.uint8).fill_(0xFF)
    layer.region("hq", torch.uint8).fill_(0x7F)
    b = _bits(run_forward(layer, dev))
    assert np.array_equal(a, b)


def test_route_checker_status_bits():
    shape = CONFIGS["tiny"]
    inp = make_layer_inputs(shape, seed=5)
    idx = inp.topk_idx.copy()
    w = inp.topk_w.copy()
    idx[0, 1] = 8          # out of range
    idx[1, 0] = -7         # out of range
    idx[2, 1] = idx[2, 0]  # duplicate
    w[3, 0] = np.nan       # non-finite on an active route
    w[4, 1] = np.inf
    inp.topk_idx, inp.topk_w = idx, w
    layer, dev, out = _gpu_run(inp, shape)
    res = M.forward_fp8(inp.x_bf16, idx, w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale)
    want = L.MOE_DEV_BAD_EXPERT | L.MOE_DEV_DUPLICATE | L.MOE_DEV_NONFINITE
    assert res.status == want
    assert layer.status() == want
    _check_stage(layer, res, shape, shape.tokens)
    _check_compaction(layer, res, shape, shape.tokens)
    assert_output_close(_bits(out), res.out_bits, "route checker")
    # with checks off only the id bounds are enforced
    dev2 = to_device(inp)
    layer2 = make_layer(shape, dev2, flags=0)
    run_forward(layer2, dev2)
    torch.cuda.synchronize()
    assert layer2.status() == L.MOE_DEV_BAD_EXPERT
    res2 = M.forward_fp8(inp.x_bf16, idx, w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale, check_routes=False)
    _check_compaction(layer2, res2, shape, shape.tokens)


def test_capacity_overflow_drops_tail():
    shape = CONFIGS["small"]
    inp = make_layer_inputs(shape, seed=6)
    layer, dev, out = _gpu_run(inp, shape, capacity_factor=0.5)
    cap = int(np.ceil(0.5 * 512 * 6))
    res = M.forward_fp8(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale,
                        row_cap=cap)
    assert res.status == L.MOE_DEV_CAPACITY and layer.status() == L.MOE_DEV_CAPACITY
    _check_compaction(layer, res, shape, shape.tokens)
    assert_output_close(_bits(out), res.out_bits, "capacity 0.5")


def test_prequantised_rows_match_bf16_staging():
    shape = CONFIGS["small"]
    inp = make_layer_inputs(shape, seed=7)
    xq, xs = M.stage_quantize_1x128(inp.x_bf16)  # "received" rows, already e4m3
    dev = to_device(inp)
    layer = make_layer(shape, dev)
    a = _bits(run_forward(layer, dev))
    xq_t = torch.from_numpy(xq).cuda()
    xs_t = torch.from_numpy(xs).cuda()
    b = _bits(run_forward(layer, dev, x=xq_t, x_scale=xs_t))
    assert np.array_equal(a, b)


def _sampled_full_size(shape, seed, n_sample, label):
    inp = make_layer_inputs(shape, seed=seed)
    layer, dev, out = _gpu_run(inp, shape)
    T = shape.tokens
    rng = np.random.default_rng(seed)
    tok = np.sort(rng.choice(T, size=n_sample, replace=False))
    res = M.forward_fp8(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale,
                        token_ids=tok)
    assert layer.status() == 0
    _check_compaction(layer, res, shape, T)
    got = _bits(out)[tok]
    assert_output_close(got, res.out_bits, label)
    # every output is finite and no live token row is left unwritten
    full = _bits(out)
    assert np.all((full & 0x7F80) != 0x7F80)


@pytest.mark.slow
def test_dsv3_shape_sampled():
    _sampled_full_size(CONFIGS["dsv3"], 0, 24, "dsv3 T=4096")


@pytest.mark.slow
@pytest.mark.parametrize("tokens", [512, 32768])
def test_dsv3_sweep_points_sampled(tokens):
    """Token-sweep points of the DSV3-like shape in the benchmark's launch
    configuration: T=512 (128-token tiles, 56 K-blocks, one compaction
    workgroup for each 1024 routes: four) and T=32768 (256-token tiles, 256
    compaction workgroups, 262144 route rows, 3.76 GB of FC2 rows)."""
    base = CONFIGS["dsv3"]
    shape = MoEShape(tokens, base.hidden, base.intermediate, base.experts, base.top_k, base.routing)
    _sampled_full_size(shape, 3, 16, f"dsv3 T={tokens}")


@pytest.mark.slow
def test_skewed_zipf_sampled():
    _sampled_full_size(CONFIGS["skewed"], 0, 24, "zipf T=8192")


@pytest.mark.slow
def test_dsv3_decode_sampled():
    """The DSV3-like shape at decode token counts, each in the launch
    configuration the benchmark uses for it: 16- and 32-token tiles, where
    every workgroup streams three or four FC2 tiles back to back (each tile's
    output stores still in flight while the next tile's first stages are
    awaited).  A token's output depends only on its own routes, so one
    oracle call over tokens sampled from the first 8, 64 and 100 serves all
    three layers."""
    base = CONFIGS["dsv3"]
    shape = MoEShape(100, base.hidden, base.intermediate, base.experts, base.top_k, base.routing)
    inp = make_layer_inputs(shape, seed=5)
    dev = to_device(inp)
    rng = np.random.default_rng(5)
    tok = np.concatenate([np.arange(8), np.sort(rng.choice(np.arange(8, 64), 12, replace=False)),
                          np.sort(rng.choice(np.arange(64, 100), 8, replace=False))])
    res = M.forward_fp8(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale,
                        token_ids=tok)
    for T, block_m in [(8, 16), (64, 16), (100, 32)]:
        sub = MoEShape(T, base.hidden, base.intermediate, base.experts, base.top_k, base.routing)
        layer = make_layer(sub, dev)
        assert layer.tactic()["block_m"] == block_m
        out = run_forward(layer, dev, tokens=T)
        torch.cuda.synchronize()
        assert layer.status() == 0
        sel = tok < T
        assert_output_close(_bits(out)[tok[sel]], res.out_bits[sel], f"dsv3 T={T}")
        if T == shape.tokens:
            _check_compaction(layer, res, shape, T)
        del layer, out


def _retile(w, fc1, inter):
    """NumPy statement of the 16x16x128 weight tile order (see moe_weights.hip)."""
    E, N, K = w.shape
    n_tiles = inter // 128 if fc1 else (N + 255) // 256
    kbs = K // 128
    out = np.zeros((E, n_tiles, kbs, 16, 2, 64, 16), np.uint8)
    lane = np.arange(64)
    for nt in range(n_tiles):
        for rb in range(16):
            if fc1:
                rows = (nt * 128 + rb * 16 if rb < 8 else inter + nt * 128 + (rb - 8) * 16) + (lane % 16)
            else:
                rows = nt * 256 + rb * 16 + (lane % 16)
            valid = rows < N
            for kb in range(kbs):
                for hilo in range(2):
                    kbyte = kb * 128 + 32 * (lane // 16) + 16 * hilo
                    idx = kbyte[:, None] + np.arange(16)[None, :]
                    vals = w[:, np.minimum(rows, N - 1)[:, None], idx]  # [E, 64, 16]
                    out[:, nt, kb, rb, hilo] = np.where(valid[None, :, None], vals, 0)
    return out.reshape(-1)


@pytest.mark.parametrize("shape,expected_m", [(CONFIGS["tiny"], None), (MoEShape(16, 384, 256, 4, 2, "topk"), None),
                                              (MoEShape(16, 384, 256, 4, 2, "topk"), 200),
                                              (MoEShape(16, 256, 128, 8, 2, "topk"), 1000)])
def test_create_time_weight_tiling_is_exact(shape, expected_m):
    inp = make_layer_inputs(shape, seed=8)
    dev = to_device(inp)
    layer = make_layer(shape, dev, expected_m=expected_m)
    torch.cuda.synchronize()
    w13t = _np(layer.region("w13t", torch.uint8))
    w2t = _np(layer.region("w2t", torch.uint8))
    assert layer.tactic()["tile_order"] == 0
    assert np.array_equal(w13t, _retile(inp.w13, True, shape.intermediate))
    assert np.array_equal(w2t, _retile(inp.w2, False, shape.intermediate))
    run = run_forward(layer, dev)
    torch.cuda.synchronize()
    res = M.forward_fp8(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale)
    assert_output_close(_bits(run), res.out_bits, f"H={shape.hidden}")


@pytest.mark.parametrize("cfg,expected_m", [("tiny", None), ("small", None), ("small", 4096)])
def test_unfused_fc1_equals_fused(cfg, expected_m):
    """The unfused FC1 (FP32 gate/up rows, then a separate SwiGLU + 1x128
    requant kernel) gives the fused epilogue's codes, scales and output bit
    for bit, and its gate/up rows match the oracle's FC1 GEMM alone."""
    shape = CONFIGS[cfg]
    inp = make_layer_inputs(shape, seed=11)
    dev = to_device(inp)
    fused = make_layer(shape, dev, expected_m=expected_m)
    a = _bits(run_forward(fused, dev))
    unf = make_layer(shape, dev, expected_m=expected_m, flags=L.MOE_FLAG_CHECK_ROUTES | L.MOE_FLAG_UNFUSED_FC1)
    b = _bits(run_forward(unf, dev))
    torch.cuda.synchronize()
    I, H = shape.intermediate, shape.hidden
    R = int(_np(fused.region("offsets", torch.int32, (shape.experts + 1,)))[-1])
    assert np.array_equal(_np(fused.region("hq", torch.uint8))[:R * I], _np(unf.region("hq", torch.uint8))[:R * I])
    assert np.array_equal(_np(fused.region("hs", torch.int32))[:R * I // 128],
                          _np(unf.region("hs", torch.int32))[:R * I // 128])
    assert np.array_equal(a, b)
    # gate/up rows against the float64 GEMM of the staged rows
    res = M.forward_fp8(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale)
    gu = _np(unf.region("gateup", torch.float32))[:R * 2 * I].reshape(R, 2 * I).astype(np.float64)
    xd = M.dequant_rows_1x128(res.xq, res.xs)
    offs = res.comp.offsets
    for e in range(shape.experts):
        lo, hi = offs[e], offs[e + 1]
        if hi == lo:
            continue
        toks = res.comp.sorted_route[lo:hi] // shape.top_k
        want = M.fc1_gateup(xd[toks], inp.w13[e], inp.w13_scale[e])
        # the GEMM's accumulation error bound (parity_util.gemm_error_bound,
        # from the MFMA's measured accumulation error); index or scale
        # mistakes give errors of the order of the values themselves
        err = np.abs(gu[lo:hi] - want)
        bound = gemm_error_bound(xd[toks], M.dequant_block128(inp.w13[e], inp.w13_scale[e]))
        assert np.all(err <= bound), f"expert {e}: {np.max(err / bound):.3f} of the bound"


@pytest.mark.parametrize("cfg,expected_m", [("tiny", None), ("small", None), ("small", 48)])
def test_unfused_bf16_gateup_against_oracle(cfg, expected_m):
    """MOE_FLAG_BF16_GATEUP: the unfused FC1 stores gate/up rounded to BF16
    before the SwiGLU, the pages' unfused reference; compared with the
    oracle's forward_fp8(bf16_gateup=True).  The BF16 gate/up values equal the
    oracle's FC1 rounded to BF16 except where the FP32 GEMM result and the
    exact one round to neighbouring BF16 values (one BF16 ulp apart)."""
    shape = CONFIGS[cfg]
    inp = make_layer_inputs(shape, seed=13)
    dev = to_device(inp)
    layer = make_layer(shape, dev, expected_m=expected_m,
                       flags=L.MOE_FLAG_CHECK_ROUTES | L.MOE_FLAG_UNFUSED_FC1 | L.MOE_FLAG_BF16_GATEUP)
    out = _bits(run_forward(layer, dev))
    torch.cuda.synchronize()
    assert layer.status() == 0
    res = M.forward_fp8(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale,
                        bf16_gateup=True)
    assert_output_close(out, res.out_bits, f"{cfg} bf16 gate/up")
    I = shape.intermediate
    R = int(res.comp.offsets[-1])
    gu = _np(layer.region("gateup", torch.int16))[:R * 2 * I].view(np.uint16).reshape(R, 2 * I)
    xd = M.dequant_rows_1x128(res.xq, res.xs)
    offs = res.comp.offsets
    from oracle.formats import bf16_bits_to_f64, bf16_rne_bits
    same = total = 0
    for e in range(shape.experts):
        lo, hi = offs[e], offs[e + 1]
        if hi == lo:
            continue
        toks = res.comp.sorted_route[lo:hi] // shape.top_k
        exact = M.fc1_gateup(xd[toks], inp.w13[e], inp.w13_scale[e])
        want = bf16_rne_bits(exact)
        got = gu[lo:hi]
        same += int(np.sum(got == want))
        total += got.size
        # the GEMM's error bound plus the GPU's BF16 rounding of its FP32
        # value (half an ulp: 2^-8 relative)
        g = bf16_bits_to_f64(got)
        bound = gemm_error_bound(xd[toks], M.dequant_block128(inp.w13[e], inp.w13_scale[e]))
        assert np.all(np.abs(g - exact) <= bound + 1.01 * 2.0 ** -8 * (np.abs(g) + bound)), f"expert {e}"
    assert same >= 0.95 * total, f"only {same}/{total} gate/up values equal the oracle's BF16 rounding"
    # h codes: the oracle's from BF16 gate/up
    hq = _np(layer.region("hq", torch.uint8))[:R * I].reshape(R, I)
    want_hq = np.stack([res.hq[p] for p in range(R)])
    assert np.mean(hq == want_hq) >= 0.99


def test_profile_mask_times_selected_kernels():
    """Events are recorded only around the selected kernel classes."""
    shape = CONFIGS["tiny"]
    inp = make_layer_inputs(shape, seed=12)
    dev = to_device(inp)
    layer = make_layer(shape, dev)
    layer.profile(True, kernels=("fc1",))
    for _ in range(3):
        run_forward(layer, dev)
    prof = layer.profile_read()
    assert prof["fc1"][1] == 3 and prof["fc1"][0] > 0
    assert all(n == 0 for k, (ms, n) in prof.items() if k != "fc1")
    layer.profile(True)
    run_forward(layer, dev)
    prof = layer.profile_read()
    assert prof["stage"][1] == 1 and prof["fc2"][1] == 1 and prof["combine"][1] == 1
    layer.profile(False)
    with pytest.raises(L.MoEError):
        L.moe_profile_enable(layer.handle, 1 << 7)
