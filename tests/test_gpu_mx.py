"""Parity of the MXFP8-weight x BF16-activation path (through the C ABI)
with the float64 oracle's ``forward_mx``.

Bit-exact: staged routes, per-expert counts, offsets, sorted route ids and
their inverse, and the create-time weight and exponent tiles.  Within the
output tolerance of ``parity_util``: the BF16 layer output.  The two-term
e4m3 split the kernels feed to the scaled MFMA is checked against its
defining bounds: hi + lo reproduces each BF16 activation to 2^-8 of its
magnitude (plus a subnormal floor far below the block maximum).
"""

import numpy as np
import pytest
import torch

from oracle import moe_ref as M
from oracle.formats import e4m3_decode
from synthetic import CONFIGS, MoEShape, make_layer_inputs
from tests.parity_util import assert_output_close, bf16_bits_to_f64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mixture_experts_ffn_route_amd import _lib as L
    from mixture_experts_ffn_route_amd.harness import make_layer, run_forward, to_device


def _np(t):
    return t.detach().cpu().numpy()


def _bits(out):
    return _np(out.view(torch.int16)).view(np.uint16)


def _mx_inputs(shape, seed, elem="e4m3", **kw):
    return make_layer_inputs(shape, seed=seed, weight_format="mxfp8_e5m2" if elem == "e5m2" else "mxfp8", **kw)


def _elem(inp):
    return "e5m2" if inp.weight_format == "mxfp8_e5m2" else "e4m3"


def _gpu_run(inp, shape, **kw):
    dev = to_device(inp)
    layer = make_layer(shape, dev, mx=_elem(inp), **kw)
    out = run_forward(layer, dev)
    torch.cuda.synchronize()
    return layer, dev, out


def _oracle(inp, **kw):
    return M.forward_mx(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale,
                        elem=_elem(inp), **kw)


def _check_compaction(layer, res, shape, T):
    E, K = shape.experts, shape.top_k
    R = int(res.comp.offsets[-1])
    assert np.array_equal(_np(layer.region("counts", torch.int32, (E,))), res.comp.counts)
    assert np.array_equal(_np(layer.region("offsets", torch.int32, (E + 1,))), res.comp.offsets)
    assert np.array_equal(_np(layer.region("sorted_route", torch.int32))[:R], res.comp.sorted_route)
    assert np.array_equal(_np(layer.region("route_pos", torch.int32))[:T * K], res.comp.route_pos)


def _split_terms(codes_hi, codes_lo, words):
    """Values of the two e4m3 terms, one E8M0 pair per 32 columns."""
    n, c = codes_hi.shape
    e_hi = (words & 0xFF).astype(np.int64) - 127
    e_lo = ((words >> 8) & 0xFF).astype(np.int64) - 127
    hi = e4m3_decode(codes_hi) * np.exp2(np.repeat(e_hi, 32, axis=1).astype(np.float64))
    lo = e4m3_decode(codes_lo) * np.exp2(np.repeat(e_lo, 32, axis=1).astype(np.float64))
    return hi, lo, e_hi, e_lo


def _check_split(x, hi, lo, e_hi, label):
    """hi + lo within 2^-8 |x| plus a floor 2^-16 below the block maximum;
    the block maximum of |x| maps into [128, 256) under the hi exponent."""
    n, c = x.shape
    amax = np.abs(x).reshape(n, c // 32, 32).max(axis=2)
    err = np.abs(x - hi - lo)
    bound = np.exp2(-8.0) * np.abs(x) + np.exp2(-16.0) * np.repeat(amax, 32, axis=1)
    assert np.all(err <= bound), f"{label}: two-term split error above its bound"
    live = amax > 0
    scaled = amax[live] / np.exp2(e_hi[live].astype(np.float64))
    assert np.all((scaled >= 128) & (scaled < 256)), f"{label}: hi exponent does not map the block max into [128, 256)"


@pytest.mark.parametrize("elem", ["e4m3", "e5m2"])
@pytest.mark.parametrize("cfg,masked", [("tiny", 0.0), ("tiny", 0.25), ("small", 0.0), ("small", 0.1)])
def test_mx_layer_parity(cfg, masked, elem):
    shape = CONFIGS[cfg]
    inp = _mx_inputs(shape, 0, elem, masked_fraction=masked)
    layer, dev, out = _gpu_run(inp, shape)
    res = _oracle(inp)
    assert layer.status() == res.status == 0
    _check_compaction(layer, res, shape, shape.tokens)
    assert_output_close(_bits(out), res.out_bits, f"mx {elem} {cfg} masked={masked}")


def test_mx_activation_split_bounds():
    shape = CONFIGS["small"]
    inp = _mx_inputs(shape, 1)
    layer, dev, out = _gpu_run(inp, shape)
    T, H = shape.tokens, shape.hidden
    xq = _np(layer.region("xq", torch.uint8))
    plane = xq.size // 2
    hi_c = xq[:T * H].reshape(T, H)
    lo_c = xq[plane:plane + T * H].reshape(T, H)
    words = _np(layer.region("xs", torch.int32))[:T * (H // 32)].reshape(T, H // 32).view(np.uint32)
    hi, lo, e_hi, _ = _split_terms(hi_c, lo_c, words)
    _check_split(bf16_bits_to_f64(inp.x_bf16), hi, lo, e_hi, "x")


def test_mx_h_split_matches_bf16_h():
    """FC1's h (bf16 of silu(g)*up) is carried as hi + lo to the split bound."""
    shape = CONFIGS["small"]
    inp = _mx_inputs(shape, 2)
    layer, dev, out = _gpu_run(inp, shape)
    res = _oracle(inp)
    I = shape.intermediate
    R = int(res.comp.offsets[-1])
    hq = _np(layer.region("hq", torch.uint8))
    plane = hq.size // 2
    words = _np(layer.region("hs", torch.int32))[:R * (I // 32)].reshape(R, I // 32).view(np.uint32)
    hi, lo, e_hi, _ = _split_terms(hq[:R * I].reshape(R, I), hq[plane:plane + R * I].reshape(R, I), words)
    want = np.stack([bf16_bits_to_f64(res.hq[p]) for p in range(R)])
    got = hi + lo
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert rel < 5e-3, f"h relative error {rel:.3e}"
    # the split itself is exact to its bound around the GPU's own bf16 h
    scale = np.abs(want).reshape(R, I // 32, 32).max(axis=2)
    assert np.all(np.abs(got - want) <= 0.02 * np.abs(want) + 0.01 * np.repeat(scale, 32, axis=1) + 1e-30)


@pytest.mark.parametrize("elem", ["e4m3", "e5m2"])
@pytest.mark.parametrize("expected_m", [2, 12, 48, 4096])
def test_mx_tactics_agree_bit_exact(expected_m, elem):
    shape = CONFIGS["small"]
    inp = _mx_inputs(shape, 3, elem)
    dev = to_device(inp)
    outs = []
    for em in (expected_m, 96):
        layer = make_layer(shape, dev, expected_m=em, mx=elem)
        outs.append(_bits(run_forward(layer, dev)))
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("expected_m", [48, 96])  # 64-token lockstep tiles; 128-token ping-pong tiles
@pytest.mark.parametrize("tokens,elem", [(0, "e4m3"), (1, "e4m3"), (37, "e5m2"), (301, "e4m3"), (301, "e5m2")])
def test_mx_ragged_token_counts(tokens, elem, expected_m):
    shape = MoEShape(512, 2048, 768, 32, 6, "topk")
    inp = _mx_inputs(shape, 4, elem)
    dev = to_device(inp)
    layer = make_layer(shape, dev, expected_m=expected_m, max_rows=512, mx=elem)
    out = run_forward(layer, dev, tokens=tokens)
    torch.cuda.synchronize()
    res = M.forward_mx(inp.x_bf16[:tokens], inp.topk_idx[:tokens], inp.topk_w[:tokens], inp.w13, inp.w13_scale,
                       inp.w2, inp.w2_scale, elem=elem)
    _check_compaction(layer, res, shape, tokens)
    if tokens:
        assert_output_close(_bits(out), res.out_bits, f"mx T={tokens}")


def _retile_mx(w, fc1, inter):
    """NumPy statement of the MX operand tile order (see moe_weights.hip)."""
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
                    kbyte = kb * 128 + 16 * (lane // 16) + 64 * hilo
                    idx = kbyte[:, None] + np.arange(16)[None, :]
                    vals = w[:, np.minimum(rows, N - 1)[:, None], idx]
                    out[:, nt, kb, rb, hilo] = np.where(valid[None, :, None], vals, 0)
    return out.reshape(-1)


def _retile_mx_scales(s, fc1, inter):
    E, N, Q = s.shape
    K = Q * 32
    n_tiles = inter // 128 if fc1 else (N + 255) // 256
    kbs = K // 128
    out = np.full((E, n_tiles, kbs, 4, 64, 4), 127, np.uint8)
    lane = np.arange(64)
    for nt in range(n_tiles):
        for rb in range(16):
            if fc1:
                rows = (nt * 128 + rb * 16 if rb < 8 else inter + nt * 128 + (rb - 8) * 16) + (lane % 16)
            else:
                rows = nt * 256 + rb * 16 + (lane % 16)
            valid = rows < N
            for kb in range(kbs):
                vals = s[:, np.minimum(rows, N - 1), kb * 4 + lane // 16]  # [E, 64]
                out[:, nt, kb, rb // 4, :, rb % 4] = np.where(valid[None, :], vals, 127)
    return out.reshape(-1)


@pytest.mark.parametrize("shape,elem", [(CONFIGS["tiny"], "e4m3"), (MoEShape(16, 384, 256, 4, 2, "topk"), "e4m3"),
                                        (MoEShape(16, 384, 256, 4, 2, "topk"), "e5m2")])
def test_mx_create_time_tiling_is_exact(shape, elem):
    inp = _mx_inputs(shape, 8, elem)
    dev = to_device(inp)
    layer = make_layer(shape, dev, mx=elem)
    torch.cuda.synchronize()
    I = shape.intermediate
    assert np.array_equal(_np(layer.region("w13t", torch.uint8)), _retile_mx(inp.w13, True, I))
    assert np.array_equal(_np(layer.region("w2t", torch.uint8)), _retile_mx(inp.w2, False, I))
    assert np.array_equal(_np(layer.region("w13s", torch.uint8)), _retile_mx_scales(inp.w13_scale, True, I))
    assert np.array_equal(_np(layer.region("w2s", torch.uint8)), _retile_mx_scales(inp.w2_scale, False, I))
    out = run_forward(layer, dev)
    torch.cuda.synchronize()
    assert_output_close(_bits(out), _oracle(inp).out_bits, f"mx H={shape.hidden}")


@pytest.mark.slow
def test_mx_skewed_zipf_sampled():
    """The mixed-precision workload: DSV3-like shape, T=8192, Zipf(1.2)
    routing with 4 empty experts, MXFP8 weights x BF16 activations."""
    shape = CONFIGS["skewed"]
    inp = _mx_inputs(shape, 0)
    layer, dev, out = _gpu_run(inp, shape)
    rng = np.random.default_rng(0)
    tok = np.sort(rng.choice(shape.tokens, size=24, replace=False))
    res = _oracle(inp, token_ids=tok)
    assert layer.status() == 0
    _check_compaction(layer, res, shape, shape.tokens)
    assert_output_close(_bits(out)[tok], res.out_bits, "mx zipf T=8192")
    full = _bits(out)
    assert np.all((full & 0x7F80) != 0x7F80)


@pytest.mark.slow
def test_mx_e5m2_dsv3_sampled():
    """DSV3-like shape, T=4096, balanced routing, MXFP8 E5M2 weights x BF16."""
    shape = CONFIGS["dsv3"]
    inp = _mx_inputs(shape, 1, "e5m2")
    layer, dev, out = _gpu_run(inp, shape)
    rng = np.random.default_rng(1)
    tok = np.sort(rng.choice(shape.tokens, size=16, replace=False))
    res = _oracle(inp, token_ids=tok)
    assert layer.status() == 0
    _check_compaction(layer, res, shape, shape.tokens)
    assert_output_close(_bits(out)[tok], res.out_bits, "mx e5m2 dsv3 T=4096")


@pytest.mark.slow
def test_mx_dsv3_small_token_counts_sampled():
    """MXFP8 x BF16 at the DSV3-like shape (H=7168) for decode and mid token
    counts, each in the benchmark's launch configuration: T=8 and 64
    (16-token tiles) and T=512 (128-token tiles).  A token's output depends
    only on its own routes, so one oracle call over tokens sampled from the
    first 8, 64 and 512 serves the three layers."""
    base = CONFIGS["dsv3"]
    shape = MoEShape(512, base.hidden, base.intermediate, base.experts, base.top_k, base.routing)
    inp = _mx_inputs(shape, 6)
    dev = to_device(inp)
    rng = np.random.default_rng(6)
    tok = np.concatenate([np.arange(8), np.sort(rng.choice(np.arange(8, 64), 8, replace=False)),
                          np.sort(rng.choice(np.arange(64, 512), 8, replace=False))])
    res = _oracle(inp, token_ids=tok)
    for T, block_m in [(8, 16), (64, 16), (512, 128)]:
        sub = MoEShape(T, base.hidden, base.intermediate, base.experts, base.top_k, base.routing)
        layer = make_layer(sub, dev, mx="e4m3")
        assert layer.tactic()["block_m"] == block_m
        out = run_forward(layer, dev, tokens=T)
        torch.cuda.synchronize()
        assert layer.status() == 0
        sel = tok < T
        assert_output_close(_bits(out)[tok[sel]], res.out_bits[sel], f"mx dsv3 T={T}")
        if T == shape.tokens:
            _check_compaction(layer, res, shape, T)
        del layer, out
