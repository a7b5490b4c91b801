"""The streaming FP8 GEMM kernel (64-token tiles of two column tiles:
weights loaded straight into a register ring two K-blocks deep; FC2 by
default, FC1 too with MOE_FLAG_STREAM_FC1) against the LDS-ring kernel
(MOE_FLAG_NO_STREAM) bit for bit, and against the float64 oracle.

Both kernels compute every output with the same operations in the same order
(same MFMA inputs, same block-scale promotion records, same epilogue), so the
BF16 output, the FC1 codes and scales and the FC2 rows must agree bit for
bit.  The cases span ragged tails, masked routes, skewed routing, an odd
number of 128-column blocks of H (the last FC2 column tile half valid), a K
of one ring depth (each tile's loads run straight into the next tile's), a
GEMM whose column tiles do not pair up (it keeps the LDS-ring kernel), and
many tiles per workgroup (the load stream carried across tiles).
"""

import numpy as np
import pytest
import torch

from oracle import moe_ref as M
from synthetic import CONFIGS, MoEShape, make_layer_inputs
from tests.parity_util import assert_output_close

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mixture_experts_ffn_route_amd import _lib as L
    from mixture_experts_ffn_route_amd.harness import make_layer, run_forward, to_device


def _np(t):
    return t.detach().cpu().numpy()


def _bits(out):
    return _np(out.view(torch.int16)).view(np.uint16)


def _run(shape, dev, expected_m, flags, tokens=None):
    layer = make_layer(shape, dev, expected_m=expected_m, flags=flags)
    out = run_forward(layer, dev, tokens=tokens)
    torch.cuda.synchronize()
    I = shape.intermediate
    R = int(_np(layer.region("counts", torch.int32, (shape.experts,))).sum())
    hq = _np(layer.region("hq", torch.uint8))[:R * I].copy()
    hs = _np(layer.region("hs", torch.float32))[:R * (I // 128)].copy()
    y = _np(layer.region("y", torch.int16))[:R * shape.hidden].copy()
    tac = layer.tactic()
    status = layer.status()
    res = (_bits(out).copy(), hq, hs.view(np.uint32), y, status)
    layer.close()
    return tac, res


S1 = L.MOE_FLAG_STREAM_FC1 if torch.cuda.is_available() else 0


def _compare(shape, inp, expected_m, want_depths, tokens=None, flags=0):
    dev = to_device(inp)
    tac_s, got = _run(shape, dev, expected_m, L.MOE_FLAG_CHECK_ROUTES | flags, tokens)
    tac_r, ref = _run(shape, dev, expected_m, L.MOE_FLAG_CHECK_ROUTES | L.MOE_FLAG_NO_STREAM, tokens)
    assert (tac_s["stream_depth_fc1"], tac_s["stream_depth_fc2"]) == want_depths, tac_s
    assert (tac_r["stream_depth_fc1"], tac_r["stream_depth_fc2"]) == (0, 0)
    assert tac_s["block_m"] == tac_r["block_m"]
    for name, a, b in zip(("out", "hq", "hs", "y"), got[:4], ref[:4]):
        assert np.array_equal(a, b), f"{name}: streaming and LDS-ring kernels differ"
    assert got[4] == ref[4]
    return tac_s


@pytest.mark.parametrize("fc1", [False, True])
@pytest.mark.parametrize("masked", [0.0, 0.1])
def test_stream_equals_lds_ring(masked, fc1):
    shape = CONFIGS["small"]  # FC1: 16 K-blocks, 6 column tiles; FC2: 6 K-blocks, 8 column tiles
    inp = make_layer_inputs(shape, seed=11, masked_fraction=masked)
    tac = _compare(shape, inp, 48, (2 if fc1 else 0, 2), flags=S1 if fc1 else 0)
    assert tac["block_m"] == 64


@pytest.mark.parametrize("expected_m", [24, 96])
def test_stream_only_at_64_token_tiles(expected_m):
    shape = CONFIGS["small"]
    inp = make_layer_inputs(shape, seed=11)
    _compare(shape, inp, expected_m, (0, 0), flags=S1)


@pytest.mark.parametrize("tokens", [0, 1, 37, 301])
def test_stream_ragged_token_counts(tokens):
    shape = CONFIGS["small"]
    inp = make_layer_inputs(shape, seed=12)
    _compare(shape, inp, 48, (2, 2), tokens=tokens, flags=S1)


def test_stream_many_tiles_per_workgroup():
    """8192 tokens at 64-token tiles: ~800 row tiles x 3 FC1 column pairs and
    x 4 FC2 column pairs, some 10 tiles per workgroup, each tile's first
    loads issued by the one before."""
    base = CONFIGS["small"]
    shape = MoEShape(8192, base.hidden, base.intermediate, base.experts, base.top_k, base.routing)
    inp = make_layer_inputs(shape, seed=13, masked_fraction=0.05)
    _compare(shape, inp, 48, (2, 2), flags=S1)


def test_stream_skewed_routing():
    base = CONFIGS["small"]
    shape = MoEShape(2048, base.hidden, base.intermediate, base.experts, base.top_k, "zipf")
    inp = make_layer_inputs(shape, seed=14)
    _compare(shape, inp, 64, (0, 2))
    _compare(shape, inp, 64, (2, 2), flags=S1)


@pytest.mark.parametrize("shape,depths", [(MoEShape(200, 384, 256, 4, 2, "topk"), (0, 2)),
                                          (MoEShape(200, 256, 256, 4, 2, "topk"), (2, 0))])
def test_stream_odd_column_blocks_and_short_k(shape, depths):
    """H = 384: FC2's second column tile has 128 valid columns of H; FC1's K
    of 3 blocks runs the LDS-ring kernel, FC2's K of 2 blocks (I = 256) the
    streaming kernel, one ring depth per tile.  H = 256: FC1 streams (K of
    2 blocks, 2 column tiles), FC2's single column tile keeps the LDS ring."""
    inp = make_layer_inputs(shape, seed=15, masked_fraction=0.1)
    _compare(shape, inp, 64, depths, flags=S1)


def test_stream_against_oracle():
    shape = CONFIGS["small"]
    inp = make_layer_inputs(shape, seed=16, masked_fraction=0.1)
    res = M.forward_fp8(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale)
    dev = to_device(inp)
    for em, flags in ((48, 0), (64, S1)):
        layer = make_layer(shape, dev, expected_m=em, flags=L.MOE_FLAG_CHECK_ROUTES | flags)
        assert layer.tactic()["stream_depth_fc2"] > 0
        assert (layer.tactic()["stream_depth_fc1"] > 0) == (flags != 0)
        out = run_forward(layer, dev)
        torch.cuda.synchronize()
        assert layer.status() == res.status
        assert_output_close(_bits(out), res.out_bits, f"stream em={em}")
        layer.close()


@pytest.mark.slow
@pytest.mark.parametrize("tokens,expected_m,block_m", [(256, None, 64), (512, 64, 64)])
def test_stream_dsv3_sampled(tokens, expected_m, block_m):
    """The DSV3-like shape at the streaming kernel's token counts (56 FC1 and
    16 FC2 K-blocks, 8 FC1 and 14 FC2 column pairs), against the oracle on
    sampled tokens and against the LDS-ring kernels bit for bit."""
    base = CONFIGS["dsv3"]
    shape = MoEShape(tokens, base.hidden, base.intermediate, base.experts, base.top_k, base.routing)
    inp = make_layer_inputs(shape, seed=17)
    em = expected_m or max(1, tokens * shape.top_k // shape.experts)
    _compare(shape, inp, em, (0, 2))
    tac = _compare(shape, inp, em, (2, 2), flags=S1)
    assert tac["block_m"] == block_m
    dev = to_device(inp)
    layer = make_layer(shape, dev, expected_m=em)
    out = run_forward(layer, dev)
    torch.cuda.synchronize()
    rng = np.random.default_rng(tokens)
    tok = np.sort(rng.choice(tokens, size=12, replace=False))
    res = M.forward_fp8(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale,
                        token_ids=tok)
    assert layer.status() == 0
    assert_output_close(_bits(out)[tok], res.out_bits, f"stream dsv3 T={tokens}")
