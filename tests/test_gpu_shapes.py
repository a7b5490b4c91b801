"""Parity over a seeded spread of small layer shapes, through the C ABI.

The named configurations exercise K in {2, 6, 8} and E in {8, 32}; here every
supported top-k (1, 2, 4, 6, 8), expert counts from 1 to 1024, H and I from
one to nine 128-column blocks (odd block counts leave the last FC2 column
tile half full), token counts from 1 to 600 (one and several compaction workgroups), several FC2 tiles
per workgroup (each tile's output stores still in flight while the next
tile's first stages are awaited), masked routes and both weight formats are
compared with the float64 oracle:
the compaction bit for bit, the output within the layer tolerance.
"""

import numpy as np
import pytest
import torch

from oracle import moe_ref as M
from synthetic import MoEShape, make_layer_inputs
from tests.parity_util import assert_output_close

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mixture_experts_ffn_route_amd.harness import make_layer, run_forward, to_device


def _shapes():
    # (T, H, I, E, K, masked fraction, MXFP8 weights)
    table = [
        (1, 128, 128, 1, 1, 0.0, False),
        (7, 640, 384, 3, 1, 0.0, True),
        (130, 1152, 640, 9, 2, 0.3, False),
        (33, 384, 128, 257, 4, 0.0, False),    # > 256 experts
        (130, 256, 640, 16, 4, 0.0, True),
        (7, 1152, 256, 6, 6, 0.0, False),
        (33, 384, 640, 64, 6, 0.3, True),
        (130, 640, 640, 9, 8, 0.0, False),
        (33, 384, 384, 257, 8, 0.3, False),
        (1, 128, 256, 8, 8, 0.0, True),
        (130, 384, 128, 1024, 2, 0.0, False),  # the largest expert count
        (300, 256, 128, 33, 8, 0.3, False),    # 2400 routes: three compaction workgroups
        (600, 128, 128, 9, 8, 0.0, False),     # 4800 routes: five compaction workgroups
        (600, 256, 256, 12, 8, 0.3, True),
        # several FC2 tiles per workgroup, so a tile's first waits run while
        # the previous tile's output stores are in flight
        (128, 2048, 512, 256, 8, 0.3, False),  # 16-token tiles, 2048 FC2 tiles
        (40, 4096, 1024, 64, 8, 0.0, False),   # 16-token tiles, 1024 FC2 tiles
        (400, 4096, 384, 32, 8, 0.0, False),   # 128-token tiles, three-stage ring, 512 FC2 tiles
        # compaction over several workgroups: the largest expert count, and one route per token
        (1100, 128, 128, 1024, 2, 0.2, False),  # 2200 routes, 3 workgroups, 1024 experts
        (2500, 128, 256, 8, 1, 0.0, True),      # 2500 routes, 3 workgroups
    ]
    return [(MoEShape(T, H, I, E, K, "topk"), m, mx, 100 + i) for i, (T, H, I, E, K, m, mx) in enumerate(table)]


SHAPES = _shapes()


def _id(case):
    s, masked, mx, _ = case
    return f"T{s.tokens}-H{s.hidden}-I{s.intermediate}-E{s.experts}-K{s.top_k}-m{masked}-{'mx' if mx else 'fp8'}"


@pytest.mark.parametrize("case", SHAPES, ids=[_id(c) for c in SHAPES])
def test_shape_parity(case):
    shape, masked, mx, seed = case
    inp = make_layer_inputs(shape, seed=seed, weight_format="mxfp8" if mx else "fp8_block",
                            masked_fraction=masked)
    dev = to_device(inp)
    layer = make_layer(shape, dev, mx=mx)
    out = run_forward(layer, dev)
    torch.cuda.synchronize()
    args = (inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale)
    res = M.forward_mx(*args) if mx else M.forward_fp8(*args)
    E, K, T = shape.experts, shape.top_k, shape.tokens
    assert np.array_equal(layer.region("counts", torch.int32, (E,)).cpu().numpy(), res.comp.counts)
    R = int(res.comp.offsets[-1])
    assert np.array_equal(layer.region("sorted_route", torch.int32).cpu().numpy()[:R], res.comp.sorted_route)
    assert np.array_equal(layer.region("route_pos", torch.int32).cpu().numpy()[:T * K], res.comp.route_pos)
    assert layer.status() == res.status
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert_output_close(got, res.out_bits, _id(case))
