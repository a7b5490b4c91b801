"""192-token ping-pong tiles (experts of 129-192 expected rows) against the
128-token LDS-ring tiles bit for bit, and against the float64 oracle.

All tactics compute every output with the same operations in the same
order, so the BF16 output, the FC1 codes and scales and the FC2 rows agree
bit for bit across tile sizes.  At 192 tokens a wave group holds 96 tokens: six
token blocks per wave, three token DMA instructions per wave and K-block,
the group's token scales from 64 + 32 lanes of two waves, and the
promotion threads of rows 96-127 idle.  The cases span ragged and masked
tokens, a K of 3 and 2 blocks, a K of one block, and the DeepSeek-V3-like
shape.
"""

import numpy as np
import pytest
import torch

from oracle import moe_ref as M
from synthetic import CONFIGS, MoEShape, make_layer_inputs
from tests.parity_util import assert_output_close

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mixture_experts_ffn_route_amd.harness import make_layer, run_forward, to_device


def _np(t):
    return t.detach().cpu().numpy()


def _run(shape, dev, expected_m, tokens=None):
    layer = make_layer(shape, dev, expected_m=expected_m)
    out = run_forward(layer, dev, tokens=tokens)
    torch.cuda.synchronize()
    I = shape.intermediate
    R = int(_np(layer.region("counts", torch.int32, (shape.experts,))).sum())
    res = (_np(out.view(torch.int16)).copy(), _np(layer.region("hq", torch.uint8))[:R * I].copy(),
           _np(layer.region("hs", torch.int32))[:R * (I // 128)].copy(),
           _np(layer.region("y", torch.int16))[:R * shape.hidden].copy(), layer.status())
    bm = layer.tactic()["block_m"]
    layer.close()
    return bm, res


_SHAPES = {"small": CONFIGS["small"], "odd": MoEShape(400, 384, 256, 4, 2, "topk"),
           "k1": MoEShape(400, 128, 128, 4, 2, "topk")}


@pytest.mark.parametrize("name,tokens,masked", [("small", None, 0.0), ("small", 301, 0.1), ("odd", None, 0.25),
                                                ("odd", 77, 0.0), ("k1", None, 0.1)])
def test_192_token_tiles_equal_128(name, tokens, masked):
    shape = _SHAPES[name]
    inp = make_layer_inputs(shape, seed=31, masked_fraction=masked)
    dev = to_device(inp)
    bm_a, a = _run(shape, dev, 160, tokens)
    bm_b, b = _run(shape, dev, 96, tokens)
    assert (bm_a, bm_b) == (192, 128)
    for nm, x, y in zip(("out", "hq", "hs", "y"), a[:4], b[:4]):
        assert np.array_equal(x, y), f"{nm}: 192- and 128-token tiles differ"
    assert a[4] == b[4]


@pytest.mark.slow
def test_192_token_tiles_dsv3_sampled():
    """T=640 of the DeepSeek-V3-like shape takes 192-token tiles by default
    (160 expected rows per expert); sampled tokens against the oracle."""
    base = CONFIGS["dsv3"]
    shape = MoEShape(640, base.hidden, base.intermediate, base.experts, base.top_k, base.routing)
    inp = make_layer_inputs(shape, seed=32)
    dev = to_device(inp)
    layer = make_layer(shape, dev)
    assert layer.tactic()["block_m"] == 192
    out = run_forward(layer, dev)
    torch.cuda.synchronize()
    rng = np.random.default_rng(640)
    tok = np.sort(rng.choice(640, size=12, replace=False))
    res = M.forward_fp8(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale,
                        token_ids=tok)
    assert layer.status() == 0
    got = _np(out.view(torch.int16)).view(np.uint16)
    assert_output_close(got[tok], res.out_bits, "dsv3 T=640 (192-token tiles)")
