"""The persistent FC1->FC2 launch (MOE_FLAG_PERSISTENT_FFN) against the two
launches, through the C ABI.

Every output element runs the same arithmetic in both forms, so the
persistent launch must reproduce the h codes, the h scales, the FC2 rows and
the layer output bit for bit; the two-launch path is held to the float64
oracle by test_gpu_parity.py, and one case here is checked against the
oracle directly.  After a forward every listed row tile's readiness counter
holds its FC1 column-tile count (I/128) and no wait has timed out.
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


def _flags(*extra):
    f = L.MOE_FLAG_CHECK_ROUTES | L.MOE_FLAG_PERSISTENT_FFN
    for x in extra:
        f |= x
    return f


def _shape(name):
    return MoEShape(40, 384, 256, 4, 2, "topk") if name == "odd" else CONFIGS[name]


def _compare(shape, sep, per, dev, tokens=None):
    a = _bits(run_forward(sep, dev, tokens=tokens))
    b = _bits(run_forward(per, dev, tokens=tokens))
    torch.cuda.synchronize()
    I, E = shape.intermediate, shape.experts
    R = int(_np(sep.region("offsets", torch.int32, (E + 1,)))[-1])
    assert R == int(_np(per.region("offsets", torch.int32, (E + 1,)))[-1])
    assert np.array_equal(_np(sep.region("hq", torch.uint8))[:R * I], _np(per.region("hq", torch.uint8))[:R * I])
    assert np.array_equal(_np(sep.region("hs", torch.int32))[:R * I // 128],
                          _np(per.region("hs", torch.int32))[:R * I // 128])
    H = shape.hidden
    assert np.array_equal(_np(sep.region("y", torch.int16))[:R * H], _np(per.region("y", torch.int16))[:R * H])
    assert np.array_equal(a, b), f"{int(np.sum(a != b))} of {a.size} output bits differ"
    status = per.status()
    assert not status & L.MOE_DEV_WAIT_TIMEOUT, "an FC2 tile timed out waiting for its FC1 rows"
    assert status == sep.status()
    m_tiles = int(_np(per.region("status", torch.int32, (8,)))[3])
    ready = _np(per.region("ready", torch.int32))[:m_tiles]
    assert np.all(ready == I // 128), ready
    return a


CASES = [
    # (shape, expected_m, masked fraction, extra flags)
    ("tiny", None, 0.0, ()),
    ("small", None, 0.25, ()),      # 128-row tiles, fully and partly masked tokens
    ("small", 8, 0.0, ()),          # 16-row tiles
    ("small", 24, 0.25, ()),        # 32-row tiles
    ("small", 48, 0.0, ()),         # 64-row tiles
    ("small", 4096, 0.0, ()),       # 128-row persistent tiles against the 256-row ping-pong launches
    ("odd", None, 0.25, ()),        # H = 384
    ("small", None, 0.25, ("fused",)),  # with the fused last-arriver combine
]


@pytest.mark.parametrize("name,expected_m,masked,extra", CASES)
def test_persistent_equals_two_launches(name, expected_m, masked, extra):
    shape = _shape(name)
    inp = make_layer_inputs(shape, seed=31, masked_fraction=masked)
    dev = to_device(inp)
    more = [L.MOE_FLAG_FUSED_COMBINE] if "fused" in extra else []
    sep = make_layer(shape, dev, expected_m=expected_m)
    per = make_layer(shape, dev, expected_m=expected_m, flags=_flags(*more))
    # the persistent form stops at 128-row tiles; the two launches it is
    # compared with may use 256 (the ping-pong kernel): every tile computes
    # the same bits
    assert per.tactic()["block_m"] == min(sep.tactic()["block_m"], 128)
    _compare(shape, sep, per, dev)


def test_persistent_against_oracle():
    shape = CONFIGS["small"]
    inp = make_layer_inputs(shape, seed=32, masked_fraction=0.25)
    dev = to_device(inp)
    per = make_layer(shape, dev, flags=_flags())
    out = run_forward(per, dev)
    torch.cuda.synchronize()
    res = M.forward_fp8(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale)
    assert_output_close(_bits(out), res.out_bits, "persistent FC1->FC2 vs oracle")


def test_persistent_repeated_and_ragged():
    """Consecutive forwards with fewer tokens each time: the compaction
    re-zeroes the counters of the row tiles it lists."""
    shape = CONFIGS["small"]
    inp = make_layer_inputs(shape, seed=33, masked_fraction=0.25)
    dev = to_device(inp)
    sep = make_layer(shape, dev)
    per = make_layer(shape, dev, flags=_flags())
    for T in (shape.tokens, 300, 17, shape.tokens):
        per.region("hq", torch.uint8).fill_(0x7F)
        _compare(shape, sep, per, dev, tokens=T)


def test_persistent_capacity_overflow():
    shape = CONFIGS["small"]
    inp = make_layer_inputs(shape, seed=34)
    dev = to_device(inp)
    sep = make_layer(shape, dev, capacity_factor=0.3)
    per = make_layer(shape, dev, capacity_factor=0.3, flags=_flags())
    _compare(shape, sep, per, dev)
    assert per.status() == L.MOE_DEV_CAPACITY


@pytest.mark.slow
@pytest.mark.parametrize("name", ["dsv3", "skewed"])
def test_persistent_full_size_equals_two_launches(name):
    """DSV3-like shape at T=4096 (balanced) and T=8192 (Zipf, 4 empty
    experts), in the launch configuration the benchmark times."""
    shape = CONFIGS[name]
    inp = make_layer_inputs(shape, seed=35)
    dev = to_device(inp)
    sep = make_layer(shape, dev)
    per = make_layer(shape, dev, flags=_flags())
    _compare(shape, sep, per, dev)
