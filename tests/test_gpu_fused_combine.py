"""The fused last-arriver combine (MOE_FLAG_FUSED_COMBINE) against the
standalone combine kernel, through the C ABI.

Both run the same FP32 arithmetic per output column, so the fused path must
give the standalone path's output bit for bit; the standalone path is held to
the float64 oracle by test_gpu_parity.py / test_gpu_mx.py, and one case here
is checked against the oracle directly as well.  After every forward the
arrival counters must be back at zero (each (token, 256-column slice) counter
reaches exactly its token's kept-route count once, and the arrival that
completes it clears it): a lost or doubled arrival would leave a counter
non-zero or an output slice unwritten.
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

FUSED = 0
if torch.cuda.is_available():
    FUSED = L.MOE_FLAG_CHECK_ROUTES | L.MOE_FLAG_FUSED_COMBINE


def _bits(out):
    return out.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def _counters_zero(layer):
    arr = layer.region("arrive", torch.int32)
    return int(torch.count_nonzero(arr).item()) == 0


def _inputs(shape, seed, mx, masked=0.0):
    wf = {False: "fp8_block", "e4m3": "mxfp8", "e5m2": "mxfp8_e5m2"}[mx]
    return make_layer_inputs(shape, seed=seed, weight_format=wf, masked_fraction=masked)


def _pair(shape, inp, mx, **kw):
    dev = to_device(inp)
    sep = make_layer(shape, dev, mx=mx, **kw)
    fus = make_layer(shape, dev, mx=mx, flags=FUSED, **kw)
    torch.cuda.synchronize()
    assert _counters_zero(fus), "arrival counters not zero after create"
    return dev, sep, fus


CASES = [
    # (shape, expected_m, weights, masked fraction)
    ("tiny", None, False, 0.0),
    ("small", None, False, 0.25),   # fully and partly masked tokens
    ("small", 4096, False, 0.0),    # 128-token fused tiles against the 256-token ping-pong FC2
    ("small", 8, False, 0.25),      # 16-token tiles
    ("odd", None, False, 0.25),     # H = 384: the last 256-column slice is half full
    ("small", None, "e4m3", 0.25),  # MXFP8 x BF16 FC2
    ("odd", None, "e5m2", 0.0),
    # 128-token MX tiles: the separate path runs the ping-pong MX kernels, the
    # fused one the lockstep kernel at the same tile (odd: K of 3 and 2 blocks)
    ("small", 4096, "e4m3", 0.25),
    ("odd", 4096, "e5m2", 0.25),
    ("k1_fc2", 4096, "e4m3", 0.0),  # I = 128: FC2 has one K-block per tile
    ("k1_fc1", 4096, "e4m3", 0.0),  # H = 128: FC1 has one K-block per tile, FC2 one half-valid column tile
    ("k1_fc2", 4096, False, 0.0),   # the same on the FP8 ping-pong kernels (256-token tiles)
    ("k1_fc1", 4096, False, 0.0),
]

_SHAPES = {"odd": MoEShape(40, 384, 256, 4, 2, "topk"), "k1_fc2": MoEShape(40, 384, 128, 4, 2, "topk"),
           "k1_fc1": MoEShape(40, 128, 256, 4, 2, "topk")}


def _shape(name):
    return _SHAPES[name] if name in _SHAPES else CONFIGS[name]


@pytest.mark.parametrize("name,expected_m,mx,masked", CASES)
def test_fused_combine_equals_separate(name, expected_m, mx, masked):
    shape = _shape(name)
    inp = _inputs(shape, 21, mx, masked)
    dev, sep, fus = _pair(shape, inp, mx, expected_m=expected_m)
    a = _bits(run_forward(sep, dev))
    b = _bits(run_forward(fus, dev))
    torch.cuda.synchronize()
    assert np.array_equal(a, b), f"{int(np.sum(a != b))} of {a.size} output bits differ"
    assert _counters_zero(fus), "arrival counters not zero after a forward"
    assert sep.status() == fus.status()


def test_fused_combine_against_oracle():
    shape = CONFIGS["small"]
    inp = make_layer_inputs(shape, seed=22, masked_fraction=0.25)
    dev = to_device(inp)
    fus = make_layer(shape, dev, flags=FUSED)
    out = run_forward(fus, dev)
    torch.cuda.synchronize()
    res = M.forward_fp8(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale)
    assert_output_close(_bits(out), res.out_bits, "fused combine vs oracle")


def test_fused_combine_reuse_poisoned_and_ragged():
    """Consecutive forwards on one layer, the second with fewer tokens and
    the intermediate rows and output poisoned in between: every output row
    is rewritten, including the zero rows of fully masked tokens."""
    shape = CONFIGS["small"]
    inp = make_layer_inputs(shape, seed=23, masked_fraction=0.25)
    dev, sep, fus = _pair(shape, inp, False)
    for T in (shape.tokens, 200, 33):
        a = _bits(run_forward(sep, dev, tokens=T))
        fus.region("y", torch.uint8).fill_(0xFF)
        b_out = run_forward(fus, dev, tokens=T)
        torch.cuda.synchronize()
        b = _bits(b_out)
        assert np.array_equal(a, b), f"T={T}: {int(np.sum(a != b))} output bits differ"
        assert _counters_zero(fus), f"T={T}: arrival counters not zero"


def test_fused_combine_capacity_overflow():
    """Routes dropped by the row capacity never arrive; their tokens are
    completed by the kept ones (or zeroed if none is kept)."""
    shape = CONFIGS["small"]
    inp = make_layer_inputs(shape, seed=24)
    dev, sep, fus = _pair(shape, inp, False, capacity_factor=0.3)
    a = _bits(run_forward(sep, dev))
    b = _bits(run_forward(fus, dev))
    torch.cuda.synchronize()
    assert fus.status() == L.MOE_DEV_CAPACITY
    assert np.array_equal(a, b)
    assert _counters_zero(fus)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["dsv3", "skewed"])
def test_fused_combine_full_size_equals_separate(name):
    """DSV3-like shape at T=4096 (balanced) and T=8192 (Zipf, 4 empty
    experts), in the launch configuration the benchmark times."""
    shape = CONFIGS[name]
    inp = make_layer_inputs(shape, seed=25)
    dev, sep, fus = _pair(shape, inp, False)
    a = _bits(run_forward(sep, dev))
    b = _bits(run_forward(fus, dev))
    torch.cuda.synchronize()
    assert np.array_equal(a, b), f"{int(np.sum(a != b))} output bits differ"
    assert _counters_zero(fus)
