"""The no-allocation entry point (moe_layer_forward_noalloc) against the
existing stage + forward entry points, through the C ABI.

The same kernels run on the same inputs, so the outputs, the status bits
and the compaction must be identical; two calls in a row, the second with
fewer tokens, check that nothing of the first call's scratch leaks into the
second, and the handle's own staged batch must be untouched by them.
"""

import numpy as np
import pytest
import torch

from synthetic import CONFIGS, MoEShape, make_layer_inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mixture_experts_ffn_route_amd import _lib as L
    from mixture_experts_ffn_route_amd.harness import make_layer, run_forward, to_device


def _bits(out):
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def _both(layer, dev, T):
    """(existing entry points' output, status), (no-alloc output, status bits)."""
    ref = _bits(run_forward(layer, dev, tokens=T))
    ref_status = layer.status()
    out = torch.full((T, dev.x.shape[1]), -1.0, dtype=torch.bfloat16, device="cuda")  # poisoned
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    layer.forward_noalloc(dev.x[:T].contiguous(), dev.topk_idx[:T].contiguous(), dev.topk_w[:T].contiguous(), out,
                          status=status)
    torch.cuda.synchronize()
    return ref, ref_status, _bits(out), int(status.cpu().numpy().view(np.uint32)[0])


@pytest.mark.parametrize("cfg,mx,tokens", [
    ("small", False, (512, 301)),          # several compaction workgroups, then one
    ("tiny", False, (16, 5)),
    ("tiny", "e4m3", (16, 7)),             # MXFP8 x BF16
    ("dsv3", False, (64, 8)),              # the decode shape
])
def test_noalloc_matches_stage_and_forward(cfg, mx, tokens):
    base = CONFIGS[cfg]
    shape = MoEShape(tokens[0], base.hidden, base.intermediate, base.experts, base.top_k, base.routing)
    inp = make_layer_inputs(shape, seed=21, masked_fraction=0.1,
                            weight_format="mxfp8" if mx else "fp8_block")
    dev = to_device(inp)
    layer = make_layer(shape, dev, mx=mx)
    for T in tokens:  # the second call is smaller
        ref, ref_status, got, got_status = _both(layer, dev, T)
        assert np.array_equal(got, ref), f"{cfg} T={T}"
        assert got_status == ref_status, (got_status, ref_status)
    # the handle's staged batch (the last moe_stage_inputs, T = tokens[-1])
    # is the one a plain forward still runs
    out2 = torch.empty((tokens[-1], shape.hidden), dtype=torch.bfloat16, device="cuda")
    layer.stage(dev.x[:tokens[-1]].contiguous(), dev.topk_idx[:tokens[-1]].contiguous(),
                dev.topk_w[:tokens[-1]].contiguous(), out=out2)
    layer.forward()
    torch.cuda.synchronize()
    ref_last = _bits(out2)
    layer.forward_noalloc(dev.x[:tokens[0]].contiguous(), dev.topk_idx[:tokens[0]].contiguous(),
                          dev.topk_w[:tokens[0]].contiguous(),
                          torch.empty((tokens[0], shape.hidden), dtype=torch.bfloat16, device="cuda"))
    out2.fill_(0)
    layer.forward()
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out2), ref_last)


def test_noalloc_rejects_calls_beyond_the_scratch():
    """About 139 KB of per-call regions per token at the DSV3-like shape: a
    1000-token call does not fit in the 64 MiB scratch and launches nothing."""
    base = CONFIGS["dsv3"]
    shape = MoEShape(1000, base.hidden, base.intermediate, base.experts, base.top_k, base.routing)
    inp = make_layer_inputs(shape, seed=22)
    dev = to_device(inp)
    layer = make_layer(shape, dev)
    out = torch.empty((1000, shape.hidden), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(L.MoEError) as ei:
        layer.forward_noalloc(dev.x, dev.topk_idx, dev.topk_w, out)
    assert ei.value.status == L.MOE_ERR_CAPACITY
    assert "no-allocation forward holds" in str(ei.value)
