"""Moves host arrays of a workload to the device and runs one layer forward
through the HIP library.  Used by the tests, ``bench.py`` and the smoke run."""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import _lib as L
from .layer import MoELayer


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


@dataclass
class DeviceInputs:
    x: torch.Tensor
    topk_idx: torch.Tensor
    topk_w: torch.Tensor
    w13: torch.Tensor
    w13_scale: torch.Tensor
    w2: torch.Tensor
    w2_scale: torch.Tensor


def to_device(inp, device="cuda") -> DeviceInputs:
    """``inp``: an object with x_bf16, topk_idx, topk_w, w13, w13_scale, w2, w2_scale arrays."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)  # noqa: E731
    return DeviceInputs(bf16_tensor(inp.x_bf16, device), t(inp.topk_idx), t(inp.topk_w), t(inp.w13),
                        t(inp.w13_scale), t(inp.w2), t(inp.w2_scale))


def make_layer(shape, dev: DeviceInputs, *, expected_m: Optional[int] = None, max_rows: Optional[int] = None,
               capacity_factor: float = 1.0, flags: int = L.MOE_FLAG_CHECK_ROUTES, mx=False) -> MoELayer:
    """``mx``: MXFP8 weights (E8M0 per 32) with BF16 activations, else FP8 block-scale;
    ``mx="e5m2"`` selects e5m2 weight codes, any other true value e4m3."""
    T = shape.tokens
    if expected_m is None:
        expected_m = max(1, T * shape.top_k // shape.experts)
    wf = (L.MOE_WEIGHT_MXFP8_E5M2 if mx == "e5m2" else L.MOE_WEIGHT_MXFP8_E4M3) if mx else L.MOE_WEIGHT_E4M3_BLOCK128
    af = L.MOE_ACT_BF16 if mx else L.MOE_ACT_E4M3_1X128
    return MoELayer(shape.hidden, shape.intermediate, shape.experts, shape.top_k, dev.w13, dev.w13_scale, dev.w2,
                    dev.w2_scale, expected_m=expected_m, max_rows=max_rows or max(T, 1),
                    capacity_factor=capacity_factor, weight_format=wf, act_format=af, flags=flags)


def run_forward(layer: MoELayer, dev: DeviceInputs, tokens: Optional[int] = None, x_scale=None, x=None):
    """Stage + forward; returns the bf16 output tensor (device)."""
    T = dev.x.shape[0] if tokens is None else tokens
    xx = dev.x if x is None else x
    out = layer.stage(xx[:T].contiguous(), dev.topk_idx[:T].contiguous(), dev.topk_w[:T].contiguous(),
                      x_scale=None if x_scale is None else x_scale[:T].contiguous())
    layer.forward()
    return out
