"""A small owner of one layer handle: torch provides the device memory and
the stream, the HIP library does every step of the forward.

    layer = MoELayer(cfg, w13, w13_scale, w2, w2_scale, expected_m=..., max_rows=...)
    out = layer.stage(x, topk_idx, topk_w)      # x: bf16 [T, H] (or e4m3 codes + x_scale)
    layer.forward()                             # writes `out` on the current stream
"""

from __future__ import annotations

from typing import Optional

import torch

from . import _lib as L


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


class MoELayer:
    def __init__(self, hidden: int, intermediate: int, num_experts: int, top_k: int,
                 w13: torch.Tensor, w13_scale: torch.Tensor, w2: torch.Tensor, w2_scale: torch.Tensor, *,
                 expected_m: int, max_rows: int, capacity_factor: float = 1.0,
                 weight_format: int = L.MOE_WEIGHT_E4M3_BLOCK128, act_format: int = L.MOE_ACT_E4M3_1X128,
                 flags: int = L.MOE_FLAG_CHECK_ROUTES, workspace: Optional[torch.Tensor] = None):
        for t in (w13, w13_scale, w2, w2_scale):
            if not (t.is_cuda and t.is_contiguous()):
                raise ValueError("weights must be contiguous device tensors")
        self.cfg = L.make_config(hidden, intermediate, num_experts, top_k, weight_format, act_format, flags)
        self.hidden, self.top_k = hidden, top_k
        self.max_rows = max_rows
        self.ws_bytes = L.moe_workspace_query(self.cfg, expected_m, max_rows, capacity_factor)
        if workspace is None:
            workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=w13.device)
        elif workspace.numel() < self.ws_bytes:
            raise ValueError("workspace too small")
        self.workspace = workspace
        self._keep = (w13, w13_scale, w2, w2_scale)  # the handle reads these in place
        self.handle = L.moe_layer_create(self.cfg, expected_m, max_rows, capacity_factor, _ptr(w13),
                                         _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), _ptr(workspace),
                                         self.ws_bytes, self._stream())
        self._staged = None

    @staticmethod
    def _stream() -> int:
        return torch.cuda.current_stream().cuda_stream

    def stage(self, x: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor,
              x_scale: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, self.hidden), dtype=torch.bfloat16, device=x.device)
        for t in (x, topk_idx, topk_w, out) + ((x_scale,) if x_scale is not None else ()):
            if not t.is_contiguous():
                raise ValueError("inputs must be contiguous")
        L.moe_stage_inputs(self.handle, _ptr(x), _ptr(x_scale), _ptr(topk_idx), _ptr(topk_w), T, _ptr(out),
                           self._stream())
        self._staged = (x, topk_idx, topk_w, x_scale, out)  # keep alive until forward
        return out

    def forward(self) -> None:
        L.moe_layer_forward(self.handle, self._stream())

    def forward_noalloc(self, x: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor, out: torch.Tensor,
                        x_scale: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None) -> None:
        """Stage + forward with the per-call regions in the library's static
        device scratch (moe_layer_forward_noalloc): ``out`` and the optional
        int32 ``status`` word are caller tensors, nothing is allocated."""
        for t in (x, topk_idx, topk_w, out) + tuple(t for t in (x_scale, status) if t is not None):
            if not t.is_contiguous():
                raise ValueError("inputs must be contiguous")
        L.moe_layer_forward_noalloc(self.handle, _ptr(x), _ptr(x_scale), _ptr(topk_idx), _ptr(topk_w), x.shape[0],
                                    _ptr(out), _ptr(status), self._stream())

    def status(self) -> int:
        return L.moe_read_status(self.handle, self._stream())

    def region(self, name: str, dtype: torch.dtype, shape=None) -> torch.Tensor:
        """A device view of a workspace region (no copy)."""
        ptr, nbytes = L.moe_layer_region(self.handle, L.REGIONS[name])
        off = ptr - self.workspace.data_ptr()
        view = self.workspace[off:off + nbytes].view(dtype)
        return view if shape is None else view[: int(torch.tensor(shape).prod())].view(*shape)

    def tactic(self) -> dict:
        return L.moe_layer_tactic(self.handle)

    def profile(self, enable=True, kernels=None) -> None:
        """Time every kernel class (``enable`` true), the named ``kernels``
        only (e.g. ``("fc1",)``), or stop (``enable`` false)."""
        mask = 0
        if enable:
            mask = L.PROFILE_ALL if kernels is None else sum(1 << L.KERNELS.index(k) for k in kernels)
        L.moe_profile_enable(self.handle, mask)

    def profile_read(self) -> dict:
        return L.moe_profile_read(self.handle)

    def close(self) -> None:
        if getattr(self, "handle", None):
            L.moe_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
