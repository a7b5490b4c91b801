"""ctypes binding of ``include/moe.h`` (argument marshalling only).

Every function here has the name of the C entry point it wraps, takes plain
integers (device pointers as ``int``) and raises ``MoEError`` for a negative
status.  The shared library is loaded as built (``build.py``); when none has
been built, it is compiled once from the HIP sources first.  If that fails,
importing this module raises ``ImportError`` -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_double, c_float, c_int32, c_int64, c_size_t, c_uint32, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_SLOT_TIMERS=1 loads the build with the 256-token GEMM's slot timers
# (build.py --slot-timers; for moe_debug_slot_timers), never built on demand.
SLOT_TIMERS = os.environ.get("MOE_SLOT_TIMERS", "0") == "1"
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x_slot_timers.so" if SLOT_TIMERS else "libmoe_mi355x.so")
MOE_SLOT_TIMER_WORDS = 32

# moe_status_t
MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE_TOO_SMALL = -3
MOE_ERR_CAPACITY = -4
MOE_ERR_STATE = -5
MOE_ERR_HIP = -6

MOE_WEIGHT_E4M3_BLOCK128 = 0
MOE_WEIGHT_MXFP8_E4M3 = 1
MOE_WEIGHT_MXFP8_E5M2 = 2
MOE_ACT_E4M3_1X128 = 0
MOE_ACT_BF16 = 1
MOE_FLAG_CHECK_ROUTES = 1
MOE_FLAG_PER_ROUTE_STAGING = 2
MOE_FLAG_UNFUSED_FC1 = 4
MOE_FLAG_FUSED_COMBINE = 8
MOE_FLAG_PERSISTENT_FFN = 16
MOE_FLAG_BF16_GATEUP = 32
MOE_FLAG_NO_STREAM = 64
MOE_FLAG_STREAM_FC1 = 128
MOE_DEV_BAD_EXPERT = 1
MOE_DEV_DUPLICATE = 2
MOE_DEV_NONFINITE = 4
MOE_DEV_CAPACITY = 8
MOE_DEV_WAIT_TIMEOUT = 16

REGIONS = {
    "status": 0, "staged_idx": 1, "staged_w": 2, "xq": 3, "xs": 4, "counts": 5, "offsets": 6,
    "sorted_route": 7, "route_pos": 8, "hq": 9, "hs": 10, "y": 11, "tiles": 12, "w13t": 13, "w2t": 14,
    "w13s": 15, "w2s": 16, "gateup": 17, "arrive": 18, "ready": 19,
}
KERNELS = ("stage", "compact", "fc1", "fc2", "combine")
PROFILE_ALL = (1 << len(KERNELS)) - 1

# Every symbol include/moe.h declares.
EXPORTS = (
    "moe_workspace_query", "moe_layer_create", "moe_stage_inputs", "moe_layer_forward",
    "moe_layer_forward_noalloc", "moe_read_status", "moe_layer_region", "moe_layer_tactic", "moe_profile_enable",
    "moe_profile_read", "moe_layer_destroy", "moe_token_bucket", "moe_status_string",
    "moe_last_error", "moe_debug_slot_timers",
)


class MoEError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


class moe_config_t(Structure):
    _fields_ = [
        ("hidden", c_int32), ("intermediate", c_int32), ("num_experts", c_int32), ("top_k", c_int32),
        ("weight_format", c_int32), ("act_format", c_int32), ("flags", c_uint32),
    ]


class moe_weights_t(Structure):
    _fields_ = [("w13", c_void_p), ("w13_scale", c_void_p), ("w2", c_void_p), ("w2_scale", c_void_p)]


class moe_tactic_t(Structure):
    _fields_ = [
        ("token_bucket", c_int32), ("block_m", c_int32), ("block_n", c_int32), ("grid_fc1", c_int32),
        ("grid_fc2", c_int32), ("row_cap", c_int32), ("max_m_tiles", c_int32), ("tile_order", c_int32),
        ("stream_depth_fc1", c_int32), ("stream_depth_fc2", c_int32),
    ]


def _load() -> ctypes.CDLL:
    if SLOT_TIMERS and not os.path.exists(LIB_PATH):
        raise ImportError(f"MOE_SLOT_TIMERS=1 needs {LIB_PATH} (build.py --slot-timers)")
    if not os.path.exists(LIB_PATH):
        # nothing built yet: compile the gfx950 library (hipcc), else fail
        try:
            from . import build as _build
            _build.build()
        except Exception as exc:  # noqa: BLE001
            raise ImportError(f"HIP library {LIB_PATH} is not built and building it failed: {exc}") from exc
    # One HIP runtime per process: torch ships its own libamdhip64 (SONAME
    # libamdhip64.so.7).  Loading torch first makes the dynamic linker bind
    # this library to that same runtime, so torch's streams and allocations
    # are valid handles here.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    i32, vp = c_int32, c_void_p
    sig = {
        "moe_workspace_query": (i32, [POINTER(moe_config_t), i32, i32, c_float, POINTER(c_size_t)]),
        "moe_layer_create": (i32, [POINTER(moe_config_t), i32, i32, c_float, POINTER(moe_weights_t), vp, c_size_t,
                                   vp, POINTER(vp)]),
        "moe_stage_inputs": (i32, [vp, vp, vp, vp, vp, i32, vp, vp]),
        "moe_layer_forward": (i32, [vp, vp]),
        "moe_layer_forward_noalloc": (i32, [vp, vp, vp, vp, vp, i32, vp, vp, vp]),
        "moe_read_status": (i32, [vp, vp, POINTER(c_uint32)]),
        "moe_layer_region": (i32, [vp, i32, POINTER(vp), POINTER(c_size_t)]),
        "moe_layer_tactic": (i32, [vp, POINTER(moe_tactic_t)]),
        "moe_profile_enable": (i32, [vp, c_uint32]),
        "moe_profile_read": (i32, [vp, POINTER(c_double), POINTER(c_int64)]),
        "moe_layer_destroy": (i32, [vp]),
        "moe_debug_slot_timers": (i32, [vp, i32]),
        "moe_token_bucket": (i32, [i32]),
        "moe_status_string": (c_char_p, [i32]),
        "moe_last_error": (c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def moe_last_error() -> str:
    return _lib.moe_last_error().decode()


def _check(status: int) -> int:
    if status < 0:
        raise MoEError(status, moe_last_error())
    return status


def make_config(hidden, intermediate, num_experts, top_k, weight_format=MOE_WEIGHT_E4M3_BLOCK128,
                act_format=MOE_ACT_E4M3_1X128, flags=MOE_FLAG_CHECK_ROUTES) -> moe_config_t:
    return moe_config_t(hidden, intermediate, num_experts, top_k, weight_format, act_format, flags)


def moe_workspace_query(cfg: moe_config_t, expected_m: int, max_rows: int, capacity_factor: float) -> int:
    n = c_size_t(0)
    _check(_lib.moe_workspace_query(ctypes.byref(cfg), expected_m, max_rows, capacity_factor, ctypes.byref(n)))
    return n.value


def moe_layer_create(cfg: moe_config_t, expected_m: int, max_rows: int, capacity_factor: float,
                     w13: int, w13_scale: int, w2: int, w2_scale: int, workspace: int, ws_bytes: int,
                     stream: int = 0) -> int:
    h = c_void_p()
    w = moe_weights_t(w13, w13_scale, w2, w2_scale)
    _check(_lib.moe_layer_create(ctypes.byref(cfg), expected_m, max_rows, capacity_factor, ctypes.byref(w),
                                 workspace, ws_bytes, stream, ctypes.byref(h)))
    return h.value


def moe_stage_inputs(layer: int, x: int, x_scale: int, topk_idx: int, topk_w: int, num_tokens: int,
                     out_bf16: int, stream: int = 0) -> None:
    _check(_lib.moe_stage_inputs(layer, x, x_scale or None, topk_idx, topk_w, num_tokens, out_bf16, stream))


def moe_layer_forward(layer: int, stream: int = 0) -> None:
    _check(_lib.moe_layer_forward(layer, stream))


def moe_layer_forward_noalloc(layer: int, x: int, x_scale: int, topk_idx: int, topk_w: int, num_tokens: int,
                              out_bf16: int, status_bits: int = 0, stream: int = 0) -> None:
    _check(_lib.moe_layer_forward_noalloc(layer, x, x_scale or None, topk_idx, topk_w, num_tokens, out_bf16,
                                          status_bits or None, stream))


def moe_read_status(layer: int, stream: int = 0) -> int:
    bits = c_uint32(0)
    _check(_lib.moe_read_status(layer, stream, ctypes.byref(bits)))
    return bits.value


def moe_layer_region(layer: int, region: int):
    p, n = c_void_p(), c_size_t(0)
    _check(_lib.moe_layer_region(layer, region, ctypes.byref(p), ctypes.byref(n)))
    return p.value or 0, n.value


def moe_layer_tactic(layer: int) -> dict:
    t = moe_tactic_t()
    _check(_lib.moe_layer_tactic(layer, ctypes.byref(t)))
    return {name: getattr(t, name) for name, _ in t._fields_}


def moe_profile_enable(layer: int, kernel_mask: int) -> None:
    """kernel_mask: bit (1 << k) per KERNELS[k] class to time, PROFILE_ALL, or 0."""
    _check(_lib.moe_profile_enable(layer, kernel_mask))


def moe_profile_read(layer: int) -> dict:
    ms = (c_double * len(KERNELS))()
    n = (c_int64 * len(KERNELS))()
    _check(_lib.moe_profile_read(layer, ms, n))
    return {k: (ms[i], n[i]) for i, k in enumerate(KERNELS)}


def moe_layer_destroy(layer: int) -> None:
    _check(_lib.moe_layer_destroy(layer))


def moe_token_bucket(tokens: int) -> int:
    return _lib.moe_token_bucket(tokens)


def moe_debug_slot_timers():
    """moe_debug_slot_timers: the slot cycle counters since the previous call
    as a list of MOE_SLOT_TIMER_WORDS ints (raises MoEError with
    MOE_ERR_UNSUPPORTED unless the timed library is loaded)."""
    buf = (ctypes.c_uint64 * MOE_SLOT_TIMER_WORDS)()
    _check(_lib.moe_debug_slot_timers(ctypes.cast(buf, c_void_p), MOE_SLOT_TIMER_WORDS))
    return list(buf)
