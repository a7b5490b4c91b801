"""Host-side checks of the C-ABI library (no GPU): it loads, exports every
symbol include/moe.h declares, and its synchronous validation returns the
documented errors before anything is launched."""

import ctypes
import os
import re

import pytest

from mixture_experts_ffn_route_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:[A-Za-z_][\w\s\*]*?)\b(moe_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _header_functions()
    assert len(names) >= 13
    assert sorted(names) == sorted(L.EXPORTS)
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_token_bucket_matches_pages_table():
    path = os.path.join(ROOT, "tests", "golden", "token_bucket.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    assert rows
    for tokens, bucket in rows:
        got = L.moe_token_bucket(int(tokens))
        if bucket == "error":
            assert got < 0
        else:
            assert got == int(bucket), (tokens, bucket, got)


def _cfg(**kw):
    base = dict(hidden=7168, intermediate=2048, num_experts=32, top_k=8)
    base.update(kw)
    return L.make_config(base["hidden"], base["intermediate"], base["num_experts"], base["top_k"],
                         kw.get("weight_format", L.MOE_WEIGHT_E4M3_BLOCK128),
                         kw.get("act_format", L.MOE_ACT_E4M3_1X128), kw.get("flags", L.MOE_FLAG_CHECK_ROUTES))


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=3), L.MOE_ERR_UNSUPPORTED),
    (dict(top_k=10), L.MOE_ERR_UNSUPPORTED),
    (dict(hidden=7000), L.MOE_ERR_UNSUPPORTED),
    (dict(intermediate=100), L.MOE_ERR_UNSUPPORTED),
    (dict(hidden=0), L.MOE_ERR_INVALID_ARG),
    (dict(num_experts=0), L.MOE_ERR_UNSUPPORTED),
    (dict(num_experts=2000), L.MOE_ERR_UNSUPPORTED),
    (dict(num_experts=4, top_k=6), L.MOE_ERR_INVALID_ARG),
    (dict(flags=0x100), L.MOE_ERR_INVALID_ARG),
    (dict(act_format=L.MOE_ACT_BF16), L.MOE_ERR_UNSUPPORTED),
    (dict(weight_format=L.MOE_WEIGHT_MXFP8_E4M3), L.MOE_ERR_UNSUPPORTED),
    (dict(weight_format=7), L.MOE_ERR_INVALID_ARG),
])
def test_query_rejects_bad_config(kw, status):
    with pytest.raises(L.MoEError) as ei:
        L.moe_workspace_query(_cfg(**kw), 64, 128, 1.0)
    assert ei.value.status == status
    assert L.moe_last_error()


@pytest.mark.parametrize("expected_m,max_rows,cf,status", [
    (0, 128, 1.0, L.MOE_ERR_INVALID_ARG),
    (64, 0, 1.0, L.MOE_ERR_INVALID_ARG),
    (64, 128, 0.0, L.MOE_ERR_INVALID_ARG),
    (64, 128, float("nan"), L.MOE_ERR_INVALID_ARG),
    (64, 128, float("inf"), L.MOE_ERR_INVALID_ARG),
    (64, 1 << 28, 1.0, L.MOE_ERR_UNSUPPORTED),
])
def test_query_rejects_bad_sizes(expected_m, max_rows, cf, status):
    with pytest.raises(L.MoEError) as ei:
        L.moe_workspace_query(_cfg(), expected_m, max_rows, cf)
    assert ei.value.status == status


def test_query_rejects_fp8_operands_of_2gib():
    """The FP8 GEMMs gather token rows with 31-bit byte offsets: the FC1
    output (route rows held * I bytes) and the staged activations must each
    stay under 2 GiB."""
    cfg = _cfg()
    K, I = 8, 2048
    rows = (1 << 31) // (K * I) - 1  # largest max_rows whose route rows * I < 2^31
    L.moe_workspace_query(cfg, 64, rows, 1.0)
    with pytest.raises(L.MoEError) as ei:
        L.moe_workspace_query(cfg, 64, rows + 1, 1.0)
    assert ei.value.status == L.MOE_ERR_UNSUPPORTED
    # a capacity factor below one holds fewer route rows
    L.moe_workspace_query(cfg, 64, rows + 1, 0.5)
    # per-route staging keeps K activation rows per token
    staged = _cfg(flags=L.MOE_FLAG_CHECK_ROUTES | L.MOE_FLAG_PER_ROUTE_STAGING)
    x_rows = (1 << 31) // (K * 7168)
    L.moe_workspace_query(staged, 64, x_rows - 1, 0.25)
    with pytest.raises(L.MoEError) as ei:
        L.moe_workspace_query(staged, 64, x_rows + 1, 0.25)
    assert ei.value.status == L.MOE_ERR_UNSUPPORTED


def test_query_sizes_scale_with_capacity_not_tactic():
    cfg = _cfg()
    a = L.moe_workspace_query(cfg, 8, 4096, 1.0)
    b = L.moe_workspace_query(cfg, 8, 8192, 1.0)
    c = L.moe_workspace_query(cfg, 8, 4096, 0.5)
    assert a % 256 == 0 and b > a and c < a
    # the y buffer dominates: row_cap * H * 2 bytes
    assert a >= 4096 * 8 * 7168 * 2
    # tactic (expected_m) changes only the tile list bound
    d = L.moe_workspace_query(cfg, 4096, 4096, 1.0)
    assert abs(d - a) < 64 * 1024
    e = L.moe_workspace_query(_cfg(flags=L.MOE_FLAG_CHECK_ROUTES | L.MOE_FLAG_PER_ROUTE_STAGING), 8, 4096, 1.0)
    assert e - a >= 4096 * 7 * 7168  # K copies of each activation row


def test_create_validation_before_any_launch():
    cfg = _cfg(hidden=256, intermediate=128, num_experts=8, top_k=2)
    n = L.moe_workspace_query(cfg, 4, 16, 1.0)
    # NULL weights
    with pytest.raises(L.MoEError) as ei:
        L.moe_layer_create(cfg, 4, 16, 1.0, 0, 0, 0, 0, 4096, n)
    assert ei.value.status == L.MOE_ERR_INVALID_ARG
    # misaligned weight codes
    with pytest.raises(L.MoEError) as ei:
        L.moe_layer_create(cfg, 4, 16, 1.0, 4097, 4096, 4096, 4096, 4096, n)
    assert ei.value.status == L.MOE_ERR_INVALID_ARG
    # misaligned workspace
    with pytest.raises(L.MoEError) as ei:
        L.moe_layer_create(cfg, 4, 16, 1.0, 4096, 4096, 4096, 4096, 4096 + 16, n)
    assert ei.value.status == L.MOE_ERR_INVALID_ARG
    # workspace too small
    with pytest.raises(L.MoEError) as ei:
        L.moe_layer_create(cfg, 4, 16, 1.0, 4096, 4096, 4096, 4096, 4096, n - 256)
    assert ei.value.status == L.MOE_ERR_WORKSPACE_TOO_SMALL


def test_null_handle_calls_fail_cleanly():
    for fn, args in [(L.moe_layer_forward, (0, 0)), (L.moe_read_status, (0, 0)), (L.moe_layer_tactic, (0,)),
                     (L.moe_profile_enable, (0, True)), (L.moe_profile_read, (0,)), (L.moe_layer_region, (0, 0))]:
        with pytest.raises(L.MoEError) as ei:
            fn(*args)
        assert ei.value.status == L.MOE_ERR_INVALID_ARG
    with pytest.raises(L.MoEError):
        L.moe_stage_inputs(0, 0, 0, 0, 0, 1, 0, 0)
    with pytest.raises(L.MoEError) as ei:
        L.moe_layer_forward_noalloc(0, 0, 0, 0, 0, 1, 0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARG
    L.moe_layer_destroy(0)  # no-op


def test_status_strings():
    for s in range(0, -7, -1):
        assert L.status_string(s).startswith("MOE_")
    assert L.status_string(-99) == "MOE_ERR_UNKNOWN"


def test_query_mx_variant_sizes():
    """MXFP8 x BF16: two e4m3 activation terms, one E8M0 word per 32 columns,
    and 1 KB of tiled weight exponents per 32 KB weight tile."""
    T, H, I, E, K = 4096, 7168, 2048, 32, 8
    fp8 = L.moe_workspace_query(_cfg(), 128, T, 1.0)
    mx = L.moe_workspace_query(_cfg(weight_format=L.MOE_WEIGHT_MXFP8_E4M3, act_format=L.MOE_ACT_BF16), 128, T, 1.0)
    R = T * K
    extra = (T * H                                   # lo-term plane of x
             + T * (H // 32) * 4 - T * (H // 128) * 4  # exponent words vs 1x128 scales
             + R * I                                 # lo-term plane of h
             + R * (I // 32) * 4 - R * (I // 128) * 4
             + E * 2 * I * H // 32 + E * H * I // 32)  # weight exponent tiles
    assert abs((mx - fp8) - extra) <= 8 * 256  # region alignment only


def test_unfused_fc1_flag():
    """MOE_FLAG_UNFUSED_FC1 is an FP8-path debug mode: it adds an FP32 [row_cap, 2I]
    gate/up region and is refused for MXFP8 weights."""
    base = L.moe_workspace_query(_cfg(), 128, 4096, 1.0)
    unf = L.moe_workspace_query(_cfg(flags=L.MOE_FLAG_CHECK_ROUTES | L.MOE_FLAG_UNFUSED_FC1), 128, 4096, 1.0)
    assert abs((unf - base) - 4096 * 8 * 2 * 2048 * 4) <= 256
    with pytest.raises(L.MoEError) as ei:
        L.moe_workspace_query(_cfg(weight_format=L.MOE_WEIGHT_MXFP8_E4M3, act_format=L.MOE_ACT_BF16,
                                   flags=L.MOE_FLAG_UNFUSED_FC1), 128, 4096, 1.0)
    assert ei.value.status == L.MOE_ERR_UNSUPPORTED


def test_stream_flags():
    """The streaming-kernel switches change no workspace size, and asking
    for the streaming FC1 while turning streaming off is refused."""
    base = L.moe_workspace_query(_cfg(), 128, 4096, 1.0)
    for f in (L.MOE_FLAG_NO_STREAM, L.MOE_FLAG_STREAM_FC1):
        assert L.moe_workspace_query(_cfg(flags=L.MOE_FLAG_CHECK_ROUTES | f), 128, 4096, 1.0) == base
    with pytest.raises(L.MoEError) as ei:
        L.moe_workspace_query(_cfg(flags=L.MOE_FLAG_NO_STREAM | L.MOE_FLAG_STREAM_FC1), 128, 4096, 1.0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARG


def test_bf16_gateup_flag():
    """MOE_FLAG_BF16_GATEUP halves the unfused gate/up region (BF16) and is
    refused without MOE_FLAG_UNFUSED_FC1."""
    unf = L.moe_workspace_query(_cfg(flags=L.MOE_FLAG_CHECK_ROUTES | L.MOE_FLAG_UNFUSED_FC1), 128, 4096, 1.0)
    b16 = L.moe_workspace_query(_cfg(flags=L.MOE_FLAG_CHECK_ROUTES | L.MOE_FLAG_UNFUSED_FC1 | L.MOE_FLAG_BF16_GATEUP),
                                128, 4096, 1.0)
    assert abs((unf - b16) - 4096 * 8 * 2 * 2048 * 2) <= 256
    with pytest.raises(L.MoEError) as ei:
        L.moe_workspace_query(_cfg(flags=L.MOE_FLAG_CHECK_ROUTES | L.MOE_FLAG_BF16_GATEUP), 128, 4096, 1.0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARG


def test_slot_timers_unsupported_in_the_plain_build():
    """moe_debug_slot_timers only works in the library built with slot
    timers; the plain build refuses it without touching the buffer."""
    if L.SLOT_TIMERS:
        pytest.skip("the timed library is loaded")
    buf = (ctypes.c_uint64 * L.MOE_SLOT_TIMER_WORDS)(*([7] * L.MOE_SLOT_TIMER_WORDS))
    st = L.lib().moe_debug_slot_timers(ctypes.cast(buf, ctypes.c_void_p), L.MOE_SLOT_TIMER_WORDS)
    assert st == L.MOE_ERR_UNSUPPORTED
    assert list(buf) == [7] * L.MOE_SLOT_TIMER_WORDS
    assert "slot timers" in L.moe_last_error()


def test_fused_combine_flag():
    """MOE_FLAG_FUSED_COMBINE adds the int32 [max_rows, ceil(H/256)] arrival
    counters and is accepted with either weight format."""
    base = L.moe_workspace_query(_cfg(), 128, 4096, 1.0)
    fus = L.moe_workspace_query(_cfg(flags=L.MOE_FLAG_CHECK_ROUTES | L.MOE_FLAG_FUSED_COMBINE), 128, 4096, 1.0)
    assert fus - base == 4096 * 28 * 4
    mx = _cfg(weight_format=L.MOE_WEIGHT_MXFP8_E4M3, act_format=L.MOE_ACT_BF16)
    mx_base = L.moe_workspace_query(mx, 128, 4096, 1.0)
    mx_fus = L.moe_workspace_query(_cfg(weight_format=L.MOE_WEIGHT_MXFP8_E4M3, act_format=L.MOE_ACT_BF16,
                                        flags=L.MOE_FLAG_FUSED_COMBINE), 128, 4096, 1.0)
    assert mx_fus - mx_base == 4096 * 28 * 4
    with pytest.raises(L.MoEError) as ei:
        L.moe_workspace_query(_cfg(flags=32), 128, 4096, 1.0)
    assert ei.value.status == L.MOE_ERR_INVALID_ARG


def test_persistent_ffn_flag():
    """MOE_FLAG_PERSISTENT_FFN adds one int32 readiness counter per row tile
    (max_m_tiles of them) and is an FP8-path option without the unfused FC1."""
    base = L.moe_workspace_query(_cfg(), 128, 4096, 1.0)
    per = L.moe_workspace_query(_cfg(flags=L.MOE_FLAG_CHECK_ROUTES | L.MOE_FLAG_PERSISTENT_FFN), 128, 4096, 1.0)
    max_m_tiles = (4096 * 8 + 127) // 128 + 32  # row_cap / block_m rounded up, plus one per expert
    assert per - base == (max_m_tiles * 4 + 255) // 256 * 256
    for kw in (dict(weight_format=L.MOE_WEIGHT_MXFP8_E4M3, act_format=L.MOE_ACT_BF16,
                    flags=L.MOE_FLAG_PERSISTENT_FFN),
               dict(flags=L.MOE_FLAG_PERSISTENT_FFN | L.MOE_FLAG_UNFUSED_FC1)):
        with pytest.raises(L.MoEError) as ei:
            L.moe_workspace_query(_cfg(**kw), 128, 4096, 1.0)
        assert ei.value.status == L.MOE_ERR_UNSUPPORTED
