"""Pins for the oracle's staging (input quantisation, route checks) and
route compaction (no GPU)."""

import numpy as np
import torch

from oracle import formats as F
from oracle import moe_ref as M
from synthetic import CONFIGS, MoEShape, make_activations, make_routing


def test_stage_quant_matches_torch_cast_and_invariants():
    x = make_activations(64, 1024, seed=5)
    # plant an all-zero block and a block with one huge and many tiny values
    x[3, 128:256] = 0
    x[4, :128] = torch.tensor(np.r_[[3.0e4], np.full(127, 1e-3)], dtype=torch.bfloat16).view(torch.int16).numpy()
    codes, s = M.stage_quantize_1x128(x)
    xf = F.bf16_bits_to_f64(x).astype(np.float32).reshape(64, 8, 128)
    # cross-check with torch's RNE cast of fl32(x / s) (a library routine)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (xf / s[:, :, None]).astype(np.float32)
    v = np.where((s == 0)[:, :, None], np.float32(0), v)
    ref = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = codes.reshape(64, 8, 128)
    nz = (s != 0)[:, :, None] | np.zeros_like(got, bool)
    assert np.array_equal(got[nz], ref[nz])
    assert np.all(got[3, 1] == 0) and s[3, 1] == 0
    # every block with amax > 0 holds a +-448 code, and the scale is fl32(amax/448)
    amax = np.abs(xf).max(axis=2)
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
    has448 = np.any((got & 0x7F) == 0x7E, axis=2)
    assert np.all(has448[amax > 0])
    # dequantisation error: half a code spacing (relative 2**-4 normal, 2**-10 absolute subnormal)
    deq = F.e4m3_decode(got) * s[:, :, None]
    err = np.abs(deq - xf)
    bound = np.maximum(np.abs(xf) * 2.0 ** -4, 2.0 ** -10 * s[:, :, None]) * (1 + 1e-6)
    assert np.all(err <= bound)


def _brute_routes(idx, w, E, check):
    T, K = idx.shape
    oi = np.full(T * K, -1, np.int32)
    ow = np.zeros(T * K, np.float32)
    st = 0
    for t in range(T):
        seen = set()
        for k in range(K):
            e = int(idx[t, k])
            if e == -1:
                continue
            if e < -1 or e >= E:
                st |= M.STATUS_BAD_EXPERT
                continue
            if check:
                if e in seen:
                    st |= M.STATUS_DUPLICATE
                    continue
                seen.add(e)
                if not np.isfinite(w[t, k]):
                    st |= M.STATUS_NONFINITE
                    continue
            oi[t * K + k] = e
            ow[t * K + k] = w[t, k]
    return oi, ow, st


def test_stage_routes_vs_brute_force():
    rng = np.random.default_rng(2)
    E, T, K = 8, 200, 4
    idx = rng.integers(-3, E + 2, (T, K)).astype(np.int32)
    w = rng.standard_normal((T, K)).astype(np.float32)
    w[rng.random((T, K)) < 0.1] = np.nan
    w[rng.random((T, K)) < 0.05] = np.inf
    for check in (True, False):
        a = M.stage_routes(idx, w, E, check)
        b = _brute_routes(idx, w, E, check)
        assert np.array_equal(a[0], b[0])
        assert np.array_equal(a[1], b[1], equal_nan=True)
        assert a[2] == b[2]


def test_masked_routes_accept_nonfinite_weights():
    # Rubin forward preparation: expert -1 may carry NaN/inf; staged as 0, no error
    idx = np.array([[0, -1, 2], [-1, -1, -1]], np.int32)
    w = np.array([[0.5, np.nan, 0.5], [np.inf, -np.inf, np.nan]], np.float32)
    si, sw, st = M.stage_routes(idx, w, 4)
    assert st == 0
    assert si.tolist() == [0, -1, 2, -1, -1, -1]
    assert sw.tolist() == [0.5, 0.0, 0.5, 0.0, 0.0, 0.0]


def _brute_compact(idx, E, cap=None):
    pairs = [(int(e), r) for r, e in enumerate(idx) if e >= 0]
    pairs.sort()  # by expert, then route id
    if cap is not None:
        pairs = pairs[:cap]
    counts = [0] * E
    for e, _ in pairs:
        counts[e] += 1
    offs = [0]
    for c in counts:
        offs.append(offs[-1] + c)
    pos = [-1] * len(idx)
    for p, (_, r) in enumerate(pairs):
        pos[r] = p
    return counts, offs, [r for _, r in pairs], pos


def test_compact_vs_brute_force():
    for shape in (CONFIGS["tiny"], CONFIGS["small"], MoEShape(37, 128, 128, 16, 4, "zipf")):
        idx, w = make_routing(shape, seed=1, masked_fraction=0.2)
        si, _, _ = M.stage_routes(idx, w, shape.experts)
        c = M.compact(si, shape.experts)
        b = _brute_compact(si, shape.experts)
        assert c.counts.tolist() == b[0]
        assert c.offsets.tolist() == b[1]
        assert c.sorted_route.tolist() == b[2]
        assert c.route_pos.tolist() == b[3]
        assert c.status == 0


def test_compact_capacity_drops_tail_in_sorted_order():
    idx, w = make_routing(CONFIGS["tiny"], seed=4)
    si, _, _ = M.stage_routes(idx, w, 8)
    cap = 20
    c = M.compact(si, 8, row_cap=cap)
    b = _brute_compact(si, 8, cap)
    assert c.status == M.STATUS_CAPACITY
    assert c.counts.tolist() == b[0] and c.sorted_route.tolist() == b[2] and c.route_pos.tolist() == b[3]
    assert M.compact(si, 8, row_cap=32).status == 0


def test_balanced_routing_is_exactly_balanced():
    shape = MoEShape(4096, 128, 128, 32, 8, "balanced")
    idx, w = make_routing(shape, seed=0)
    counts = np.bincount(idx.ravel(), minlength=32)
    assert np.all(counts == 4096 * 8 // 32)
    assert np.all(np.sort(idx, axis=1)[:, 1:] != np.sort(idx, axis=1)[:, :-1])  # distinct per token
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)


def test_zipf_routing_has_zero_token_experts():
    idx, w = make_routing(CONFIGS["skewed"], seed=0)
    counts = np.bincount(idx.ravel(), minlength=32)
    assert np.sum(counts == 0) == 4
    assert counts.max() > 3 * np.median(counts[counts > 0])
