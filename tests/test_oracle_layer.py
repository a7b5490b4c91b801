"""Pins for the oracle's GEMM steps, SwiGLU/requantisation, combine and the
whole-layer wiring (no GPU).

* exact rational arithmetic (``fractions.Fraction``) for FC1 on the tiny shape;
* one-hot weight closed forms (catch a dropped scale, swapped gate/up, a
  transposed operand);
* brute-force loops on tiny shapes;
* requantisation invariants;
* combine identities (K=1, power-of-two weights, all-masked, masked NaN);
* deduplicated staging == per-route staging, bit for bit;
* figures the pages print that follow from the shapes.
"""

import math
import os
from fractions import Fraction
from itertools import combinations

import numpy as np
import pytest

from oracle import formats as F
from oracle import moe_ref as M
from synthetic import CONFIGS, MoEShape, make_layer_inputs, make_routing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _frac_e4m3(code):
    return Fraction(float(F.e4m3_decode(np.array([code], np.uint8))[0]))


@pytest.fixture(scope="module")
def tiny():
    return make_layer_inputs(CONFIGS["tiny"], seed=0)


def test_fc1_exact_rational_tiny(tiny):
    xq, xs = M.stage_quantize_1x128(tiny.x_bf16)
    e = 2
    rows = [0, 5, 11]
    xr = M.dequant_rows_1x128(xq[rows], xs[rows])
    gu = M.fc1_gateup(xr, tiny.w13[e], tiny.w13_scale[e])
    H = tiny.shape.hidden
    for i, t in enumerate(rows):
        for n in range(0, gu.shape[1], 7):
            exact = Fraction(0)
            absum = Fraction(0)
            for k in range(H):
                p = (_frac_e4m3(xq[t, k]) * Fraction(float(xs[t, k // 128]))
                     * _frac_e4m3(tiny.w13[e, n, k]) * Fraction(float(tiny.w13_scale[e, n // 128, k // 128])))
                exact += p
                absum += abs(p)
            assert abs(Fraction(gu[i, n]) - exact) <= absum * Fraction(H, 2 ** 52), (t, n)


def _one_hot_weights(rng, n_rows, n_cols, nonzero_col):
    codes = np.zeros((n_rows, n_cols), np.uint8)
    vals = rng.integers(0x20, 0x58, n_rows).astype(np.uint8) | (rng.integers(0, 2, n_rows).astype(np.uint8) << 7)
    codes[np.arange(n_rows), nonzero_col] = vals
    scales = rng.uniform(0.5, 2.0, (n_rows // 128, n_cols // 128)).astype(np.float32)
    return codes, scales


def test_fc1_swiglu_one_hot_closed_form():
    rng = np.random.default_rng(0)
    H, I, n = 256, 128, 5
    jg = rng.integers(0, H, I)
    ju = rng.integers(0, H, I)
    w13, s13 = _one_hot_weights(rng, 2 * I, H, np.r_[jg, ju])
    xq = rng.integers(0, 0x7E, (n, H)).astype(np.uint8) | (rng.integers(0, 2, (n, H)).astype(np.uint8) << 7)
    xs = rng.uniform(0.001, 0.01, (n, H // 128)).astype(np.float32)
    xr = M.dequant_rows_1x128(xq, xs)
    gu = M.fc1_gateup(xr, w13, s13)
    h, codes, scales = M.fc1_swiglu_requant(xr, w13, s13)
    for r in range(n):
        for c in range(I):
            g = float(_frac_e4m3(xq[r, jg[c]]) * Fraction(float(xs[r, jg[c] // 128]))
                      * _frac_e4m3(w13[c, jg[c]]) * Fraction(float(s13[0, jg[c] // 128])))
            u = float(_frac_e4m3(xq[r, ju[c]]) * Fraction(float(xs[r, ju[c] // 128]))
                      * _frac_e4m3(w13[I + c, ju[c]]) * Fraction(float(s13[1, ju[c] // 128])))
            assert gu[r, c] == g and gu[r, I + c] == u
            want = g / (1.0 + math.exp(-g)) * u
            assert abs(h[r, c] - want) <= 1e-15 * abs(want) + 1e-300
    # requantisation invariants
    deq = F.e4m3_decode(codes) * np.repeat(scales, 128, axis=1)
    assert np.all(np.abs(F.e4m3_decode(codes)) <= 448)
    amax = np.abs(h).reshape(n, 1, 128).max(axis=2)
    assert np.array_equal(scales, (amax / 448.0).astype(np.float32))
    assert np.all(np.any((codes.reshape(n, 1, 128) & 0x7F) == 0x7E, axis=2)[amax > 0])
    assert np.all(np.abs(deq - h) <= np.maximum(np.abs(h) * 2.0 ** -4, 2.0 ** -10 * np.repeat(scales, 128, 1)) * 1.000001)


def test_fc2_one_hot_closed_form():
    rng = np.random.default_rng(1)
    H, I, n = 256, 256, 3
    j = rng.integers(0, I, H)
    w2, s2 = _one_hot_weights(rng, H, I, j)
    hd = rng.standard_normal((n, I))
    y = M.fc2(hd, w2, s2)
    for r in range(n):
        for c in range(H):
            want = float(Fraction(hd[r, j[c]]) * _frac_e4m3(w2[c, j[c]]) * Fraction(float(s2[c // 128, j[c] // 128])))
            assert y[r, c] == want


def test_fc2_and_fc1_brute_force_loops():
    rng = np.random.default_rng(3)
    n, H, I = 3, 256, 128
    w = rng.integers(0, 0x7E, (2 * I, H)).astype(np.uint8) | (rng.integers(0, 2, (2 * I, H)).astype(np.uint8) << 7)
    sw = rng.uniform(1e-3, 1e-2, (2, 2)).astype(np.float32)
    x = rng.standard_normal((n, H))
    gu = M.fc1_gateup(x, w, sw)
    for r in range(n):
        for c in range(0, 2 * I, 5):
            terms = [x[r, k] * float(F.e4m3_decode(np.array([w[c, k]]))[0]) * float(sw[c // 128, k // 128])
                     for k in range(H)]
            assert abs(gu[r, c] - math.fsum(terms)) <= 1e-12 * sum(abs(t) for t in terms)
    w2 = w[:, :I].copy()  # [2I=256 rows=H, I cols]
    y = M.fc2(x[:, :I], w2, sw[:, :1])
    for r in range(n):
        for c in range(0, 256, 3):
            terms = [x[r, k] * float(F.e4m3_decode(np.array([w2[c, k]]))[0]) * float(sw[c // 128, 0])
                     for k in range(I)]
            assert abs(y[r, c] - math.fsum(terms)) <= 1e-12 * sum(abs(t) for t in terms)


def test_combine_identities():
    rng = np.random.default_rng(5)
    T, K, H = 6, 3, 256
    R = T * K
    y = rng.standard_normal((R, H)) * 3
    route_pos = np.arange(R, dtype=np.int32)
    w = rng.uniform(0.1, 1, R).astype(np.float32)
    out = M.combine(y, route_pos, w, T, K)
    # power-of-two weights commute with rounding
    out2 = M.combine(y, route_pos, w * np.float32(2), T, K)
    assert np.array_equal(F.bf16_bits_to_f64(out2), 2 * F.bf16_bits_to_f64(out))
    # K = 1, weight 1: the output is the rounded row
    one = M.combine(y[:T], np.arange(T, dtype=np.int32), np.ones(T, np.float32), T, 1)
    assert np.array_equal(one, F.bf16_rne_bits(y[:T]))
    # an all-masked token gives +0
    rp = route_pos.copy()
    rp[0:K] = -1
    z = M.combine(y, rp, w, T, K)
    assert np.all(z[0] == 0)


def test_masked_nan_weights_do_not_change_output(tiny):
    idx, w = make_routing(CONFIGS["tiny"], seed=0, masked_fraction=0.25)
    args = (tiny.x_bf16, idx, None, tiny.w13, tiny.w13_scale, tiny.w2, tiny.w2_scale)
    w_nan = w.copy()
    w_zero = np.where(idx < 0, np.float32(0), w)
    a = M.forward_fp8(args[0], idx, w_nan, *args[3:])
    b = M.forward_fp8(args[0], idx, w_zero, *args[3:])
    assert a.status == 0
    assert np.array_equal(a.out_bits, b.out_bits)
    assert np.all(a.out_bits[-1] == 0)  # last token fully masked -> +0


def test_dedup_equals_per_route_staging():
    for cfg in ("tiny",):
        inp = make_layer_inputs(CONFIGS[cfg], seed=2)
        a = M.forward_fp8(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale)
        b = M.forward_fp8(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale,
                          per_route_staging=True)
        assert np.array_equal(a.out_bits, b.out_bits)


def test_forward_fp8_vs_per_route_loop(tiny):
    """Whole-layer wiring: loop over tokens and slots, no compaction."""
    xq, xs = M.stage_quantize_1x128(tiny.x_bf16)
    res = M.forward_fp8(tiny.x_bf16, tiny.topk_idx, tiny.topk_w, tiny.w13, tiny.w13_scale, tiny.w2, tiny.w2_scale)
    T, K = tiny.topk_idx.shape
    I = tiny.shape.intermediate
    w13d = [M.dequant_block128(tiny.w13[e], tiny.w13_scale[e]) for e in range(8)]
    w2d = [M.dequant_block128(tiny.w2[e], tiny.w2_scale[e]) for e in range(8)]
    for t in range(T):
        xd = F.e4m3_decode(xq[t]) * np.repeat(xs[t], 128)
        acc = np.zeros(tiny.shape.hidden)
        for k in range(K):
            e = int(tiny.topk_idx[t, k])
            gu = np.array([math.fsum(xd * w13d[e][n]) for n in range(2 * I)])
            h = gu[:I] / (1 + np.exp(-gu[:I])) * gu[I:]
            s = np.float32(np.abs(h).max() / 448.0)
            q = F.e4m3_encode_rne_sat(h / np.float64(s))
            hd = F.e4m3_decode(q) * np.float64(s)
            assert np.array_equal(q, res.hq[int(res.comp.route_pos[t * K + k])])
            y = np.array([math.fsum(hd * w2d[e][n]) for n in range(tiny.shape.hidden)])
            acc += np.float64(tiny.topk_w[t, k]) * y
        want = F.bf16_bits_to_f64(F.bf16_rne_bits(acc))
        got = F.bf16_bits_to_f64(res.out_bits[t])
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7)
        assert np.all(np.abs(got - want) <= ulp)


def test_forward_mx_one_hot_and_loop():
    shape = MoEShape(8, 256, 128, 4, 2, "topk")
    inp = make_layer_inputs(shape, seed=3, weight_format="mxfp8")
    rng = np.random.default_rng(9)
    # one-hot W13 gate/up rows with random E8M0 exponents
    E, H, I = 4, 256, 128
    jg, ju = rng.integers(0, H, I), rng.integers(0, H, I)
    w13 = np.zeros((E, 2 * I, H), np.uint8)
    w13[:, np.arange(I), jg] = 0x38  # 1.0
    w13[:, I + np.arange(I), ju] = 0x40  # 2.0
    e13 = rng.integers(120, 134, (E, 2 * I, H // 32)).astype(np.uint8)
    res = M.forward_mx(inp.x_bf16, inp.topk_idx, inp.topk_w, w13, e13, inp.w2, inp.w2_scale)
    x = F.bf16_bits_to_f64(inp.x_bf16)
    for p, hb in res.hq.items():
        r = int(res.comp.sorted_route[p])
        t, e = r // 2, int(inp.topk_idx[r // 2, r % 2])
        g = x[t, jg] * 2.0 ** (e13[e, np.arange(I), jg // 32].astype(np.float64) - 127)
        u = 2 * x[t, ju] * 2.0 ** (e13[e, I + np.arange(I), ju // 32].astype(np.float64) - 127)
        want = F.bf16_rne_bits(g / (1 + np.exp(-g)) * u)
        assert np.array_equal(hb, want)
    # dense MX weights: per-route loop
    res = M.forward_mx(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale)
    for t in range(8):
        acc = np.zeros(H)
        for k in range(2):
            e = int(inp.topk_idx[t, k])
            wd = F.e4m3_decode(inp.w13[e]) * np.repeat(2.0 ** (inp.w13_scale[e].astype(np.float64) - 127), 32, 1)
            gu = wd @ x[t]
            h = F.bf16_bits_to_f64(F.bf16_rne_bits(gu[:I] / (1 + np.exp(-gu[:I])) * gu[I:]))
            w2d = F.e4m3_decode(inp.w2[e]) * np.repeat(2.0 ** (inp.w2_scale[e].astype(np.float64) - 127), 32, 1)
            acc += np.float64(inp.topk_w[t, k]) * (w2d @ h)
        want = F.bf16_bits_to_f64(F.bf16_rne_bits(acc))
        got = F.bf16_bits_to_f64(res.out_bits[t])
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7)
        assert np.all(np.abs(got - want) <= ulp)


def _page_figures():
    out = {}
    with open(os.path.join(GOLDEN, "page_figures.txt")) as f:
        for ln in f:
            if ln.strip() and not ln.startswith("#"):
                k, v = ln.split()[:2]
                out[k] = float(v)
    return out


def test_page_figure_dedup_saving():
    """About 43% fewer dispatch bytes for K=6, EP=4, random routing (E=32)."""
    fig = _page_figures()
    E, K, EP = 32, 6, 4
    per = E // EP
    expected_distinct = EP * (1 - math.comb(E - per, K) / math.comb(E, K))
    saving = 1 - expected_distinct / K
    assert abs(saving - fig["dedup_saving_k6_ep4"]) < 0.01
    idx, _ = make_routing(MoEShape(20000, 128, 128, E, K, "topk"), seed=0)
    mc = 1 - np.mean([len(set((row // per).tolist())) for row in idx]) / K
    assert abs(mc - saving) < 0.005


def test_page_figure_fused_fc1_buffer():
    """About 1 GiB of BF16 gate/up avoided per rank at DSV3 EP8 (capacity 2048)."""
    fig = _page_figures()
    ep, capacity, k, two_i = 8, 2048, 8, 2 * CONFIGS["dsv3"].intermediate
    assert ep * capacity * k * two_i * 2 == fig["fused_fc1_bytes"]


def test_every_oracle_function_has_a_pin():
    """Every public function of the oracle (and each optional branch that a
    GPU path is compared with) names the tests that pin it, and those tests
    exist."""
    import importlib
    import inspect
    import re

    from oracle import formats as OF
    for mod, prefix in ((M, ""), (OF, "formats.")):
        for name, fn in inspect.getmembers(mod, inspect.isfunction):
            if name.startswith("_") or fn.__module__ != mod.__name__:
                continue
            assert prefix + name in M.PIN_STATUS, f"{prefix + name} has no PIN_STATUS entry"
    for branch in ("forward_mx[elem=e5m2]", "forward_fp8[bf16_gateup=True]", "fc1_swiglu_requant[bf16_gateup=True]"):
        assert branch in M.PIN_STATUS, branch
    for key, text in M.PIN_STATUS.items():
        assert text.startswith("pinned:"), key
        refs = re.findall(r"(test_\w+)::(test_\w+)", text)
        assert refs, f"{key} names no pinning test"
        for module, test in refs:
            mod = importlib.import_module(f"tests.{module}")
            assert callable(getattr(mod, test, None)), f"{key}: {module}::{test} does not exist"
