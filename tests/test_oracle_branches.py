"""Branch-level pins of the oracle (no GPU): the e5m2 element type of the
MXFP8 x BF16 layer and the BF16 gate/up mode of the FP8 layer.

* ``forward_mx(elem="e5m2")``: one-hot e5m2 W13 and W2 closed forms whose
  values are decoded here from the OCP E5M2 bit fields (not through the
  oracle's decoder), and a per-route loop over dense e5m2 weights with exact
  sums.  The MX variant of "feat(moe_ep): MXFP8 x BF16 integration"
  (PR #4604, Description: E4M3/E5M2 MXFP8 weights, MXFP8 decoding, BF16
  activations).
* ``forward_fp8(bf16_gateup=True)``: a one-hot W13 closed form in which the
  gate and up values change when rounded to BF16, so the rounding's place
  (gate/up, before SwiGLU) is visible in the h codes.  The unfused FC1 of
  "feat(moe_ep): add SM90 push FP8 mega-MoE backend for Hopper" (PR #4069,
  Description, fused-FC1 bullet) stores a BF16 gate/up intermediate.

Each pin is run once more against a deliberately broken copy of the oracle
function it guards (the mistake planted on the CPU, in a monkeypatched
oracle), and must fail there: a pin that a plausible mistake passes pins
nothing.
"""

import math

import numpy as np
import pytest

from oracle import formats as F
from oracle import moe_ref as M
from synthetic import MoEShape, make_layer_inputs


def _e5m2_value(code: int) -> float:
    """OCP E5M2 (finite codes only) from the bit fields: sign, exponent bits
    6..2 with bias 15, mantissa bits 1..0; exponent 0 is subnormal."""
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 2) & 0x1F, code & 0x3
    assert e != 31
    return sign * ((m / 4.0) * 2.0 ** -14 if e == 0 else (1.0 + m / 4.0) * 2.0 ** (e - 15))


def _ulp_close(got_bits, want):
    """got (bf16 bits) within one bf16 ulp of the float64 value `want` rounded."""
    w = F.bf16_bits_to_f64(F.bf16_rne_bits(want))
    g = F.bf16_bits_to_f64(got_bits)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(w), 1e-30))) - 7)
    return bool(np.all(np.abs(g - w) <= ulp))


# ----------------------------------------------------------------------------
# forward_mx(elem="e5m2")
# ----------------------------------------------------------------------------

E, H, I = 4, 256, 128
SHAPE_MX = MoEShape(8, H, I, E, 2, "topk")


def _pin_mx_e5m2_one_hot():
    """One-hot e5m2 W13 (gate 0x3c = 1.0, up 0x40 = 2.0) and one-hot e5m2 W2
    with random codes, random E8M0 exponents everywhere."""
    inp = make_layer_inputs(SHAPE_MX, seed=5, weight_format="mxfp8_e5m2")
    rng = np.random.default_rng(11)
    jg, ju = rng.integers(0, H, I), rng.integers(0, H, I)
    w13 = np.zeros((E, 2 * I, H), np.uint8)
    w13[:, np.arange(I), jg] = 0x3C
    w13[:, I + np.arange(I), ju] = 0x40
    e13 = rng.integers(120, 134, (E, 2 * I, H // 32)).astype(np.uint8)
    j2 = rng.integers(0, I, H)
    # e5m2 codes with exponent field 10..19 and any mantissa, either sign
    c2 = ((rng.integers(10, 20, (E, H)) << 2) | rng.integers(0, 4, (E, H))
          | (rng.integers(0, 2, (E, H)) << 7)).astype(np.uint8)
    w2 = np.zeros((E, H, I), np.uint8)
    for e in range(E):
        w2[e, np.arange(H), j2] = c2[e]
    e2 = rng.integers(122, 132, (E, H, I // 32)).astype(np.uint8)
    res = M.forward_mx(inp.x_bf16, inp.topk_idx, inp.topk_w, w13, e13, w2, e2, elem="e5m2")
    x = F.bf16_bits_to_f64(inp.x_bf16)
    T, K = inp.topk_idx.shape
    acc = np.zeros((T, H))
    for p, hb in res.hq.items():
        r = int(res.comp.sorted_route[p])
        t, e = r // K, int(inp.topk_idx[r // K, r % K])
        g = x[t, jg] * 1.0 * np.exp2(e13[e, np.arange(I), jg // 32].astype(np.float64) - 127)
        u = x[t, ju] * 2.0 * np.exp2(e13[e, I + np.arange(I), ju // 32].astype(np.float64) - 127)
        want_h = F.bf16_rne_bits(g / (1 + np.exp(-g)) * u)
        assert np.array_equal(hb, want_h), "h of the e5m2 one-hot W13"
        hd = F.bf16_bits_to_f64(hb)
        vals = np.array([_e5m2_value(int(c)) for c in c2[e]])
        want_y = hd[j2] * vals * np.exp2(e2[e, np.arange(H), j2 // 32].astype(np.float64) - 127)
        assert np.array_equal(res.y[p], want_y), "y of the e5m2 one-hot W2"
        acc[t] += np.float64(inp.topk_w[t, r % K]) * want_y
    assert np.array_equal(res.out_bits, F.bf16_rne_bits(acc)), "combined output"


def _pin_mx_e5m2_loop():
    """Dense e5m2 weights: token by token and slot by slot, exact sums."""
    inp = make_layer_inputs(SHAPE_MX, seed=7, weight_format="mxfp8_e5m2")
    res = M.forward_mx(inp.x_bf16, inp.topk_idx, inp.topk_w, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale,
                       elem="e5m2")
    x = F.bf16_bits_to_f64(inp.x_bf16)
    table = np.array([_e5m2_value(c) if (c >> 2) & 0x1F != 31 else np.nan for c in range(256)])
    T, K = inp.topk_idx.shape
    for t in range(T):
        acc = np.zeros(H)
        for k in range(K):
            e = int(inp.topk_idx[t, k])
            w13d = table[inp.w13[e]] * np.repeat(np.exp2(inp.w13_scale[e].astype(np.float64) - 127), 32, 1)
            gu = np.array([math.fsum(w13d[n] * x[t]) for n in range(2 * I)])
            h = F.bf16_bits_to_f64(F.bf16_rne_bits(gu[:I] / (1 + np.exp(-gu[:I])) * gu[I:]))
            w2d = table[inp.w2[e]] * np.repeat(np.exp2(inp.w2_scale[e].astype(np.float64) - 127), 32, 1)
            y = np.array([math.fsum(w2d[n] * h) for n in range(H)])
            acc += np.float64(inp.topk_w[t, k]) * y
        assert _ulp_close(res.out_bits[t], acc), f"token {t}"


def test_forward_mx_e5m2_one_hot():
    _pin_mx_e5m2_one_hot()


def test_forward_mx_e5m2_per_route_loop():
    _pin_mx_e5m2_loop()


def test_mx_e5m2_pins_catch_element_type_mistakes(monkeypatch):
    """A dequant_mx that decodes W2 (or every weight) as e4m3 fails both pins."""
    orig = M.dequant_mx
    calls = {"n": 0}

    def w2_as_e4m3(codes, e8m0, elem="e4m3"):
        calls["n"] += 1
        # forward_mx decodes W13 then W2 per expert: every second call is W2
        return orig(codes, e8m0, "e4m3" if calls["n"] % 2 == 0 else elem)

    monkeypatch.setattr(M, "dequant_mx", w2_as_e4m3)
    with pytest.raises(AssertionError):
        _pin_mx_e5m2_one_hot()
    calls["n"] = 0
    with pytest.raises(AssertionError):
        _pin_mx_e5m2_loop()
    monkeypatch.setattr(M, "dequant_mx", lambda c, s, elem="e4m3": orig(c, s, "e4m3"))
    with pytest.raises(AssertionError):
        _pin_mx_e5m2_loop()


# ----------------------------------------------------------------------------
# forward_fp8(bf16_gateup=True)
# ----------------------------------------------------------------------------

def _pin_bf16_gateup():
    """One-hot W13 (one code per gate/up row) with float32 scales that are
    not powers of two: gate = x_j * c * s_w exactly in float64, which has more
    than 8 significant bits, so the BF16 rounding of gate and up before SwiGLU
    changes h.  The h codes must be those of the closed form
    requant(silu(bf16(g)) * bf16(u))."""
    Hh, Ih, Ee = 256, 128, 2
    shape = MoEShape(12, Hh, Ih, Ee, 1, "topk")
    inp = make_layer_inputs(shape, seed=13)
    rng = np.random.default_rng(17)
    jg, ju = rng.integers(0, Hh, Ih), rng.integers(0, Hh, Ih)
    cg = (rng.integers(0x28, 0x50, Ih) | (rng.integers(0, 2, Ih) << 7)).astype(np.uint8)
    cu = (rng.integers(0x28, 0x50, Ih) | (rng.integers(0, 2, Ih) << 7)).astype(np.uint8)
    w13 = np.zeros((Ee, 2 * Ih, Hh), np.uint8)
    w13[:, np.arange(Ih), jg] = cg
    w13[:, Ih + np.arange(Ih), ju] = cu
    s13 = rng.uniform(0.3, 3.0, (Ee, 2, Hh // 128)).astype(np.float32)
    res = M.forward_fp8(inp.x_bf16, inp.topk_idx, inp.topk_w, w13, s13, inp.w2, inp.w2_scale, bf16_gateup=True)
    plain = M.forward_fp8(inp.x_bf16, inp.topk_idx, inp.topk_w, w13, s13, inp.w2, inp.w2_scale)
    xq, xs = M.stage_quantize_1x128(inp.x_bf16)
    xd = F.e4m3_decode(xq) * np.repeat(xs.astype(np.float64), 128, axis=1)
    changed = 0
    for p, codes in res.hq.items():
        r = int(res.comp.sorted_route[p])
        t, e = r, int(inp.topk_idx[r, 0])
        g = xd[t, jg] * F.e4m3_decode(cg) * s13[e, 0, jg // 128].astype(np.float64)
        u = xd[t, ju] * F.e4m3_decode(cu) * s13[e, 1, ju // 128].astype(np.float64)
        gb, ub = F.bf16_bits_to_f64(F.bf16_rne_bits(g)), F.bf16_bits_to_f64(F.bf16_rne_bits(u))
        h = gb / (1.0 + np.exp(-gb)) * ub
        s = np.float32(np.abs(h).max() / 448.0)
        want = F.e4m3_encode_rne_sat(h / np.float64(s)) if s > 0 else np.zeros(Ih, np.uint8)
        assert np.array_equal(codes, want), f"h codes of route {r}"
        assert res.hs[p][0] == s
        changed += int(np.sum(codes != plain.hq[p]))
    # the pin can tell the modes apart: BF16 gate/up moves some codes
    assert changed > 0


def test_forward_fp8_bf16_gateup_one_hot():
    _pin_bf16_gateup()


def test_bf16_gateup_pin_catches_misplaced_rounding(monkeypatch):
    """Ignoring the flag, or rounding h (after SwiGLU) instead of gate/up,
    fails the pin."""
    orig = M.fc1_swiglu_requant
    monkeypatch.setattr(M, "fc1_swiglu_requant", lambda x, w, s, bf16_gateup=False: orig(x, w, s, False))
    with pytest.raises(AssertionError):
        _pin_bf16_gateup()

    def round_h(x, w, s, bf16_gateup=False):
        gu = M.fc1_gateup(x, w, s)
        i = gu.shape[1] // 2
        h = M.silu(gu[:, :i]) * gu[:, i:]
        if bf16_gateup:
            h = F.bf16_bits_to_f64(F.bf16_rne_bits(h))
        codes, scales = M.requant_1x128(h)
        return h, codes, scales

    monkeypatch.setattr(M, "fc1_swiglu_requant", round_h)
    with pytest.raises(AssertionError):
        _pin_bf16_gateup()
