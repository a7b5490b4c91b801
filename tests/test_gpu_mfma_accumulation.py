"""Accumulation error of the FP8 GEMM's MFMA, measured through the layer.

One K-block (H = 128) and unit block scales make the FC1 GEMM's FP32 gate/up
output (the unfused FC1's MOE_REGION_GATEUP) exactly one
16x16x128 f8f6f4 MFMA per output: each value is the MFMA's sum of 128 e4m3
products.  Every product is exact in float64, so ``math.fsum`` gives the exact
sum; the test measures how far the MFMA's FP32 result lies from it, on random
codes (products spread over 2^-18 .. 2^17.6) and on rows built so that a large
partial sum hides a small term until it cancels.

Reading (measured here on MI355X): the MFMA does not sum its products
exactly.  On random codes its result differs from the exact sum by up to
2^-11.2 of the largest product, with both signs equally often (a rounding, not
a truncation); 0.07% of the results are the correctly rounded sum.  In the
hidden-term rows a product 2^-14.8 below the largest (7 beside 448 * 448) is
lost, one 2^-10.8 below (112) is kept.  No single alignment of the products
to the largest exponent with a fixed number of fraction bits reproduces the
random results, so the bound used is the measured one with margin:
    |MFMA result - exact sum| <= 2^-10 * max_k |a_k * b_k|.

The activation rows are e4m3 values with one +-448 per 128-block, so the
staged 1x128 scale is amax / 448 = 1 and the staged codes are the values
themselves; the weights carry block scale 1.  The promotion's final multiply
(mantissa product 1/4, then 2^2) is then exact.

The bound found here is the one the unfused gate/up check of
``test_gpu_parity`` builds on.
"""

import math

import numpy as np
import pytest
import torch

from oracle.formats import bf16_rne_bits, e4m3_decode
from mixture_experts_ffn_route_amd import _lib as L
from mixture_experts_ffn_route_amd.harness import make_layer, run_forward, to_device
from synthetic import MoEShape
from synthetic.workloads import LayerInputs

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
# |MFMA result - exact sum| <= MFMA_BETA * max_k |a_k b_k|, per output
MFMA_BETA = 2.0 ** -10

_FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)  # e4m3 codes but NaN


def _code(v):
    """e4m3 code of an exactly representable value."""
    vals = e4m3_decode(_FINITE)
    idx = np.where(vals == v)[0]
    assert idx.size, v
    return _FINITE[idx[0]]


def _inputs(rows_codes, w_codes):
    """Layer inputs: T rows of activation codes [T, 128], one expert with
    gate/up weight codes [256, 128] and unit scales; I = 128, top-1."""
    T = rows_codes.shape[0]
    shape = MoEShape(T, 128, 128, 1, 1, "topk")
    x = e4m3_decode(rows_codes)
    inp = LayerInputs(shape, "fp8_block", bf16_rne_bits(x), np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32),
                      w_codes[None].astype(np.uint8), np.ones((1, 2, 1), np.float32),
                      np.full((1, 128, 128), _code(1.0), np.uint8), np.ones((1, 1, 1), np.float32))
    return shape, inp


def _measure(rows_codes, w_codes):
    shape, inp = _inputs(rows_codes, w_codes)
    dev = to_device(inp)
    layer = make_layer(shape, dev, flags=L.MOE_FLAG_CHECK_ROUTES | L.MOE_FLAG_UNFUSED_FC1)
    run_forward(layer, dev)
    torch.cuda.synchronize()
    assert layer.status() == 0
    T = rows_codes.shape[0]
    gu = layer.region("gateup", torch.float32)[: T * 256].view(T, 256).cpu().numpy().astype(np.float64)
    # rows stay in token order (one expert, ascending route id)
    x = e4m3_decode(rows_codes)
    w = e4m3_decode(w_codes)
    exact = np.array([[math.fsum(x[t] * w[n]) for n in range(256)] for t in range(T)])
    pmax = np.max(np.abs(x)[:, None, :] * np.abs(w)[None, :, :], axis=2)
    err = np.abs(gu - exact)
    ratio = np.where(pmax > 0, err / np.where(pmax > 0, pmax, 1), 0.0)
    assert np.all(err[pmax == 0] == 0)
    # FP32 rounding of the exact sum, for the "correctly rounded" count
    rounded = exact.astype(np.float32).astype(np.float64)
    return gu, exact, ratio, np.mean(gu == rounded)


def _rows_with_448(rng, T):
    codes = rng.choice(_FINITE, size=(T, 128))
    codes[:, 0] = np.where(rng.random(T) < 0.5, _code(448.0), _code(-448.0))
    return codes


def test_mfma_sum_of_random_e4m3_products():
    rng = np.random.default_rng(0)
    rows = _rows_with_448(rng, 128)
    w = rng.choice(_FINITE, size=(256, 128))
    gu, exact, ratio, exact_frac = _measure(rows, w)
    print(f"random codes: max |err| / max|p| = 2^{np.log2(ratio.max()):.2f}, correctly rounded {exact_frac:.4f}")
    assert ratio.max() <= MFMA_BETA


def test_mfma_sum_with_hidden_small_terms():
    """Rows of 63 products of +448*448, one small product, 64 of -448*448:
    a running FP32 sum passes 2^24 before the large terms cancel, so a
    summation that rounds its partial sums to FP32 loses the small term."""
    T = 64
    rng = np.random.default_rng(1)
    rows = np.full((T, 128), _code(448.0), np.uint8)
    small_vals = [1.0, 0.5, 0.25, 2.0 ** -6, 1.5, 3.0]
    w = np.zeros((256, 128), np.uint8)
    for n in range(256):
        perm = rng.permutation(128)
        w[n, perm[:63]] = _code(448.0)
        w[n, perm[63:127]] = _code(-448.0)
        w[n, perm[127]] = _code(small_vals[n % len(small_vals)])
    gu, exact, ratio, exact_frac = _measure(rows, w)
    print(f"hidden small terms: max |err| / max|p| = 2^{np.log2(max(ratio.max(), 2.0 ** -60)):.2f}, "
          f"correctly rounded {exact_frac:.4f}, max |err| = {np.abs(gu - exact).max():.3e}")
    assert ratio.max() <= MFMA_BETA
