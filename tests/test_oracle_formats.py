"""Pins for the oracle's number formats (no GPU).

e4m3 / E8M0 decoders are checked exhaustively against torch's float8 dtypes
(library routines) and against values the OCP 8-bit floating point spec fixes;
the encoders against torch's casts on every rounding midpoint and against an
exact-rational brute force where torch would round twice.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden")


def _torch_e4m3(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_e4m3_decode_exhaustive_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(codes)
    ref = _torch_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_decode_spec_values():
    # tests/golden/e4m3_spec_values.txt: code -> value fixed by the OCP FP8 E4M3 definition
    with open(f"{GOLDEN}/e4m3_spec_values.txt") as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    for code, val in rows:
        got = F.e4m3_decode(np.array([int(code, 16)], np.uint8))[0]
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(Fraction(val)), (code, val, got)
            assert math.copysign(1.0, got) == math.copysign(1.0, float(Fraction(val)) if val != "-0" else -0.0)


def test_e8m0_decode_exhaustive_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e8m0_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def _midpoint_cases():
    pos = F.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    v32 = mids.astype(np.float32)
    assert np.array_equal(v32.astype(np.float64), mids)  # midpoints are float32-exact
    up = np.nextafter(v32, np.float32(np.inf))
    dn = np.nextafter(v32, np.float32(0))
    vals = np.concatenate([v32, up, dn, pos.astype(np.float32)])
    return np.concatenate([vals, -vals])


def test_e4m3_encode_midpoints_vs_torch():
    v = _midpoint_cases()
    ours = F.e4m3_encode_rne_sat(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_random_vs_torch_after_clamp():
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(200000) * np.exp2(rng.integers(-14, 10, 200000))).astype(np.float32)
    ours = F.e4m3_encode_rne_sat(v.astype(np.float64))
    ref = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_saturation_and_specials():
    v = np.array([448.0, 449.0, 463.9, 464.0, 1e9, np.inf, -np.inf, -500.0, np.nan, 0.0, -0.0, -1e-30])
    got = F.e4m3_encode_rne_sat(v)
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x00, 0x80, 0x80]


def _brute_e4m3(x: float) -> int:
    """Nearest e4m3 code by exact rational distance, ties to even code."""
    a = Fraction(abs(x))
    best = None
    for c in range(127):
        d = abs(Fraction(float(F.e4m3_decode(np.array([c], np.uint8))[0])) - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    c = 126 if a >= 448 else best[1]
    return c | (0x80 if math.copysign(1.0, x) < 0 else 0)


def test_e4m3_encode_float64_near_midpoints_vs_exact():
    # float64 one ulp around each midpoint: torch would round through float32
    pos = F.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    vals = np.concatenate([np.nextafter(mids, np.inf), np.nextafter(mids, 0), mids])
    got = F.e4m3_encode_rne_sat(vals)
    for x, g in zip(vals[::3], got[::3]):
        assert g == _brute_e4m3(float(x)), x
    for x, g in zip(vals[1::5], got[1::5]):
        assert g == _brute_e4m3(float(x)), x


def test_bf16_rne_float32_inputs_vs_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, 300000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    ours = F.bf16_rne_bits(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def _brute_bf16(x: float) -> float:
    a = Fraction(abs(x))
    if a == 0:
        return math.copysign(0.0, x)
    k = math.floor(math.log2(abs(x)))
    while Fraction(2) ** k > a:
        k -= 1
    while Fraction(2) ** (k + 1) <= a:
        k += 1
    q = Fraction(2) ** max(k - 7, -133)
    n = a // q
    rem = a - n * q
    if rem * 2 > q or (rem * 2 == q and n % 2 == 1):
        n += 1
    r = float(n * q)
    return math.copysign(r, x)


def test_bf16_rne_float64_single_rounding():
    # values just above a bf16 midpoint that a float32 detour would turn into a tie
    rng = np.random.default_rng(11)
    base = rng.integers(0x3F80, 0x4780, 2000).astype(np.uint32) << 16
    lo = base.view(np.float32).astype(np.float64)
    ulp = np.exp2(np.floor(np.log2(lo)) - 7)
    mid = lo + ulp / 2
    vals = np.concatenate([mid, np.nextafter(mid, np.inf), np.nextafter(mid, 0), -mid * 3.0 ** -40])
    got = F.bf16_bits_to_f64(F.bf16_rne_bits(vals))
    for x, g in zip(vals, got):
        assert g == _brute_bf16(float(x)), x


def test_bf16_overflow_and_subnormals():
    big = (2 - 2.0 ** -8) * 2.0 ** 127
    got = F.bf16_bits_to_f64(F.bf16_rne_bits(np.array([big, np.nextafter(big, 0), 2.0 ** -133, 2.0 ** -134,
                                                       3 * 2.0 ** -135, -0.0])))
    assert got[0] == np.inf
    assert got[1] == (2 - 2.0 ** -7) * 2.0 ** 127
    assert got[2] == 2.0 ** -133
    assert got[3] == 0.0  # tie to even (zero)
    assert got[4] == 2.0 ** -133
    assert got[5] == 0.0 and np.signbit(got[5])


def test_e5m2_decode_exhaustive_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e5m2_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e5m2_decode_spec_values():
    # tests/golden/e5m2_spec_values.txt: code -> value fixed by the OCP FP8 E5M2 definition
    with open(f"{GOLDEN}/e5m2_spec_values.txt") as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    for code, val in rows:
        got = F.e5m2_decode(np.array([int(code, 16)], np.uint8))[0]
        if val == "nan":
            assert math.isnan(got)
        elif val in ("inf", "-inf"):
            assert got == float(val)
        else:
            assert got == float(Fraction(val)), (code, val, got)
            assert math.copysign(1.0, got) == (-1.0 if val.startswith("-") else 1.0)
