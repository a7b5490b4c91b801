"""Number formats, decoded and encoded from their bit-level definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

* OCP 8-bit floating point E4M3 ("fn" flavour: no infinities, 0x7F/0xFF are
  NaN, largest finite magnitude 448) -- the e4m3 format of the FP8 block-scale
  path in "feat(moe_ep): add SM90 push FP8 mega-MoE backend for Hopper"
  (Description: FC1 with fused SwiGLU + 1x128 quantization) and the MXFP8
  weights of "feat(moe_ep): MXFP8 x BF16 integration" (Description).
* OCP 8-bit floating point E5M2 (IEEE-like: exponent field 31 is inf or NaN,
  largest finite magnitude 57344) -- the second MXFP8 element type of
  "feat(moe_ep): MXFP8 x BF16 integration" (Description).
* OCP MX E8M0 shared scale: value 2**(v - 127), v = 255 is NaN.
* bfloat16: 1 sign, 8 exponent, 7 mantissa bits (the layer's output type).

Encoders round to nearest, ties to even, by exact comparison against the
midpoint of the two neighbouring representable values.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _e4m3_fields(c: np.ndarray) -> np.ndarray:
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


_E4M3_TABLE = _e4m3_fields(np.arange(256, dtype=np.int64))


def e4m3_decode(codes) -> np.ndarray:
    """Decode e4m3 codes (uint8) to float64 from the bit fields.

    sign = bit 7, exponent field e = bits 6..3 (bias 7), mantissa m = bits 2..0.
    e == 0: subnormal (m / 8) * 2**-6; otherwise (1 + m / 8) * 2**(e - 7);
    codes 0x7F and 0xFF are NaN.  (The 256 values are evaluated once from the
    fields and looked up.)
    """
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def _e5m2_fields(c: np.ndarray) -> np.ndarray:
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    m = c & 0x3
    mag = np.where(e == 0, (m / 4.0) * 2.0 ** -14, (1.0 + m / 4.0) * np.exp2(e - 15.0))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return sign * mag


_E5M2_TABLE = _e5m2_fields(np.arange(256, dtype=np.int64))


def e5m2_decode(codes) -> np.ndarray:
    """Decode e5m2 codes (uint8) to float64 from the bit fields.

    sign = bit 7, exponent field e = bits 6..2 (bias 15), mantissa m = bits 1..0.
    e == 0: subnormal (m / 4) * 2**-14; e == 31: +-inf (m == 0) or NaN;
    otherwise (1 + m / 4) * 2**(e - 15).
    """
    return _E5M2_TABLE[np.asarray(codes, dtype=np.uint8)]


def e8m0_decode(codes) -> np.ndarray:
    """Decode E8M0 scale bytes to float64: 2**(v - 127); v == 255 is NaN."""
    v = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    return np.where(v == 255, np.nan, np.exp2(v - 127.0))


# Non-negative finite e4m3 magnitudes, indexed by code 0..126 (monotonic).
_E4M3_POS = e4m3_decode(np.arange(127, dtype=np.uint8))


def e4m3_encode_rne_sat(values) -> np.ndarray:
    """Round float64 values to e4m3 codes: nearest, ties to even, saturating.

    Magnitudes at or above 448 (including +-inf) map to +-448; NaN maps to
    0x7F.  The sign bit is kept for negative zero and for negative values that
    round to zero.
    """
    v = np.asarray(values, dtype=np.float64)
    a = np.abs(v)
    lo = np.searchsorted(_E4M3_POS, a, side="right") - 1  # largest code with value <= a
    lo = np.clip(lo, 0, 126)
    hi = np.minimum(lo + 1, 126)
    mid = (_E4M3_POS[lo] + _E4M3_POS[hi]) * 0.5  # exact: neighbours are dyadic
    up = (a > mid) | ((a == mid) & ((lo & 1) == 1))
    code = np.where(up, hi, lo)
    code = np.where(a >= E4M3_MAX, 126, code)
    code = code.astype(np.uint8) | np.where(np.signbit(v), np.uint8(0x80), np.uint8(0))
    return np.where(np.isnan(v), np.uint8(0x7F), code).astype(np.uint8)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_rne_bits(values) -> np.ndarray:
    """Round float64 values once to bfloat16 (nearest, ties to even); return bits.

    The quantum of a value in [2**(k-1), 2**k) is 2**(k-8) (8 significant
    bits), never below the subnormal quantum 2**-133.  Overflow goes to inf.
    """
    v = np.asarray(values, dtype=np.float64)
    a = np.abs(v)
    _, k = np.frexp(a)  # a = f * 2**k, f in [0.5, 1)
    q = np.exp2(np.maximum(k.astype(np.float64) - 8.0, -133.0))
    n = np.floor(a / q)
    frac = a / q - n
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(n, 2.0) == 1.0))
    r = (n + up) * q
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    r = np.where(np.isinf(a), np.inf, r)
    r = np.where(np.signbit(v), -r, r)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.isnan(v), np.uint16(0x7FC0), bits).astype(np.uint16)
