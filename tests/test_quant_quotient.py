"""The staging quantiser forms x / s without a division per element:

    inv = fl32(1 / s),  q0 = fl32(x * inv),  r = fma(-q0, s, x),  q = fma(r, inv, q0)

for blocks with s = fl32(amax / 448) >= 2^-90 (smaller s divides).  The codes
it stores must be those of the IEEE quotient, RNE_sat_e4m3(fl32(x / s)), the
definition the oracle follows.  This checks that identity on the CPU for
every bf16 x with |x| <= amax, over a sample of the bf16 amax values (all of
them with MOE_FULL_QUOTIENT_CHECK=1, a few minutes), emulating the float32
steps exactly:
  - q0 * s, r * inv and x - q0 * s are exact in float64 (24-bit by 24-bit
    products; x and q0 * s are within a factor of two);
  - q0 + r * inv may round twice in float64, which can only show as a float64
    sum lying exactly on a float32 midpoint; those cases are settled with
    exact rationals.
"""

import os
from fractions import Fraction

import numpy as np

from oracle.formats import e4m3_encode_rne_sat

S_MIN = np.float32(2.0 ** -90)


def _rn32(v: Fraction) -> np.float32:
    """Nearest float32 to a rational, ties to even (normal and subnormal)."""
    if v == 0:
        return np.float32(0.0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (max(e, -126) - 23)
    m = a / ulp
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return np.float32((1 if v > 0 else -1) * float(n * ulp))


def _quotients(x: np.ndarray, s: np.float32, sign_fix: bool = True) -> np.ndarray:
    """The kernel's float32 quotients of x by s (s >= S_MIN), given the sign
    of x (the sums alone turn x = -0 into +0)."""
    inv = np.float32(1.0) / s
    with np.errstate(invalid="ignore"):
        q0 = x * inv
    r = (x.astype(np.float64) - q0.astype(np.float64) * np.float64(s)).astype(np.float32)
    t = q0.astype(np.float64) + r.astype(np.float64) * np.float64(inv)
    q = t.astype(np.float32)
    back = q.astype(np.float64)
    tie = (back != t) & (np.abs(t - back) == np.spacing(np.abs(q)).astype(np.float64) / 2)
    for i in np.nonzero(tie)[0]:
        q[i] = _rn32(Fraction(float(q0[i])) + Fraction(float(r[i])) * Fraction(float(inv)))
    return np.copysign(q, x) if sign_fix else q


def test_division_free_quotient_gives_the_ieee_codes():
    step = 1 if os.environ.get("MOE_FULL_QUOTIENT_CHECK") == "1" else 8
    amax_bits = np.arange(1, 0x7f80, step, dtype=np.uint32)  # positive finite bf16
    amaxs = (amax_bits << 16).view(np.float32)
    xb = np.arange(0, 0x10000, dtype=np.uint32)
    xb = xb[((xb >> 7) & 0xff) != 0xff]  # finite bf16, both signs
    xall = (xb << 16).view(np.float32)
    xall = xall[np.argsort(np.abs(xall), kind="stable")]
    xabs = np.abs(xall)
    checked = 0
    for amax in amaxs:
        s = np.float32(amax / np.float32(448.0))
        if s < S_MIN:
            continue
        x = xall[:np.searchsorted(xabs, amax, side="right")]
        want = x / s  # IEEE float32 division
        got = _quotients(x, s)
        # -0 == +0 in float comparison: the sign bits are compared too
        diff = (want != got) | (np.signbit(want) != np.signbit(got))
        if diff.any():
            wc = e4m3_encode_rne_sat(want[diff].astype(np.float64))
            gc = e4m3_encode_rne_sat(got[diff].astype(np.float64))
            bad = np.nonzero(wc != gc)[0]
            assert bad.size == 0, (float(amax), float(x[diff][bad[0]]))
        checked += x.size
    assert checked > 10_000_000


def test_a_plausible_mistake_is_caught():
    """Without the correction step (q = fl32(x * inv)) some codes differ."""
    found = False
    for bits in range(0x3f80, 0x4400, 3):
        amax = np.float32(np.uint32(bits << 16).view(np.float32))
        s = np.float32(amax / np.float32(448.0))
        xb = np.arange(0x0000, 0x7f80, dtype=np.uint32)
        x = (xb << 16).view(np.float32)
        x = x[x <= amax]
        crude = x * (np.float32(1.0) / s)
        if np.any(e4m3_encode_rne_sat((x / s).astype(np.float64)) != e4m3_encode_rne_sat(crude.astype(np.float64))):
            found = True
            break
    assert found


def test_negative_zero_keeps_its_code():
    """x = -0 must give code 0x80 (the IEEE quotient is -0); the correction
    sums alone give +0 (code 0x00)."""
    x = np.array([-0.0, 0.0, -1.0, 1.0], np.float32)
    s = np.float32(np.float32(1.0) / np.float32(448.0))
    assert list(e4m3_encode_rne_sat(_quotients(x, s).astype(np.float64))[:2]) == [0x80, 0x00]
    assert list(e4m3_encode_rne_sat((x / s).astype(np.float64))[:2]) == [0x80, 0x00]
    assert e4m3_encode_rne_sat(_quotients(x, s, sign_fix=False).astype(np.float64))[0] == 0x00
