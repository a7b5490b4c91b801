"""CPU emulation of the FP8 GEMMs' block-scale promotion (no GPU).

One output of the FP8 block-scale GEMMs is sum_kb F_kb * P_kb, where F_kb =
sx * sw is the product of the K-block's activation and weight scales (float32)
and P_kb the product of its e4m3 codes.  The kernels keep the accumulator in
units of the current block's scale mantissa times a running power of two
(``promo_step`` in ``csrc/moe_device.h``): per K-block they multiply it by a
ratio below 4 in magnitude, add P_kb scaled by the E8M0 factor 2^(e - ref) of
the MFMA, and at the end form ldexp(acc * m, ref).

This file replays that recursion step by step in float32 (numpy, the same
operations in the same order; the MFMA's sum P_kb rounded once to float32) on
rows whose block scales span the whole float32 range -- zero blocks,
subnormal scales, neighbours 2^100 apart -- and compares with the exact sum.
It also replays the carry rule the kernels used before (a block whose scale
product is below 2^-100 keeps the previous product), which these rows break.
"""

import math
from fractions import Fraction

import numpy as np

from oracle import formats as F

f32 = np.float32


def _frexp(x):
    """(mantissa in [0.5, 1), exponent) of a float32, 0 -> (0, 0); exact."""
    m, e = math.frexp(float(x))
    return f32(m), int(e)


def _rcp(x):
    return f32(f32(1.0) / f32(x))


def promo_emulated(sx, sw, P):
    """The kernels' recursion (promo_step + the scaled MFMA + the final ldexp)."""
    acc = f32(0.0)
    pm, pe = f32(0.0), 0
    for kb in range(len(P)):
        mx, ex = _frexp(sx[kb])
        mw, ew = _frexp(sw[kb])
        m = f32(mx * mw)
        e = ex + ew
        if m == 0:
            r, sh = f32(1.0), 0
        elif pm == 0:
            r, sh = f32(0.0), 127
            pm, pe = m, e
        else:
            ref = max(pe, e)
            r = f32(math.ldexp(float(f32(pm * _rcp(m))), pe - ref))
            pm, pe = m, ref
            sh = max(127 + e - ref, 0)
        # the MFMA: acc * r (VALU), plus the block's code product at 2^(sh - 127)
        acc = f32(f32(acc * r) + f32(math.ldexp(float(P[kb]), sh - 127)))
    if pm == 0:
        return f32(0.0)
    return f32(math.ldexp(float(f32(acc * pm)), pe))


def carry_emulated(sx, sw, P):
    """The earlier rule: acc kept divided by F_kb, a product below 2^-100
    carrying the previous one."""
    acc, pf = f32(0.0), f32(1.0)
    with np.errstate(over="ignore", invalid="ignore"):
        return _carry(sx, sw, P, acc, pf)


def _carry(sx, sw, P, acc, pf):
    for kb in range(len(P)):
        fn = f32(sx[kb] * sw[kb])
        fn = fn if abs(fn) >= 2.0 ** -100 else pf
        r = f32(pf * _rcp(fn)) if kb > 0 else f32(0.0)
        acc = f32(f32(acc * r) + f32(P[kb]))
        pf = fn
    return f32(acc * pf)


def exact(sx, sw, P):
    return sum(Fraction(float(a)) * Fraction(float(b)) * Fraction(float(p)) for a, b, p in zip(sx, sw, P))


def _rows(seed=0, kbs=56):
    """Block scales of every kind: O(1), spread over 2^-40..2^20, one block
    near the old 2^-100 carry bound among O(1) blocks, whole rows below
    2^-100, subnormal scales, zero blocks, and neighbours 2^100 apart."""
    rng = np.random.default_rng(seed)
    codes = F.e4m3_decode(np.arange(0, 0x7E, dtype=np.uint8))
    out = []

    def P():  # a K-block's code product: 128 e4m3 x e4m3 products
        a = rng.choice(codes, 128) * rng.choice([-1, 1], 128)
        b = rng.choice(codes, 128) * rng.choice([-1, 1], 128)
        return f32(float(np.dot(a, b)))  # summed exactly in float64, rounded once

    def row(sx, sw):
        out.append((np.asarray(sx, f32), np.asarray(sw, f32), [P() for _ in range(len(sx))]))

    u = lambda n: rng.uniform(1e-3, 1e-2, n)  # noqa: E731
    row(u(kbs), u(kbs))
    row(u(kbs) * np.exp2(rng.integers(-40, 21, kbs)), u(kbs))
    sx = u(kbs)
    sx[kbs // 2] = 2.0 ** -96
    row(sx, u(kbs) * 2.0 ** -6)
    row(u(kbs) * 1e-26, u(kbs))  # every product below 2^-100
    row(np.full(kbs, 2.0 ** -140), u(kbs))  # subnormal activation scales
    sx = u(kbs)
    sx[::3] = 0.0  # zero blocks (their codes may be anything: they add nothing)
    row(sx, u(kbs))
    sx = u(kbs)
    sx[0] = 0.0
    row(sx, u(kbs))  # the sum starts at a later block
    sx = u(kbs)
    sx[1::2] *= 2.0 ** -100  # neighbours 2^100 apart, both ways
    row(sx, u(kbs))
    sx = u(kbs)
    sx[:kbs // 2] *= 2.0 ** 60
    sx[kbs // 2:] *= 2.0 ** -60
    row(sx, u(kbs))
    row(np.zeros(kbs), u(kbs))  # every block zero: the output is 0
    return out


def test_promotion_matches_exact_sums():
    for sx, sw, P in _rows():
        want = exact(sx, sw, P)
        got = promo_emulated(sx, sw, P)
        bound = sum(abs(Fraction(float(a)) * Fraction(float(b)) * Fraction(float(p)))
                    for a, b, p in zip(sx, sw, P))
        # 2^-20 of the sum of magnitudes covers float32 rounding over 56
        # blocks (ratio, product, sum) and the float32 range of the result
        tiny = Fraction(2) ** -149
        assert abs(Fraction(float(got)) - want) <= bound * Fraction(1, 2 ** 20) + tiny, (float(got), float(want))
        if bound == 0:
            assert got == 0


def test_the_earlier_carry_rule_is_caught():
    """The carry rule gets rows with products below 2^-100 wrong by many
    orders of magnitude; the promotion test above must not accept it."""
    bad = 0
    for sx, sw, P in _rows():
        want = exact(sx, sw, P)
        got = carry_emulated(sx, sw, P)
        bound = sum(abs(Fraction(float(a)) * Fraction(float(b)) * Fraction(float(p)))
                    for a, b, p in zip(sx, sw, P))
        if not np.isfinite(got) or abs(Fraction(float(got)) - want) > bound * Fraction(1, 2 ** 20) + Fraction(2) ** -149:
            bad += 1
    assert bad >= 2
