"""The quantize kernels' refined quotient (bf16 input, FP4 / Int4 codebooks),
checked in exact rational arithmetic (CPU only).

With rcp within 1 ulp of 1/c1, x = fl(w rcp), r = fma(-c1, x, w) and
xr = fma(r, rcp, x) must equal fl32(w / c1) for every pair of bf16 values
with |w| <= c1 and a normal quotient: the kernels then compare xr with a
switch point exactly, without the division fallback. Each step is emulated
as one correctly rounded binary32 operation on exact rationals; rcp is taken
correctly rounded and one ulp off in each direction.
"""
import random
from fractions import Fraction as F

import pytest


def rn32(q):
    """Nearest binary32 to the rational q (ties to even; gradual underflow)."""
    if q == 0:
        return F(0)
    s = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1
    e = max(e, -126)
    ulp = F(2) ** (e - 23)
    m = a / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        fl += 1
    return s * fl * ulp


def ulp32(v):
    e = v.numerator.bit_length() - v.denominator.bit_length()
    if F(2) ** e > v:
        e -= 1
    return F(2) ** (max(e, -126) - 23)


@pytest.mark.parametrize("seed", [1, 2])
def test_refined_quotient_is_correctly_rounded_on_bf16_pairs(seed):
    rng = random.Random(seed)
    mants = list(range(128, 256))  # bf16 significands (8 bits, leading one)
    checked = 0
    for cm in rng.sample(mants, 12):
        ce = rng.choice((0, 5, -9, 40))
        c1 = F(cm, 128) * F(2) ** ce
        r0 = rn32(1 / c1)
        for rcp in (r0, r0 + ulp32(r0), r0 - ulp32(r0)):
            for wm in rng.sample(mants, 64):
                for we in (0, -1, -4, -11):
                    w = rng.choice((1, -1)) * F(wm, 128) * F(2) ** (ce + we)
                    if abs(w) > c1:
                        continue
                    x = rn32(w * rcp)
                    r = rn32(w - c1 * x)
                    xr = rn32(x + r * rcp)
                    assert xr == rn32(w / c1), (w, c1, rcp)
                    checked += 1
    assert checked > 5000
