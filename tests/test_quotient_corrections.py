"""The K-cache write path takes its E4M3 codes from the correctly rounded
binary32 quotient key / scale, computed without a division per element:
y = RN(1 / scale) once per key, then q0 = RN(x y) and two fma corrections
q <- RN(q + RN(x - scale q) y).  This checks that recipe in exact rational
arithmetic (each fma rounded once, from the exact value) against RN(x / scale),
on random pairs and on quotients at and one ulp beside E4M3 midpoints, over
the scale range where the kernel uses it ([2^-80, 2^80])."""
import random
import struct
from fractions import Fraction as Fr

import numpy as np


def rn32(v: Fr) -> float:
    """Round a rational to the nearest binary32, ties to even (normal range)."""
    if v == 0:
        return 0.0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fr(2) ** e > a:
        e -= 1
    while Fr(2) ** (e + 1) <= a:
        e += 1
    ulp = Fr(2) ** (max(e, -126) - 23)
    m = a / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and fl % 2 == 1):
        fl += 1
    return (1 if v > 0 else -1) * float(fl * ulp)


def f32(x):
    return struct.unpack("f", struct.pack("f", x))[0]


def corrected_quotient(x, s):
    y = rn32(Fr(1) / Fr(s))
    q = rn32(Fr(x) * Fr(y))
    for _ in range(2):
        r = rn32(Fr(x) - Fr(s) * Fr(q))
        q = rn32(Fr(r) * Fr(y) + Fr(q))
    return q


def test_two_corrections_give_the_correctly_rounded_quotient():
    rng = random.Random(17)
    n = 0
    while n < 3000:
        m = f32(abs(rng.gauss(0, 1)) * 2.0 ** rng.randint(-70, 70)) or 1.0
        s = rn32(Fr(m) / 448)
        if not (2.0 ** -80 <= s <= 2.0 ** 80):
            continue
        if n % 3 == 0:  # at or one ulp beside an E4M3 midpoint
            mid = (rng.randint(16, 31) + 0.5) * 2.0 ** rng.randint(-9, 4)
            x = rn32(Fr(mid) * Fr(s))
            step = rng.choice([0, 1, -1])
            if step:
                x = float(np.nextafter(np.float32(x), np.float32(step * np.inf)))
        else:
            x = f32(rng.uniform(-1, 1) * m)
        if abs(x) < 2.0 ** -100:
            continue
        assert corrected_quotient(x, s) == rn32(Fr(x) / Fr(s)), (x, s)
        n += 1
