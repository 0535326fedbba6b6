"""Exact-arithmetic helpers for the oracle pins (Python integers / Fractions).

Written independently of the oracle's C code: rounding here goes through
Python's arbitrary-precision integers, not through a fixed-point accumulator.
"""
from fractions import Fraction
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f32(x) -> float:
    return float(np.float32(x))


def round_to_f32(v: Fraction) -> float:
    """Correctly rounded (nearest, ties to even) fp32 value of a rational."""
    if v == 0:
        return 0.0
    sign = -1.0 if v < 0 else 1.0
    a = abs(v)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp_e = max(e - 23, -149)
    scaled = a / (Fraction(2) ** ulp_e)          # value in units of the ulp
    q, r = divmod(scaled.numerator, scaled.denominator)
    twice = 2 * r
    if twice > scaled.denominator or (twice == scaled.denominator and q % 2 == 1):
        q += 1
    val = q * (2.0 ** ulp_e) if ulp_e >= -1074 else 0.0
    if val >= 2.0 ** 128:
        return sign * float("inf")
    return sign * float(np.float32(val))


def e2m1_table():
    pos = golden("e2m1_values.json")["positive_values_by_code"]
    return [Fraction(v) for v in pos] + [-Fraction(v) for v in pos]


def e2m1_nearest_code(x: Fraction) -> int:
    """Brute force: the E2M1 code whose value is nearest to x (ties to the code
    with an even mantissa bit), saturating at +-6; sign bit copied from x."""
    pos = [Fraction(v) for v in golden("e2m1_values.json")["positive_values_by_code"]]
    sign = 8 if x < 0 else 0
    a = abs(x)
    best = None
    for c, v in enumerate(pos):
        d = abs(a - v)
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return sign | best[1]
