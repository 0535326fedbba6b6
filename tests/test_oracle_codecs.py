"""Pins the oracle's element codecs against independent definitions.

* E2M1 decode: the OCP MX v1.0 value table (tests/golden/e2m1_values.json).
* E2M1 encode: brute-force nearest value with ties to the even mantissa code,
  computed with Fractions over that table (not the oracle's exponent logic).
* E4M3 decode / encode: PyTorch's float8_e4m3fn conversion (an independent
  library implementation; it rounds to nearest even, and turns values beyond
  464 into NaN where the oracle saturates at 448).
* E8M0 decode: PyTorch's float8_e8m0fnu.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests.exact import e2m1_nearest_code, e2m1_table


def test_e2m1_decode_table(orc):
    tab = e2m1_table()
    for code in range(16):
        assert Fraction(orc.e2m1_value(code)) == tab[code], code
        assert np.signbit(orc.e2m1_value(code)) == bool(code & 8)


def _e2m1_sweep():
    pos = [Fraction(v) for v in (0, .5, 1, 1.5, 2, 3, 4, 6)]
    xs = set()
    for a, b in zip(pos, pos[1:]):
        mid = (a + b) / 2
        for d in (Fraction(0), Fraction(1, 2 ** 30), -Fraction(1, 2 ** 30)):
            xs.add(mid + d)
        xs.add(a)
    xs.update([Fraction(6), Fraction(7), Fraction(1000), Fraction(1, 2 ** 40)])
    rng = np.random.default_rng(5)
    xs.update(Fraction(float(v)) for v in rng.uniform(0, 8, 2000).astype(np.float32))
    return sorted(xs)


def test_e2m1_encode_brute_force(orc):
    for x in _e2m1_sweep():
        for s in ((1, -1) if x != 0 else (1,)):
            v = s * x
            assert orc.e2m1_encode(float(v)) == e2m1_nearest_code(v) | (8 if s < 0 else 0), v


def test_e2m1_negative_zero(orc):
    assert orc.e2m1_encode(-0.0) == 8
    assert orc.e2m1_encode(-0.1) == 8
    assert orc.e2m1_encode(0.25) == 0      # midpoint 0 / 0.5 -> even (0)


def test_e4m3_decode_all_codes(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        v = orc.e4m3_value(c)
        if np.isnan(ref[c]):
            assert np.isnan(v), c
        else:
            assert v == ref[c] and np.signbit(v) == np.signbit(ref[c]), c


def test_e4m3_encode_vs_torch(orc):
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    vals = np.unique(vals[np.isfinite(vals) & (vals >= 0)])
    xs = list(vals)
    for a, b in zip(vals, vals[1:]):
        m = (a + b) / 2
        xs += [m, np.nextafter(np.float32(m), np.float32(0)), np.nextafter(np.float32(m), np.float32(1e9))]
    xs += list(np.random.default_rng(6).uniform(0, 464, 5000))
    xs += list(2.0 ** np.random.default_rng(7).uniform(-14, 8.8, 5000))
    x = np.array(xs, np.float32)
    x = x[x <= 464]
    x = np.concatenate([x, -x])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(v)) for v in x])
    bad = np.nonzero(got != ref)[0]
    assert len(bad) == 0, [(x[i], got[i], ref[i]) for i in bad[:5]]


def test_e4m3_saturates(orc):
    for v in (448.0, 464.0, 465.0, 480.0, 1e6, 3.0e38):
        assert orc.e4m3_encode(v) == 0x7E
        assert orc.e4m3_encode(-v) == 0xFE
    assert orc.e4m3_value(0x7E) == 448.0


def test_e8m0_decode(orc):
    ref = torch.arange(255, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for c in range(255):
        assert orc.e8m0_value(c) == ref[c], c
    assert np.isnan(orc.e8m0_value(255))
