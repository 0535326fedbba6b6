"""Pins the oracle's group quantisers (main FP4, MXFP4 indexer, 8-bit SWA).

Pins: the scale rules checked as properties (for MXFP4: 2^e <= amax/4 <
2^(e+1); for the main format: scale = E4M3 rounding of fl32(amax/6), the
rounding taken by PyTorch's float8_e4m3fn), element codes checked against the
brute-force nearest-value encoder of test_oracle_codecs / PyTorch, round-trip
error bounds, idempotence, exact representability of the dequantised values
in bf16 and fp16, zero groups, and the 2,688 = 448 x 6 saturation point
('KV cache diet' page).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests.exact import e2m1_nearest_code

RNG = np.random.default_rng(11)


def _nib(codes, i):
    return (codes[i // 2] >> 4) & 15 if i & 1 else codes[i // 2] & 15


def _groups(n, width, scale_spread=True):
    x = RNG.standard_normal((n, width)).astype(np.float32)
    if scale_spread:
        x *= (2.0 ** RNG.integers(-20, 12, (n, 1))).astype(np.float32)
    return x


def test_main_scale_rule_and_codes(orc):
    x = _groups(200, 512)
    codes, scales = orc.pack_main(x)
    for r in range(0, 200, 7):
        for g in range(32):
            grp = x[r, 16 * g:16 * g + 16]
            amax = np.float32(np.max(np.abs(grp)))
            t = np.float32(amax / np.float32(6))
            ref_sc = int(torch.tensor([float(t)], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)[0])
            assert scales[r, g] == ref_sc
            s = np.float32(orc.e4m3_value(ref_sc))
            for i in range(16):
                c = _nib(codes[r], 16 * g + i)
                if s == 0:
                    assert c == 0
                else:
                    y = np.float32(grp[i] / s)
                    assert c == e2m1_nearest_code(Fraction(float(y))), (r, g, i)


def test_main_roundtrip_bound_idempotent_exact(orc):
    x = _groups(300, 512)
    codes, scales = orc.pack_main(x)
    xh = orc.dequant_main(codes, scales)
    s = np.repeat(np.array([[orc.e4m3_value(int(c)) for c in row] for row in scales]), 16, axis=1)
    amax = np.repeat(np.abs(x).reshape(300, 32, 16).max(-1), 16, axis=1)
    ok = (s >= 2.0 ** -6) & (s < 448)
    # with a normal, unsaturated E4M3 scale the error is at most one E2M1 step (= s, between 4s and 6s)
    assert np.all(np.abs(x - xh)[ok] <= s[ok] * 1.0001)
    # a subnormal or saturated (448) scale may clip the group: error below max(s, amax - 6s)
    lim = np.maximum(s, amax - 6 * s)
    assert np.all(np.abs(x - xh)[~ok] <= lim[~ok] * 1.0001)
    # idempotent: quantising the dequantised values reproduces the codes
    c2, s2 = orc.pack_main(xh)
    norm = (s >= 2.0 ** -6).reshape(300, 32, 16)[:, :, 0]
    assert np.array_equal(s2[norm], scales[norm])
    # dequantised values are exact in bf16 and in fp16
    assert np.array_equal(xh.astype(np.float16).astype(np.float32), xh)
    b = torch.from_numpy(xh).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(b, xh)


def test_main_zero_and_tiny_groups(orc):
    x = np.zeros((2, 512), np.float32)
    x[1, :16] = 2.0 ** -14         # amax/6 < 2^-10: scale encodes to zero
    c, s = orc.pack_main(x)
    assert not c.any() and not s.any()
    assert not orc.dequant_main(c, s).any()


def test_index_scale_rule_and_codes(orc):
    x = _groups(200, 128)
    codes, scales = orc.pack_index(x)
    for r in range(200):
        for g in range(4):
            grp = x[r, 32 * g:32 * g + 32]
            amax = Fraction(float(np.max(np.abs(grp))))
            e = int(scales[r, g]) - 127
            assert Fraction(2) ** e <= amax / 4 < Fraction(2) ** (e + 1)
            for i in range(32):
                c = _nib(codes[r], 32 * g + i)
                assert c == e2m1_nearest_code(Fraction(float(grp[i])) / Fraction(2) ** e)


def test_index_roundtrip_and_zero(orc):
    x = _groups(200, 128)
    codes, scales = orc.pack_index(x)
    xh = orc.dequant_index(codes, scales)
    unit = np.repeat(2.0 ** (scales.astype(np.int64) - 127), 32, axis=1)
    assert np.all(np.abs(x - xh) <= 2 * unit)
    c2, s2 = orc.pack_index(xh)
    assert np.array_equal(s2, scales) and np.array_equal(c2 & 0x77, codes & 0x77)
    c, s = orc.pack_index(np.zeros((1, 128), np.float32))
    assert not c.any() and np.all(s == 0)


def test_swa_scale_rule_and_codes(orc):
    x = _groups(100, 512)
    codes, scales = orc.pack_swa(x)
    for r in range(0, 100, 3):
        for g in range(32):
            grp = x[r, 16 * g:16 * g + 16]
            amax = Fraction(float(np.max(np.abs(grp))))
            e = int(scales[r, g]) - 127
            assert Fraction(2) ** e <= amax / 256 < Fraction(2) ** (e + 1)
            y = (grp.astype(np.float64) * 2.0 ** -e).astype(np.float32)
            ref = torch.from_numpy(np.clip(y, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(codes[r, 16 * g:16 * g + 16], ref)


def test_swa_roundtrip(orc):
    x = _groups(100, 512)
    codes, scales = orc.pack_swa(x)
    xh = orc.dequant_swa(codes, scales)
    amax = np.repeat(np.abs(x).reshape(100, 32, 16).max(-1), 16, axis=1)
    # 3 mantissa bits: relative step 2^-3 at worst; saturation costs < amax/8
    assert np.all(np.abs(x - xh) <= amax / 8 + 1e-30)
    b = torch.from_numpy(xh).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(b, xh)
