"""Pins the oracle's lightning-indexer score.

Definition ('DeepSeek-V4' paper page, section 2.3.1, index-score equation;
section 2.3.4: the indexer attention is computed in FP4):
    I_s = sum_h w_h * ReLU(q_h . K_s)
with q_h and K_s the MXFP4-dequantised indexer query head and key.  The
oracle takes the dot product exactly, rounds it once to fp32 (nearest even)
and folds the heads with a sequential fp32 fma chain acc = fma(w_h, r_h, acc),
h = 0 .. Hi-1.

Pins: exact rational brute force (Python Fractions, values decoded from the
golden E2M1 table and E8M0 = 2^(c-127)) of both the dot product and the whole
fma fold, on random and adversarial inputs (large exponent spread,
cancellation, ties, subnormal and overflowing results); the exact rounding
routine against Fractions; special cases (one-hot w, zero w, scaling w by 2);
closeness to a float64 numpy evaluation on N(0,1) inputs.
"""
from fractions import Fraction

import numpy as np
import pytest

from tests.exact import e2m1_table, round_to_f32

TAB = e2m1_table()
RNG = np.random.default_rng(21)


def _nib(codes, i):
    return (int(codes[i // 2]) >> 4) & 15 if i & 1 else int(codes[i // 2]) & 15


def exact_dot(qc, qs, kc, ks) -> Fraction:
    tot = Fraction(0)
    for i in range(128):
        g = i // 32
        qv = TAB[_nib(qc, i)] * Fraction(2) ** (int(qs[g]) - 127)
        kv = TAB[_nib(kc, i)] * Fraction(2) ** (int(ks[g]) - 127)
        tot += qv * kv
    return tot


def exact_score(qc, qs, w, kc, ks) -> float:
    acc = 0.0
    for h in range(len(w)):
        d = round_to_f32(exact_dot(qc[h], qs[h], kc, ks))
        r = d if d > 0 else 0.0
        acc = round_to_f32(Fraction(float(w[h])) * Fraction(r) + Fraction(acc))
    return acc + 0.0


def _rand_codes(n, width_bytes):
    return RNG.integers(0, 256, (n, width_bytes), dtype=np.uint8)


def test_round_pow2_sum_vs_fractions(orc):
    cases = []
    for _ in range(3000):
        n = int(RNG.integers(1, 5))
        S = RNG.integers(-4608, 4609, n)
        base = int(RNG.integers(-250, 230))
        spread = int(RNG.choice([0, 3, 9, 10, 24, 40, 80, 200]))
        E = base + RNG.integers(0, spread + 1, n)
        cases.append((S, np.minimum(E, 250)))
    # hand-made: exact ties, cancellation, subnormal and overflow
    cases += [
        (np.array([2 ** 24 + 1]), np.array([0])),               # tie -> even (down)
        (np.array([2 ** 24 + 3]), np.array([0])),               # tie -> even (up)
        (np.array([2 ** 24 + 1, 1]), np.array([0, -200])),      # tie broken by a tiny term
        (np.array([2 ** 24 + 1, -1]), np.array([0, -200])),
        (np.array([4608, -4608]), np.array([100, 100])),        # exact zero
        (np.array([3, -1]), np.array([-150, -149])),            # subnormal result
        (np.array([1]), np.array([-150])),                      # half of the smallest subnormal
        (np.array([3]), np.array([-151])),
        (np.array([4608, 4608, 4608, 4608]), np.array([250, 250, 250, 250])),   # overflow
    ]
    for S, E in cases:
        exact = sum((Fraction(int(s)) * Fraction(2) ** int(e) for s, e in zip(S, E)), Fraction(0))
        assert orc.round_pow2_sum(S, E) == round_to_f32(exact), (S, E)


def test_head_dot_exact_random(orc):
    for _ in range(300):
        qc, kc = _rand_codes(1, 64)[0], _rand_codes(1, 64)[0]
        qs = RNG.integers(100, 150, 4).astype(np.uint8)
        ks = RNG.integers(100, 150, 4).astype(np.uint8)
        assert orc.head_dot(qc, qs, kc, ks) == round_to_f32(exact_dot(qc, qs, kc, ks))


def test_head_dot_adversarial_scales(orc):
    """Scale exponents spread across the whole E8M0 range."""
    for _ in range(300):
        qc, kc = _rand_codes(1, 64)[0], _rand_codes(1, 64)[0]
        qs = RNG.integers(0, 255, 4).astype(np.uint8)
        ks = RNG.integers(0, 255, 4).astype(np.uint8)
        assert orc.head_dot(qc, qs, kc, ks) == round_to_f32(exact_dot(qc, qs, kc, ks))


def test_head_dot_cancellation(orc):
    """Two groups that cancel exactly except for a small third group."""
    qc = np.zeros(64, np.uint8)
    kc = np.zeros(64, np.uint8)
    qc[0] = 0x07; kc[0] = 0x07            # group 0: 6 * 6
    qc[16] = 0x0F; kc[16] = 0x07          # group 1: -6 * 6
    qc[32] = 0x02; kc[32] = 0x01          # group 2: 1 * 0.5
    qs = np.array([140, 140, 100, 127], np.uint8)
    ks = np.array([127, 127, 100, 127], np.uint8)
    assert orc.head_dot(qc, qs, kc, ks) == round_to_f32(exact_dot(qc, qs, kc, ks)) != 0


def test_index_score_exact_fold(orc):
    for Hi in (1, 8, 16):
        qc = _rand_codes(Hi, 64)
        qs = RNG.integers(118, 130, (Hi, 4)).astype(np.uint8)
        w = RNG.random(Hi).astype(np.float32)
        w[RNG.random(Hi) < 0.2] *= -1           # negative weights too
        kc = _rand_codes(40, 64)
        ks = RNG.integers(118, 130, (40, 4)).astype(np.uint8)
        got = orc.index_score(qc, qs, w, kc, ks)
        for s in range(40):
            ref = exact_score(qc, qs, w, kc[s], ks[s])
            assert got[s] == ref and (got[s] != 0 or not np.signbit(got[s])), (Hi, s)


def test_index_score_special_cases(orc):
    Hi = 8
    qc = _rand_codes(Hi, 64)
    qs = RNG.integers(120, 130, (Hi, 4)).astype(np.uint8)
    kc = _rand_codes(64, 64)
    ks = RNG.integers(120, 130, (64, 4)).astype(np.uint8)
    dots = np.array([[round_to_f32(exact_dot(qc[h], qs[h], kc[s], ks[s])) for s in range(64)]
                     for h in range(Hi)], np.float32)
    for h in range(Hi):
        w = np.zeros(Hi, np.float32); w[h] = 1
        assert np.array_equal(orc.index_score(qc, qs, w, kc, ks), np.maximum(dots[h], 0))
    assert not orc.index_score(qc, qs, np.zeros(Hi, np.float32), kc, ks).any()
    w = RNG.random(Hi).astype(np.float32)
    assert np.array_equal(orc.index_score(qc, qs, 2 * w, kc, ks), 2 * orc.index_score(qc, qs, w, kc, ks))


def test_index_score_close_to_float64(orc):
    q = RNG.standard_normal((8, 128)).astype(np.float32)
    k = RNG.standard_normal((500, 128)).astype(np.float32)
    w = RNG.random(8).astype(np.float32)
    qc, qs = orc.pack_index(q)
    kc, ks = orc.pack_index(k)
    qh = orc.dequant_index(qc, qs).astype(np.float64)
    kh = orc.dequant_index(kc, ks).astype(np.float64)
    ref = (np.maximum(qh @ kh.T, 0) * w[:, None].astype(np.float64)).sum(0)
    got = orc.index_score(qc, qs, w, kc, ks)
    assert np.allclose(got, ref, rtol=1e-6, atol=1e-6)
