"""Pins of the write-path oracle (oracle/compress.py) against what the
mathematics fixes, independent of the oracle's own code:

* compression ('DeepSeek-V4' page, section 2.3.1 and 2.3.2): equal logits
  give the plain mean of the 2m (m for the first entry, m' for the heavily
  compressed branch) rows; a dominant logit selects its row; constant values
  are reproduced for any logits (the weights sum to 1 per channel); a bias
  of ln 3 on the b stream weighs it three times (the softmax normalises the
  two streams jointly); adding one constant to every logit of an entry
  changes nothing;
* RMSNorm (section 2.3.3): unit root-mean-square, scale invariance, the
  closed form for a constant vector;
* RoPE (section 2.3.3, last 64 channels): identity at position 0, the first
  c - 64 channels untouched, pair norms kept, angles adding up, the
  frequency of the first and last pair written out.
"""
import numpy as np
import pytest

from oracle import compress as oc

RNG = np.random.default_rng(7)


def streams(n, c):
    return [RNG.standard_normal((n, c)) for _ in range(4)]


@pytest.mark.parametrize("m", [1, 2, 4])
def test_equal_logits_give_the_mean(m):
    n, c = 6 * m, 16
    ca, _, cb, _ = streams(n, c)
    z = np.zeros((n, c))
    b = np.zeros((m, c))
    e = oc.compress_overlap(ca, z, cb, z, b, b, m)
    assert e.shape == (6, c)
    assert np.allclose(e[0], ca[:m].mean(axis=0), rtol=0, atol=1e-14)
    for i in range(1, 6):
        ref = (ca[m * i:m * (i + 1)].sum(axis=0) + cb[m * (i - 1):m * i].sum(axis=0)) / (2 * m)
        assert np.allclose(e[i], ref, rtol=0, atol=1e-14)
    h = oc.compress_block(ca, z, b, m)
    for i in range(6):
        assert np.allclose(h[i], ca[m * i:m * (i + 1)].mean(axis=0), rtol=0, atol=1e-14)


def test_dominant_logit_selects_its_row():
    m, n, c = 4, 16, 8
    ca, za, cb, zb = streams(n, c)
    za[:] = 0
    zb[:] = 0
    b = np.zeros((m, c))
    # entry 2, channel 3: token 9 of the a stream (block 2 = tokens 8..11)
    za[9, 3] = 1e4
    # entry 2, channel 5: token 6 of the b stream (block 1 = tokens 4..7)
    zb[6, 5] = 1e4
    e = oc.compress_overlap(ca, za, cb, zb, b, b, m)
    assert e[2, 3] == pytest.approx(ca[9, 3], abs=1e-12)
    assert e[2, 5] == pytest.approx(cb[6, 5], abs=1e-12)
    # token 6's b logit belongs to entry 2 only; entry 1 uses block 0 for b
    assert not np.isclose(e[1, 5], cb[6, 5])


def test_constant_values_survive_any_logits():
    m, n, c = 4, 20, 32
    _, za, _, zb = streams(n, c)
    ba, bb = RNG.standard_normal((m, c)), RNG.standard_normal((m, c))
    v = np.full((n, c), 2.5)
    assert np.allclose(oc.compress_overlap(v, za * 3, v, zb * 3, ba, bb, m), 2.5, rtol=0, atol=1e-13)
    assert np.allclose(oc.compress_block(v, za * 3, ba, m), 2.5, rtol=0, atol=1e-13)


def test_joint_normalisation_of_both_streams():
    m, n, c = 2, 8, 4
    ca, _, cb, _ = streams(n, c)
    z = np.zeros((n, c))
    ba = np.zeros((m, c))
    bb = np.full((m, c), np.log(3.0))
    e = oc.compress_overlap(ca, z, cb, z, ba, bb, m)
    for i in range(1, n // m):
        ref = (ca[m * i:m * (i + 1)].sum(axis=0) + 3 * cb[m * (i - 1):m * i].sum(axis=0)) / (m + 3 * m)
        assert np.allclose(e[i], ref, rtol=0, atol=1e-13)


def test_logit_shift_invariance():
    m, n, c = 4, 16, 8
    ca, za, cb, zb = streams(n, c)
    ba, bb = RNG.standard_normal((m, c)), RNG.standard_normal((m, c))
    e0 = oc.compress_overlap(ca, za, cb, zb, ba, bb, m)
    e1 = oc.compress_overlap(ca, za + 7.0, cb, zb + 7.0, ba, bb, m)
    assert np.allclose(e0, e1, rtol=1e-12, atol=1e-13)
    # shifting only the a stream is not a no-op (the two streams share one softmax)
    e2 = oc.compress_overlap(ca, za + 7.0, cb, zb, ba, bb, m)
    assert not np.allclose(e0[1:], e2[1:])
    assert np.allclose(e0[0], e2[0], rtol=1e-12, atol=1e-13)   # entry 0 has no b part


def test_rms_norm():
    x = RNG.standard_normal((5, 512)) * 3
    y = oc.rms_norm(x, np.ones(512), 0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13)
    assert np.allclose(oc.rms_norm(x * 1e-3, np.ones(512), 0.0), y, rtol=1e-12)
    w = RNG.standard_normal(512)
    assert np.allclose(oc.rms_norm(x, w, 0.0), y * w, rtol=1e-12)
    a, eps = 0.5, 1e-2
    yc = oc.rms_norm(np.full((1, 512), a), np.ones(512), eps)
    assert np.allclose(yc, a / np.sqrt(a * a + eps), rtol=1e-14)


def test_rope_tail():
    c = 512
    x = RNG.standard_normal((3, c))
    assert np.array_equal(oc.rope_tail(x, [0, 0, 0]), x)
    pos = np.array([1, 17, 1000003])
    y = oc.rope_tail(x, pos)
    assert np.array_equal(y[:, :c - 64], x[:, :c - 64])
    n_x = x[:, c - 64::2] ** 2 + x[:, c - 63::2] ** 2
    n_y = y[:, c - 64::2] ** 2 + y[:, c - 63::2] ** 2
    assert np.allclose(n_x, n_y, rtol=1e-12)
    assert np.allclose(oc.rope_tail(oc.rope_tail(x, pos), 2 * pos), oc.rope_tail(x, 3 * pos), rtol=1e-9, atol=1e-9)
    # the frequencies: pair 0 turns by 1 rad per position, pair 31 by 10000^(-62/64)
    e = np.zeros((1, c))
    e[0, c - 64] = 1.0
    e[0, c - 2] = 1.0
    r = oc.rope_tail(e, [3])
    assert r[0, c - 64] == pytest.approx(np.cos(3.0), abs=1e-15)
    assert r[0, c - 63] == pytest.approx(np.sin(3.0), abs=1e-15)
    th = 3.0 * 10000.0 ** (-62.0 / 64.0)
    assert r[0, c - 2] == pytest.approx(np.cos(th), abs=1e-15)
    assert r[0, c - 1] == pytest.approx(np.sin(th), abs=1e-15)


def test_write_entries_order():
    """Compression, then the norm, then the rotation at positions pos0 + m i."""
    m, n, c = 4, 12, 128
    ca, za, cb, zb = streams(n, c)
    ba, bb = RNG.standard_normal((m, c)), RNG.standard_normal((m, c))
    w = 1 + 0.1 * RNG.standard_normal(c)
    e = oc.write_entries(m, ca, za, ba, cb, zb, bb, norm_weight=w, eps=1e-6, pos0=40)
    step = oc.compress_overlap(ca, za, cb, zb, ba, bb, m)
    step = oc.rms_norm(step, w, 1e-6)
    step = oc.rope_tail(step, [40, 44, 48])
    assert np.allclose(e, step, rtol=1e-14, atol=1e-14)
    # no norm, no rotation: the compression alone
    assert np.allclose(oc.write_entries(m, ca, za, ba, rope=False), oc.compress_block(ca, za, ba, m))
