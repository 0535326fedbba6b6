"""The seeded input generator: determinism, ranges and the distributions the
configurations ask for (N(0,1) via Irwin-Hall, U(0,1), ~5% boosted keys,
log-uniform lengths, permutations, given pools)."""
import numpy as np

import synth


def test_normal_stats_and_bounds():
    x = synth.normal(0, synth.T_LATENT, np.arange(1 << 18, dtype=np.uint64))
    assert abs(float(x.mean())) < 0.01 and abs(float(x.var()) - 1) < 0.01
    assert np.all(np.abs(x) <= 6)
    # exact in fp32: integer multiples of 2^-16
    assert np.array_equal(np.round(x.astype(np.float64) * 65536) / 65536, x.astype(np.float64))


def test_deterministic_and_streams_differ():
    a = synth.normal_bf16(3, synth.T_Q, (4, 512))
    b = synth.normal_bf16(3, synth.T_Q, (4, 512))
    c = synth.normal_bf16(3, synth.T_QIDX, (4, 512))
    d = synth.normal_bf16(4, synth.T_Q, (4, 512))
    assert np.array_equal(a, b) and not np.array_equal(a, c) and not np.array_equal(a, d)
    rows = synth.normal_bf16_rows(3, synth.T_Q, [2, 0], 512)
    assert np.array_equal(rows, a[[2, 0]])


def test_bf16_rounding():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    assert got.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0 + 2 ** -7]


def test_uniform_and_boost():
    u = synth.uniform(1, synth.T_W, np.arange(1 << 16, dtype=np.uint64))
    assert u.min() >= 0 and u.max() < 1 and abs(float(u.mean()) - 0.5) < 0.01
    m = synth.boost_mask(2, np.arange(1 << 18))
    assert abs(float(m.mean()) - 0.05) < 0.003


def test_pool_lengths_pages():
    p = synth.given_pool(2, 5, 131072, 2048)
    assert len(p) == 2048 and np.all(np.diff(p) > 0) and p.min() >= 0 and p.max() < 131072
    L = synth.ragged_lengths(4, 256)
    assert L.min() >= 4096 and L.max() < 4096 * 256
    perm = synth.page_permutation(4, 1000)
    assert np.array_equal(np.sort(perm), np.arange(1000))
