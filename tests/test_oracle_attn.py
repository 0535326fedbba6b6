"""Pins the oracle's attention (fp64 joint softmax over selected + SWA entries).

Definitions: shared-KV MQA, each selected entry used as key and value
('DeepSeek-V4' paper page, section 2.3.1); the sliding-window entries are used
together with the selected entries in the same core attention and a per-head
sink logit adds exp(z'_h) to the denominator (section 2.3.3); latent
attention with the absorbed query equals attention with up-projected keys and
values (MLA article, section 4, matrix absorption).

Pins: scipy.special.softmax / logsumexp on tiny inputs (top-k >= context, so
the sparse attention is the dense one); closed forms (one entry gives the
entry; q = 0 gives the mean; two entries give sigmoid weights via
scipy.special.expit; q = 0 with a sink gives sum / (n + e^sink)); the
sink -> -inf limit; the LSE merge of a split set equals the joint softmax;
permutation invariance; the absorption identity with random up-projections.
"""
import numpy as np
import pytest
from scipy.special import expit, logsumexp, softmax

RNG = np.random.default_rng(41)
SIG = 512 ** -0.5


def _data(H=4, n=6, m=3, C=512):
    q = RNG.standard_normal((H, C)).astype(np.float32)
    K = RNG.standard_normal((n, C)).astype(np.float32)
    W = RNG.standard_normal((m, C)).astype(np.float32)
    return q, K, W


def test_dense_softmax_scipy(orc):
    q, K, W = _data()
    o, lse = orc.attention(q, K, W, sigma=SIG)
    E = np.concatenate([K, W]).astype(np.float64)
    z = SIG * (q.astype(np.float64) @ E.T)
    ref = softmax(z, axis=1) @ E
    assert np.allclose(o, ref, rtol=1e-6, atol=1e-6)
    assert np.allclose(lse, logsumexp(z, axis=1), rtol=1e-6)


def test_single_entry_and_zero_query(orc):
    q, K, W = _data(n=1, m=0)
    o, lse = orc.attention(q, K, None, sigma=SIG)
    assert np.array_equal(o, np.repeat(K, 4, axis=0))
    _, K5, _ = _data(n=5)
    o, lse = orc.attention(np.zeros((2, 512), np.float32), K5, None, sigma=SIG)
    assert np.allclose(o, K5.astype(np.float64).mean(0)[None], atol=1e-6)
    assert np.allclose(lse, np.log(5))


def test_two_entries_sigmoid(orc):
    q, K, _ = _data(H=3, n=2)
    o, _ = orc.attention(q, K, None, sigma=SIG)
    z = SIG * (q.astype(np.float64) @ K.astype(np.float64).T)
    a = expit(z[:, 0] - z[:, 1])[:, None]
    ref = a * K[0].astype(np.float64) + (1 - a) * K[1].astype(np.float64)
    assert np.allclose(o, ref, rtol=1e-6, atol=1e-7)


def test_sink(orc):
    q, K, W = _data()
    o0, lse0 = orc.attention(q, K, W, sigma=SIG)
    o1, lse1 = orc.attention(q, K, W, sink=np.full(4, -1e30, np.float32), sigma=SIG)
    assert np.array_equal(o0, o1) and np.array_equal(lse0, lse1)
    s = np.array([0.0, 1.0, -2.0, 3.0], np.float32)
    o, lse = orc.attention(np.zeros((4, 512), np.float32), K, W, sink=s, sigma=SIG)
    tot = np.concatenate([K, W]).astype(np.float64).sum(0)
    ref = tot[None] / (9 + np.exp(s.astype(np.float64)))[:, None]
    assert np.allclose(o, ref, rtol=1e-6, atol=1e-7)
    assert np.allclose(lse, np.log(9 + np.exp(s.astype(np.float64))), rtol=1e-6)
    # sink only: output 0, lse = sink
    o, lse = orc.attention(np.zeros((4, 512), np.float32), None, None, sink=s, sigma=SIG)
    assert not o.any() and np.allclose(lse, s)


def test_empty_set(orc):
    o, lse = orc.attention(np.ones((2, 512), np.float32), None, None, sigma=SIG)
    assert not o.any() and np.all(np.isneginf(lse))


def test_lse_merge_equals_joint(orc):
    q, K, W = _data(n=40, m=20)
    o, lse = orc.attention(q, K, W, sigma=SIG)
    oa, la = orc.attention(q, K[:25], None, sigma=SIG)
    ob, lb = orc.attention(q, K[25:], W, sigma=SIG)
    la, lb = la.astype(np.float64), lb.astype(np.float64)
    M = np.maximum(la, lb)
    wa, wb = np.exp(la - M), np.exp(lb - M)
    merged = (wa[:, None] * oa + wb[:, None] * ob) / (wa + wb)[:, None]
    assert np.allclose(merged, o, rtol=1e-5, atol=1e-6)
    assert np.allclose(M + np.log(wa + wb), lse, rtol=1e-6)


def test_permutation_invariance(orc):
    q, K, W = _data(n=30, m=10)
    o, lse = orc.attention(q, K, W, sigma=SIG)
    p = RNG.permutation(30)
    o2, lse2 = orc.attention(q, K[p], W[::-1], sigma=SIG)
    assert np.allclose(o, o2, rtol=1e-6, atol=1e-7) and np.allclose(lse, lse2, rtol=1e-7)


def test_absorption_identity(orc):
    """Naive MLA: k_{j,i} = W_UK[i] c_j, v_{j,i} = W_UV[i] c_j, attention with
    q_i.  Absorbed: attention over the latents c_j with q_abs = W_UK[i]^T q_i,
    then W_UV[i] applied to the result.  They agree to rounding."""
    H, dh, C, n = 4, 32, 512, 12
    c = RNG.standard_normal((n, C)).astype(np.float32)
    Wuk = RNG.standard_normal((H, dh, C)) / np.sqrt(C)
    Wuv = RNG.standard_normal((H, dh, C)) / np.sqrt(C)
    qh = RNG.standard_normal((H, dh))
    sigma = dh ** -0.5
    naive = np.zeros((H, dh))
    for i in range(H):
        k = c.astype(np.float64) @ Wuk[i].T
        v = c.astype(np.float64) @ Wuv[i].T
        naive[i] = softmax(sigma * (k @ qh[i])) @ v
    q_abs = np.stack([Wuk[i].T @ qh[i] for i in range(H)])
    # the oracle takes fp32 queries: feed q_abs rounded, and compare with the
    # naive path evaluated on the same rounded absorbed query
    q32 = q_abs.astype(np.float32)
    lat, _ = orc.attention(q32, c, None, sigma=sigma)
    absorbed = np.stack([Wuv[i] @ lat[i].astype(np.float64) for i in range(H)])
    assert np.allclose(absorbed, naive, rtol=1e-4, atol=1e-5)
    # in exact fp64 arithmetic (numpy) the identity holds to ~1e-15
    for i in range(H):
        s_naive = (c.astype(np.float64) @ Wuk[i].T) @ qh[i]
        s_abs = c.astype(np.float64) @ q_abs[i]
        assert np.max(np.abs(s_naive - s_abs)) < 1e-12
