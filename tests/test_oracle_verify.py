"""Pins of the oracle's speculative verification (Lynx paper Section 4.3;
the notes' Eq. (10) acceptance min(1, p/q) and Eq. (11) correction
max(0, p - q)) against what the mathematics fixes:

* identical draft and target distributions accept every draft;
* a draft the target gives no mass is rejected and never re-emitted;
* the acceptance frequency over a grid of uniforms is min(1, p/q);
* the lossless property: the emitted token is distributed exactly as the
  target distribution, at the first position and for the bonus token after
  a fully accepted draft (Monte Carlo, 5-sigma bounds) -- a swapped ratio or
  a residual max(0, q - p) fails it;
* inverse-CDF sampling picks the closed-form index on a uniform and a
  one-hot target.
"""
import numpy as np

import oracle


def softmax(l):
    e = np.exp(l - l.max())
    return e / e.sum()


def test_identical_distributions_accept_everything():
    rng = np.random.default_rng(1)
    for T in (1, 3, 8):
        t = rng.normal(0, 2, size=(T + 1, 50)).astype(np.float32)
        d = t[:T].copy()
        s = rng.integers(0, 50, size=T)
        for _ in range(20):
            n, tok = oracle.spec_verify(d, t, s, rng.random(T), rng.random())
            assert n == T and 0 <= tok < 50


def test_draft_without_target_mass_is_rejected():
    rng = np.random.default_rng(2)
    d = rng.normal(0, 1, size=(2, 20)).astype(np.float32)
    t = rng.normal(0, 1, size=(3, 20)).astype(np.float32)
    t[0, 7] = -1e30  # p(7) = 0 at position 0
    for _ in range(50):
        n, tok = oracle.spec_verify(d, t, np.array([7, 3]), rng.random(2), rng.random())
        assert n == 0 and tok != 7


def test_acceptance_frequency_is_min_one_ratio():
    rng = np.random.default_rng(3)
    d = rng.normal(0, 1, size=(1, 12)).astype(np.float32)
    t = rng.normal(0, 1, size=(2, 12)).astype(np.float32)
    p, q = softmax(t[0].astype(np.float64)), softmax(d[0].astype(np.float64))
    for s in range(12):
        grid = (np.arange(1000) + 0.5) / 1000
        acc = np.mean([oracle.spec_verify(d, t, np.array([s]), np.array([u]), 0.5)[0]
                       for u in grid])
        assert abs(acc - min(1.0, p[s] / q[s])) <= 1e-3 + 1e-9


def test_emitted_tokens_follow_the_target_distribution():
    """Draw s ~ q and uniforms; the first emitted token (s if accepted, else
    the correction) must follow p_0, and after an accepted draft the bonus
    token must follow p_1."""
    rng = np.random.default_rng(4)
    V, N = 6, 120000
    d = np.array([[1.5, 0.2, -0.3, 0.9, -1.2, 0.0]], np.float32)
    t = np.array([[0.1, 1.1, -0.8, 0.4, 0.3, -0.5],
                  [-0.7, 0.2, 1.3, 0.0, 0.6, -1.1]], np.float32)
    q = softmax(d[0].astype(np.float64))
    p0, p1 = softmax(t[0].astype(np.float64)), softmax(t[1].astype(np.float64))
    s_draw = rng.choice(V, size=N, p=q)
    first = np.zeros(V)
    bonus = np.zeros(V)
    for i in range(N):
        n, tok = oracle.spec_verify(d, t, s_draw[i:i + 1], rng.random(1), rng.random())
        if n == 1:
            first[s_draw[i]] += 1
            bonus[tok] += 1
        else:
            first[tok] += 1
    f = first / N
    assert np.all(np.abs(f - p0) <= 5 * np.sqrt(p0 * (1 - p0) / N)), (f, p0)
    nb = bonus.sum()
    b = bonus / nb
    assert np.all(np.abs(b - p1) <= 5 * np.sqrt(p1 * (1 - p1) / nb)), (b, p1)
    # accepted share = sum_x min(p0, q)
    assert abs(nb / N - np.minimum(p0, q).sum()) <= 5 * np.sqrt(0.25 / N)


def test_inverse_cdf_closed_forms():
    V = 40
    d = np.zeros((1, V), np.float32)
    uniform = np.zeros((2, V), np.float32)
    for i in range(V):
        n, tok = oracle.spec_verify(d, uniform, np.array([5]), np.array([0.0]), (i + 0.5) / V)
        assert (n, tok) == (1, i)
    onehot = np.full((2, V), -1e30, np.float32)
    onehot[:, 17] = 0.0
    d1 = onehot[:1].copy()
    for u in (0.0, 0.3, 0.999999):
        assert oracle.spec_verify(d1, onehot, np.array([17]), np.array([0.5]), u) == (1, 17)
