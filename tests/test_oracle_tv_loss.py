"""Pins of the teacher-forced block-logit, L1-loss and tau_greedy oracle
against closed forms, finite differences and hand-worked examples."""

import math

import numpy as np

from oracle import tv_loss as T


def _rng(seed):
    return np.random.default_rng(seed)


def test_block_logits_zero_w2_is_base():
    rng = _rng(1)
    base = rng.standard_normal((5, 40))
    w1 = rng.standard_normal((40, 8))
    np.testing.assert_array_equal(T.block_logits(base, w1, np.zeros((8, 40)), [3, 0, 39, 7, 7]), base)


def test_block_logits_one_hot_spike():
    """W1 = c I (V <= r) and W2 = c P_pi: the bias of previous token x is c^2
    at pi(x) and zero elsewhere."""
    V, r, c = 6, 8, 3.0
    pi = np.array([2, 0, 5, 1, 3, 4])
    w1 = np.zeros((V, r)); w1[np.arange(V), np.arange(V)] = c
    w2 = np.zeros((r, V)); w2[np.arange(V), pi] = c
    base = _rng(2).standard_normal((4, V))
    prev = np.array([1, 4, 4, 0])
    got = T.block_logits(base, w1, w2, prev)
    want = base.copy()
    want[np.arange(4), pi[prev]] += c * c
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_softcap_limits():
    base = np.array([[0.0, 1e-3, -2.0, 500.0, -1e4]])
    w1, w2 = np.zeros((1, 1)), np.zeros((1, 5))
    got = T.block_logits(base, w1, w2, [0], softcap=30.0)
    np.testing.assert_allclose(got[0, :2], [0.0, 1e-3], rtol=1e-6)          # identity near 0
    assert abs(got[0, 2] - 30.0 * math.tanh(-2.0 / 30.0)) < 1e-12
    assert 29.99 < got[0, 3] <= 30.0 and got[0, 4] == -30.0                  # saturates at +-c
    np.testing.assert_array_equal(T.block_logits(base, w1, w2, [0], softcap=0.0), base)


def test_l1_two_class_closed_form():
    rng = _rng(3)
    d, t = rng.standard_normal((7, 2)) * 3, rng.standard_normal((7, 2)) * 3
    sig = lambda z: 1.0 / (1.0 + np.exp(-z))
    want = 2.0 * np.abs(sig(d[:, 1] - d[:, 0]) - sig(t[:, 1] - t[:, 0]))
    np.testing.assert_allclose(T.l1_distance(d, t), want, rtol=1e-12, atol=1e-15)


def test_l1_identical_and_disjoint():
    rng = _rng(4)
    d = rng.standard_normal((3, 50))
    np.testing.assert_allclose(T.l1_distance(d, d + 7.5), 0.0, atol=1e-14)  # shift invariant
    a = np.zeros((1, 50)); a[0, 3] = 60.0
    b = np.zeros((1, 50)); b[0, 9] = 60.0
    assert abs(T.l1_distance(a, b)[0] - 2.0) < 1e-20 + 1e-12


def test_loss_two_position_hand_example():
    """gamma = 2, decay = 4: weights 1 and e^-1/4; one masked-out block."""
    rng = _rng(5)
    d, t = rng.standard_normal((1, 2, 2, 9)), rng.standard_normal((1, 2, 2, 9))
    m = np.array([[[1, 1], [0, 0]]])
    l1 = T.l1_distance(d, t)
    w1 = math.exp(-0.25)
    want = (l1[0, 0, 0] + w1 * l1[0, 0, 1]) / (1.0 + w1)
    assert abs(T.l1_loss(d, t, m, decay=4.0) - want) < 1e-14
    assert T.l1_loss(d, t, np.zeros_like(m)) == 0.0


def test_grad_matches_central_differences():
    rng = _rng(6)
    d, t = rng.standard_normal((2, 1, 3, 11)), rng.standard_normal((2, 1, 3, 11))
    m = np.array([[[1, 1, 0]], [[1, 0, 0]]])
    g = T.l1_loss_grad(d, t, m)
    h = 1e-6
    num = np.zeros_like(d)
    for idx in np.ndindex(d.shape):
        dp, dm = d.copy(), d.copy()
        dp[idx] += h
        dm[idx] -= h
        num[idx] = (T.l1_loss(dp, t, m) - T.l1_loss(dm, t, m)) / (2 * h)
    np.testing.assert_allclose(g, num, rtol=0, atol=1e-8)
    # the softmax gradient sums to zero over the vocabulary of every row
    np.testing.assert_allclose(g.sum(axis=-1), 0.0, atol=1e-15)
    assert np.all(g[0, 0, 2] == 0) and np.all(g[1, 0, 1:] == 0)  # masked rows get no gradient


def test_tau_greedy():
    rng = _rng(7)
    d = rng.standard_normal((2, 3, 4, 20))
    t = d + 0.01 * rng.standard_normal(d.shape)
    t[0, 1, 2] = -d[0, 1, 2]                   # argmax moves: rejection at k = 2
    m = np.ones((2, 3, 4), dtype=np.uint8)
    m[1, 2, 1:] = 0                             # eval mask cuts block (1, 2) after k = 0
    tau = T.tau_greedy(d, t, m)
    want = np.full((2, 3), 5.0)
    want[0, 1] = 3.0
    want[1, 2] = 2.0
    np.testing.assert_array_equal(tau, want)
    assert np.all(T.tau_greedy(d, d, np.zeros_like(m)) == 1.0)
