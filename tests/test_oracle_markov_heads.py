"""Pins of the gated and recurrent Markov-head oracle against the vanilla
head (itself pinned on its own), closed forms built from one-hot embeddings
and constant gates, and the agreement of its teacher-forced and sampled
forms."""

import math

import numpy as np

from oracle import markov_heads as H
from oracle import tv_loss as T


def _onehot_weights(V, r, c, pi):
    """W1 = c I (V <= r): the embedding of token x is c e_x; W2 = P_pi: rank
    channel j feeds vocabulary entry pi(j)."""
    w1 = np.zeros((V, r)); w1[np.arange(V), np.arange(V)] = c
    w2 = np.zeros((r, V)); w2[np.arange(V), pi] = 1.0
    return w1, w2


def _rand(seed, R, G, V, r, d):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((R, G, V)), rng.standard_normal((R, G, d)), rng.standard_normal((V, r)) * 0.5,
            rng.standard_normal((r, V)) * 0.5, rng.integers(0, V, size=(R, G)))


def test_gated_saturated_gate_is_the_vanilla_head():
    """A gate driven to 1 by the hidden state (sigmoid(60) = 1 in float64)
    leaves W2(W1[x]): the vanilla head's block logits, also soft-capped."""
    R, G, V, r, d = 3, 4, 30, 6, 5
    base, _, w1, w2, prev = _rand(1, R, G, V, r, d)
    hidden = np.ones((R, G, d))
    wg = np.zeros((r, d + r)); wg[:, :d] = 60.0 / d
    for cap in (0.0, 2.5):
        got = H.block_logits(H.GATED, base, hidden, w1, w2, wg, prev, softcap=cap)
        want = T.block_logits(base.reshape(-1, V), w1, w2, prev.ravel(), softcap=cap).reshape(R, G, V)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_gated_zero_gate_weights_halve_the_bias():
    R, G, V, r, d = 2, 3, 25, 4, 7
    base, hidden, w1, w2, prev = _rand(2, R, G, V, r, d)
    got = H.block_logits(H.GATED, base, hidden, w1, w2, np.zeros((r, d + r)), prev) - base
    vanilla = T.block_logits(base.reshape(-1, V), w1, w2, prev.ravel()).reshape(R, G, V) - base
    np.testing.assert_allclose(got, 0.5 * vanilla, rtol=0, atol=1e-12)


def test_gated_gate_reads_the_embedding_after_the_hidden_state():
    """W_g = [0 | beta I]: the gate of channel j is sigmoid(beta * W1[x]_j);
    with W1 = c I and beta c = ln 3 the gate at x is 3/4, so the bias is
    (3/4) c at pi(x) and zero elsewhere.  The random hidden state must not
    matter."""
    V, r, d, c = 5, 8, 6, 2.0
    pi = np.array([3, 0, 4, 1, 2])
    w1, w2 = _onehot_weights(V, r, c, pi)
    wg = np.zeros((r, d + r)); wg[:, d:] = (math.log(3.0) / c) * np.eye(r)
    rng = np.random.default_rng(3)
    base = rng.standard_normal((2, 3, V))
    hidden = rng.standard_normal((2, 3, d)) * 4
    prev = np.array([[0, 4, 4], [2, 1, 3]])
    got = H.block_logits(H.GATED, base, hidden, w1, w2, wg, prev)
    want = base.copy()
    for b in range(2):
        for k in range(3):
            want[b, k, pi[prev[b, k]]] += 0.75 * c
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_rnn_closed_form_recurrence():
    """W_g reads only the constant hidden state: gate 3/4 everywhere.  W_c
    reads only the embedding (b I), W_o only the state (a I).  With W1 = c I
    the state is the geometric sum
        s_k = (1/4) tanh(b c) sum_{i <= k} (3/4)^(k - i) e_{x_{i-1}}
    from s_{-1} = 0, and position k's bias is tanh(a s_{k-1}) mapped by P_pi
    (zero at the block's first position)."""
    V, r, d, c, a, b = 4, 6, 3, 1.5, 0.8, 0.7
    pi = np.array([2, 3, 0, 1])
    w1, w2 = _onehot_weights(V, r, c, pi)
    eta = 0.5
    w = np.zeros((3, r, 2 * r + d))
    w[0, :, 2 * r:] = math.log(3.0) / (d * eta)
    w[1, :, r:2 * r] = b * np.eye(r)
    w[2, :, :r] = a * np.eye(r)
    R, G = 2, 5
    rng = np.random.default_rng(4)
    base = rng.standard_normal((R, G, V))
    hidden = np.full((R, G, d), eta)
    prev = rng.integers(0, V, size=(R, G))
    got = H.block_logits(H.RNN, base, hidden, w1, w2, w, prev)
    for row in range(R):
        for k in range(G):
            s_prev = np.zeros(r)  # s_{k-1}
            for i in range(k):
                s_prev[prev[row, i]] += 0.25 * math.tanh(b * c) * 0.75 ** (k - 1 - i)
            want = base[row, k].copy()
            for j in range(V):
                want[pi[j]] += math.tanh(a * s_prev[j])
            np.testing.assert_allclose(got[row, k], want, rtol=0, atol=1e-12)


def test_rnn_saturated_gate_keeps_zero_state():
    """Gate 1 (sigmoid(60)) keeps s = 0; W_o = [0 | a I | 0] then gives the
    bias tanh(a c) at pi(x) at every position, whatever W_c and h are."""
    V, r, d, c, a = 5, 5, 4, 1.2, 0.9
    pi = np.array([4, 2, 0, 3, 1])
    w1, w2 = _onehot_weights(V, r, c, pi)
    rng = np.random.default_rng(5)
    w = np.zeros((3, r, 2 * r + d))
    w[0, :, 2 * r:] = 60.0 / d
    w[1] = rng.standard_normal((r, 2 * r + d))
    w[2, :, r:2 * r] = a * np.eye(r)
    base = rng.standard_normal((1, 6, V))
    prev = rng.integers(0, V, size=(1, 6))
    got = H.block_logits(H.RNN, base, np.ones((1, 6, d)), w1, w2, w, prev)
    want = base.copy()
    want[0, np.arange(6), pi[prev[0]]] += math.tanh(a * c)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_sampling_agrees_with_teacher_forcing():
    """Greedy sampling equals its own teacher-forced replay, and the block
    logits with previous tokens (first_prev, x_0, .., x_{gamma-2}) equal the
    sampled step logits; temperature sampling too, with the Gumbel values."""
    R, G, V, r, d = 3, 5, 40, 6, 8
    base, hidden, w1, w2, _ = _rand(6, R, G, V, r, d)
    rng = np.random.default_rng(7)
    first = rng.integers(0, V, size=R)
    heads = {H.GATED: rng.standard_normal((r, d + r)) * 0.5, H.RNN: rng.standard_normal((3, r, 2 * r + d)) * 0.5}
    for kind, wh in heads.items():
        for temp in (0.0, 0.7):
            tok, z, l = H.sample_block_tokens(kind, base * 3, hidden, w1, w2, wh, first, temperature=temp, seed=11)
            np.testing.assert_array_equal(tok, np.argmax(z, axis=-1))
            tok2, _, l2 = H.sample_block_tokens(kind, base * 3, hidden, w1, w2, wh, first, temperature=temp,
                                                seed=11, teacher=tok)
            np.testing.assert_array_equal(tok2, tok)
            np.testing.assert_array_equal(l2, l)
            prev = np.concatenate([first[:, None], tok[:, :-1]], axis=1)
            np.testing.assert_allclose(H.block_logits(kind, base * 3, hidden, w1, w2, wh, prev), l,
                                       rtol=0, atol=1e-12)
