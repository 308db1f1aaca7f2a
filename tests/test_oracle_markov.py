"""Pins for the Markov-head oracle (CPU only)."""

import math

import numpy as np

import workloads as W
from oracle import markov as OM
from oracle import philox


def test_zero_w2_is_the_rank0_degenerate_case():
    """W2 = 0 (the DFlash degenerate configuration, page 1 §3.13): step
    logits equal the base logits bit for bit and every token is the row-wise
    argmax of its own base slice, with no dependence on the previous token."""
    c = W.markov_case(21, R=5, gamma=6, V=97, r=8, wdtype="f32", base_std=2.0,
                      w1_std=1.0, w2_std=1.0)
    w2 = np.zeros_like(c.w2)
    tok, z, l = OM.sample_block_tokens(c.base, c.w1, w2, c.first_prev)
    assert np.array_equal(l, c.base.astype(np.float64))
    assert np.array_equal(tok, np.argmax(c.base, axis=2))


def test_permutation_chain_closed_form():
    """W1 = c*I (V <= r, zero padded) and W2 = c*P_pi give bias[v] =
    c^2 [v == pi(prev)].  With c^2 far above the base range the chain follows
    the permutation: token_i = pi^(i+1)(first_prev)."""
    rng = np.random.default_rng(3)
    V, r, R, G, c = 11, 16, 6, 9, 30.0
    pi = rng.permutation(V)
    w1 = np.zeros((V, r))
    w1[np.arange(V), np.arange(V)] = c
    w2 = np.zeros((r, V))
    w2[np.arange(V), pi] = c
    base = rng.standard_normal((R, G, V))
    first = rng.integers(0, V, size=R)
    tok, _, _ = OM.sample_block_tokens(base, w1, w2, first)
    expect = np.zeros((R, G), dtype=np.int64)
    cur = first.copy()
    for i in range(G):
        cur = pi[cur]
        expect[:, i] = cur
    assert np.array_equal(tok, expect)


def test_rank1_alternating_chain():
    """r = 1: bias[v] = alpha[prev] * beta[v].  With zero base, alpha = +1 on
    even tokens and -1 on odd ones, and beta's maximum at an odd index v1 and
    minimum at an even index v0, the greedy chain alternates v1, v0, v1, ...
    from an even first token."""
    V = 10
    beta = np.array([0.0, 0.1, -0.9, 0.2, 0.3, 0.5, -0.2, 0.9, 0.05, -0.1])
    v1, v0 = int(np.argmax(beta)), int(np.argmin(beta))
    assert v1 % 2 == 1 and v0 % 2 == 0
    alpha = np.where(np.arange(V) % 2 == 0, 1.0, -1.0)[:, None]
    tok, _, _ = OM.sample_block_tokens(np.zeros((1, 7, V)), alpha, beta[None, :], [4])
    assert tok[0].tolist() == [v1, v0, v1, v0, v1, v0, v1]


def test_step_logits_elementwise():
    """The bias is sum_j W1[prev, j] * W2[j, v], checked element by element
    with Python floats on a tiny case (a transposed or mis-indexed operand
    fails it)."""
    rng = np.random.default_rng(4)
    V, r = 7, 3
    w1 = rng.standard_normal((V, r))
    w2 = rng.standard_normal((r, V))
    base = rng.standard_normal((2, V))
    prev = [5, 2]
    l = OM.step_logits(base, w1, w2, prev)
    for i in range(2):
        for v in range(V):
            s = base[i, v]
            for j in range(r):
                s += float(w1[prev[i], j]) * float(w2[j, v])
            assert abs(l[i, v] - s) < 1e-14


def test_ties_take_the_lowest_index():
    base = np.zeros((1, 2, 6))
    base[0, 0, [2, 4]] = 1.0
    base[0, 1, [0, 5]] = 3.0
    tok, _, _ = OM.sample_block_tokens(base, np.zeros((6, 2)), np.zeros((2, 6)), [0])
    assert tok[0].tolist() == [2, 0]


def test_teacher_forcing_with_own_tokens_is_free_running():
    c = W.markov_case(22, R=4, gamma=5, V=64, r=8, wdtype="f32", base_std=1.0,
                      w1_std=1.0, w2_std=1.0, temperature=0.7, philox_seed=99)
    t1, z1, _ = OM.sample_block_tokens(c.base, c.w1, c.w2, c.first_prev, 0.7, 99)
    t2, z2, _ = OM.sample_block_tokens(c.base, c.w1, c.w2, c.first_prev, 0.7, 99, teacher=t1)
    assert np.array_equal(t1, t2) and np.array_equal(z1, z2)


def test_gumbel_max_matches_softmax_frequencies():
    """Gumbel-max sampling draws token v with probability softmax(l/T)_v:
    chi-square test over 20000 independent seeds on V = 8 (one step)."""
    V, T, n = 8, 0.8, 20000
    l = np.array([0.3, -1.0, 1.2, 0.0, 0.5, -0.4, 2.0, 0.9])
    # the sampler's own noise for step 0 of row 0 under each seed
    g = np.stack([philox.gumbel(s, 0, 0, V) for s in range(n)])
    tok = np.argmax(l / T + g, axis=1)
    p = np.exp(l / T - np.max(l / T))
    p /= p.sum()
    counts = np.bincount(tok, minlength=V)
    chi2 = ((counts - n * p) ** 2 / (n * p)).sum()
    assert chi2 < 7 + 5 * math.sqrt(14)
    # and the sampler itself uses exactly that noise
    tk, z, _ = OM.sample_block_tokens(np.tile(l, (1, 1, 1)), np.zeros((V, 1)), np.zeros((1, V)),
                                      [0], temperature=T, seed=12345)
    assert tk[0, 0] == np.argmax(l / T + philox.gumbel(12345, 0, 0, V))


def test_small_temperature_is_greedy():
    c = W.markov_case(23, R=6, gamma=4, V=300, r=8, wdtype="f32", base_std=3.0,
                      w1_std=1.0, w2_std=0.5)
    tg, _, _ = OM.sample_block_tokens(c.base, c.w1, c.w2, c.first_prev, 0.0)
    ts, _, _ = OM.sample_block_tokens(c.base, c.w1, c.w2, c.first_prev, 1e-4, 5)
    assert np.array_equal(tg, ts)


def test_acceptable_tokens_margin():
    z = np.array([1.0, 3.0, 2.9995, 3.0 - 2e-3])
    assert OM.acceptable_tokens(z, 1e-3).tolist() == [1, 2]
    assert OM.acceptable_tokens(z, 1e-4).tolist() == [1]
