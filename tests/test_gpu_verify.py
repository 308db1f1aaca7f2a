"""Lossless verify step on the GPU vs the oracle.

Bars: the number of kept drafts is exact except where the decisive
acceptance test is a float32 near-tie (|u - p/q| within 1e-4 relative);
the extra token equals the oracle's draw wherever the oracle's top-2 margin
of the Gumbel-max values exceeds 1e-3 and otherwise lies within 1e-3 of the
maximum; greedy verification is exact."""

import numpy as np
import pytest
import torch

from gpu_util import DEV, dev
from oracle import philox
from oracle import verify as VF

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsp():
    import semi_autoregressive_block_amd as m
    return m


def _inputs(seed, R, K, V, spread=0.7):
    rng = np.random.default_rng(seed)
    t = (rng.standard_normal((R, K + 1, V)) * 2).astype(np.float32)
    d = (t[:, :K] + rng.standard_normal((R, K, V)) * spread).astype(np.float32)
    q = VF.softmax(d)
    x = np.array([[rng.choice(V, p=q[i, k]) for k in range(K)] for i in range(R)], dtype=np.int32).reshape(R, K)
    return d, t, x


def _oracle_z(d, t, k, K, V, T, seed, row):
    g = philox.gumbel(seed, row, k, V, stream=1)
    if k == K:
        return t[k].astype(np.float64) / T + g
    p, q = VF.softmax(t[k] / T), VF.softmax(d[k] / T)
    with np.errstate(divide="ignore"):
        return np.log(np.maximum(p - q, 0.0)) + g


def _check(dsp, d, t, x, T, seed, rows=None):
    R, K = x.shape
    V = t.shape[-1]
    n, tok = dsp.verify(dev(d), dev(t), dev(x), temperature=T, seed=seed)
    n, tok = n.cpu().numpy(), tok.cpu().numpy()
    rows = range(R) if rows is None else rows
    same = 0
    for i in rows:
        n_or, tok_or, ratios, us = VF.verify_row(d[i], t[i], x[i], T, seed, i)
        if n[i] != n_or:
            k = min(n[i], n_or)
            assert abs(us[k] - ratios[k]) <= 1e-4 * max(1.0, ratios[k]), (i, n[i], n_or)
            continue
        same += 1
        z = _oracle_z(d[i], t[i], n_or, K, V, T, seed, i)
        assert z[tok[i]] >= z.max() - 1e-3, (i, tok[i], tok_or)
        top2 = np.sort(z)[-2:]
        if top2[1] - top2[0] > 1e-3:
            assert tok[i] == tok_or, (i, tok[i], tok_or)
    assert same >= 0.9 * len(rows)
    return n


@pytest.mark.parametrize("R,K,V,T", [(64, 4, 1000, 1.0), (48, 8, 4099, 0.7), (5, 1, 7, 1.3)])
def test_random_blocks(dsp, R, K, V, T):
    d, t, x = _inputs(R + K + V, R, K, V)
    n = _check(dsp, d, t, x, T, seed=R * 7 + 1)
    if R >= 48:
        assert 0 < n.mean() < K  # both outcomes occur


def test_bonus_only_block(dsp):
    """K = 0: nothing to verify, one token drawn from the target."""
    d, t, x = _inputs(3, 16, 0, 300)
    n = _check(dsp, d, t, x, 1.0, seed=9)
    assert np.all(n == 0)


def test_greedy(dsp):
    R, K, V = 6, 5, 500
    rng = np.random.default_rng(4)
    t = rng.standard_normal((R, K + 1, V)).astype(np.float32)
    d = rng.standard_normal((R, K, V)).astype(np.float32)
    x = np.argmax(t[:, :K], axis=-1).astype(np.int32)
    for i in range(R):
        if i < K:
            x[i, i] = (x[i, i] + 1) % V  # row i rejects at position i; the last row keeps all
    n, tok = dsp.verify(dev(d), dev(t), dev(x), temperature=0.0)
    n_or, tok_or = VF.verify(d, t, x, temperature=0.0)
    np.testing.assert_array_equal(n.cpu().numpy(), n_or)
    np.testing.assert_array_equal(tok.cpu().numpy(), tok_or)
    np.testing.assert_array_equal(n_or, [0, 1, 2, 3, 4, 5])


def test_serving_shape_all_rows(dsp):
    """128 requests, K = 16, V = 151936: the kept count of every row, the
    extra token of 32 rows (the first, the last and every fourth)."""
    R, K, V = 128, 16, 151936
    g = torch.Generator(device=DEV).manual_seed(77)
    t = torch.randn((R, K + 1, V), generator=g, device=DEV) * 2
    d = t[:, :K] + torch.randn((R, K, V), generator=g, device=DEV) * 0.3
    x = torch.distributions.Categorical(logits=d).sample().to(torch.int32)
    n, tok = dsp.verify(d, t, x, temperature=1.0, seed=31)
    n, tok = n.cpu().numpy(), tok.cpu().numpy()
    dn, tn, xn = d.cpu().numpy(), t.cpu().numpy(), x.cpu().numpy()
    token_rows = set(range(0, R, 4)) | {R - 1}
    same = checked = 0
    for i in range(R):
        n_or, tok_or, ratios, us = VF.verify_row(dn[i], tn[i], xn[i], 1.0, 31, i)
        if int(n[i]) != n_or:
            k = min(int(n[i]), n_or)
            assert abs(us[k] - ratios[k]) <= 1e-4 * max(1.0, ratios[k]), (i, int(n[i]), n_or)
            continue
        same += 1
        if i in token_rows:
            checked += 1
            z = _oracle_z(dn[i], tn[i], n_or, K, V, 1.0, 31, i)
            assert z[int(tok[i])] >= z.max() - 1e-3, (i, int(tok[i]), tok_or)
            top2 = np.sort(z)[-2:]
            if top2[1] - top2[0] > 1e-3:
                assert int(tok[i]) == tok_or, (i, int(tok[i]), tok_or)
    assert same >= R - 2 and checked >= 30
    assert 0 < n.mean() < K


def _masked_inputs(seed, R, K, V, strip_threads=(0, 5), frac=0.3):
    """Target and draft logits with -inf entries: index 0 of every row, the
    whole strip of vocabulary entries that thread c of a 256-thread
    workgroup reads with 16-byte loads (4 (c + 256 j) + e), and a random
    fraction; the drafted tokens are drawn from the draft's own softmax, so
    they never sit on a -inf draft logit but do sit on -inf target logits."""
    rng = np.random.default_rng(seed)
    t = (rng.standard_normal((R, K + 1, V)) * 2).astype(np.float32)
    d = (t[:, :K] + rng.standard_normal((R, K, V)) * 0.7).astype(np.float32)
    strip = np.zeros(V, dtype=bool)
    for c in strip_threads:
        for j in range(0, V // 4, 256):
            q = j + c
            if 4 * q < V:
                strip[4 * q:4 * q + 4] = True
    strip[0] = True
    mt = (rng.random((R, K + 1, V)) < frac) | strip
    md = (rng.random((R, K, V)) < frac) | strip
    t[mt] = -np.inf
    d[md] = -np.inf
    q = VF.softmax(d)
    x = np.array([[rng.choice(V, p=q[i, k]) for k in range(K)] for i in range(R)], dtype=np.int32).reshape(R, K)
    return d, t, x


@pytest.mark.parametrize("V", [4096, 4099])
def test_masked_logits_sampled(dsp, V):
    """-inf target and draft logits (masked vocabulary entries) at T = 1 and
    T = 0.8: kept counts and extra tokens match the oracle, no row comes
    out as the all-rejected token 0."""
    R, K = 40, 6
    d, t, x = _masked_inputs(V, R, K, V)
    for T, seed in ((1.0, 3), (0.8, 4)):
        n = _check(dsp, d, t, x, T, seed=seed)
        assert 0 < n.mean() < K
        _, tok = dsp.verify(dev(d), dev(t), dev(x), temperature=T, seed=seed)
        tok = tok.cpu().numpy()
        for i in range(R):  # the extra token never lands on a masked target entry
            assert np.isfinite(t[i, n[i], tok[i]]), (i, n[i], tok[i])


def test_masked_logits_greedy(dsp):
    """Greedy verification with -inf target logits: exact."""
    R, K, V = 12, 5, 4096
    d, t, x = _masked_inputs(11, R, K, V)
    am = np.argmax(t[:, :K], axis=-1).astype(np.int32)
    x = am.copy()
    for i in range(min(R, K)):
        x[i, i] = (x[i, i] + 1) % V
    n, tok = dsp.verify(dev(d), dev(t), dev(x), temperature=0.0)
    n_or, tok_or = VF.verify(d, t, x, temperature=0.0)
    np.testing.assert_array_equal(n.cpu().numpy(), n_or)
    np.testing.assert_array_equal(tok.cpu().numpy(), tok_or)


def test_greedy_ties(dsp):
    """Greedy with tied target maxima: the lowest tied index is the target's
    choice, so a draft on the higher tied index is rejected and the extra
    token is the lower one."""
    R, K, V = 6, 3, 1000
    rng = np.random.default_rng(12)
    t = rng.standard_normal((R, K + 1, V)).astype(np.float32)
    d = rng.standard_normal((R, K, V)).astype(np.float32)
    lo, hi = 17, 801
    t[:, :, lo] = t[:, :, hi] = 9.0
    x = np.full((R, K), lo, dtype=np.int32)
    x[1, 0] = hi
    x[2, 2] = hi
    n, tok = dsp.verify(dev(d), dev(t), dev(x), temperature=0.0)
    n_or, tok_or = VF.verify(d, t, x, temperature=0.0)
    np.testing.assert_array_equal(n.cpu().numpy(), n_or)
    np.testing.assert_array_equal(tok.cpu().numpy(), tok_or)
    np.testing.assert_array_equal(n_or, [K, 0, 2, K, K, K])
    assert np.all(tok_or == lo)


def test_long_drafts_sampled(dsp):
    """K = 40 drafts (the decision takes positions in chunks of 16): stops
    before 16, between 16 and 31, and rows that keep all 40."""
    R, K, V = 32, 40, 600
    d, t, x = _inputs(77, R, K, V, spread=0.05)
    n = _check(dsp, d, t, x, 1.0, seed=5)
    assert (n < 16).any() and ((n >= 16) & (n < 32)).any() and (n == K).any()


def test_long_drafts_greedy(dsp):
    """K = 40 at T = 0: a stop at each chunk edge and inside each chunk."""
    R, K, V = 12, 40, 500
    rng = np.random.default_rng(78)
    t = rng.standard_normal((R, K + 1, V)).astype(np.float32)
    d = rng.standard_normal((R, K, V)).astype(np.float32)
    x = np.argmax(t[:, :K], axis=-1).astype(np.int32)
    stops = [0, 1, 15, 16, 17, 31, 32, 33, 39]
    for i, k in enumerate(stops):
        x[i, k] = (x[i, k] + 1) % V
    n, tok = dsp.verify(dev(d), dev(t), dev(x), temperature=0.0)
    n_or, tok_or = VF.verify(d, t, x, temperature=0.0)
    np.testing.assert_array_equal(n.cpu().numpy(), n_or)
    np.testing.assert_array_equal(tok.cpu().numpy(), tok_or)
    np.testing.assert_array_equal(n_or, stops + [K] * (R - len(stops)))


def test_bad_token_past_the_stop_is_flagged(dsp):
    """An out-of-range draft token is reported wherever it lies; one past the
    stopping position changes nothing else."""
    R, K, V = 3, 20, 300
    rng = np.random.default_rng(79)
    t = rng.standard_normal((R, K + 1, V)).astype(np.float32)
    d = rng.standard_normal((R, K, V)).astype(np.float32)
    x = np.argmax(t[:, :K], axis=-1).astype(np.int32)
    x[1, 2] = (x[1, 2] + 1) % V  # row 1 stops at position 2
    n_or, tok_or = VF.verify(d, t, x, temperature=0.0)
    xb = x.copy()
    xb[1, 18] = V  # never tested
    from semi_autoregressive_block_amd import _lib
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    n, tok = dsp.verify(dev(d), dev(t), dev(xb), temperature=0.0, status=st)
    assert int(st.item()) & _lib.STATUS_BAD_TOKEN
    np.testing.assert_array_equal(n.cpu().numpy(), n_or)
    np.testing.assert_array_equal(tok.cpu().numpy(), tok_or)
    st.zero_()
    dsp.verify(dev(d), dev(t), dev(x), temperature=0.0, status=st)
    assert int(st.item()) == 0


def test_bad_draft_token_is_flagged(dsp):
    d, t, x = _inputs(5, 2, 3, 64)
    x[1, 0] = 64
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    dsp.verify(dev(d), dev(t), dev(x), status=st)
    from semi_autoregressive_block_amd import _lib
    assert int(st.item()) & _lib.STATUS_BAD_TOKEN
