"""Pins of the verify-step oracle: the output distribution is the target's
(the lossless property, checked by chi-square over many independent rows),
the acceptance frequency equals sum_v min(p_v, q_v) (one minus the total
variation distance), closed cases (identical, disjoint supports) and a
hand-built greedy block."""

import numpy as np
from scipy import stats

from oracle import verify as VF

R, K, V = 6000, 3, 5


def _logits(seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((K, V)) * 1.3, rng.standard_normal((K + 1, V)) * 1.3


def _draft_tokens(dl, seed):
    """x_k ~ q_k for every row, from numpy's generator (independent of the
    Philox streams the verify step uses)."""
    rng = np.random.default_rng(seed)
    q = VF.softmax(dl)
    return np.stack([rng.choice(V, size=R, p=q[k]) for k in range(K)], axis=1)


def _chi2_ok(samples, p):
    counts = np.bincount(samples, minlength=len(p))
    live = p > 1e-12
    assert counts[~live].sum() == 0  # nothing outside the target's support
    return stats.chisquare(counts[live], len(samples) * p[live] / p[live].sum()).pvalue > 1e-3


def _run(dl, tl, x, seed=5):
    return VF.verify(np.broadcast_to(dl, (R, K, V)), np.broadcast_to(tl, (R, K + 1, V)), x, 1.0, seed)


def test_output_tokens_follow_the_target():
    dl, tl = _logits(1)
    x = _draft_tokens(dl, 2)
    n, extra = _run(dl, tl, x)
    p = VF.softmax(tl)
    first = np.where(n >= 1, x[:, 0], extra)
    assert _chi2_ok(first, p[0])
    kept = n >= 1  # given the first draft kept, the second output token follows p_1
    second = np.where(n[kept] >= 2, x[kept, 1], extra[kept])
    assert _chi2_ok(second, p[1])
    # acceptance of position 0: sum_v min(p_v, q_v)
    a = np.minimum(p[0], VF.softmax(dl)[0]).sum()
    assert abs(kept.mean() - a) < 4 * np.sqrt(a * (1 - a) / R)


def test_identical_distributions_keep_every_draft_and_draw_the_bonus_from_the_target():
    dl, tl = _logits(3)
    tl[:K] = dl
    x = _draft_tokens(dl, 4)
    n, extra = _run(dl, tl, x)
    assert np.all(n == K)
    assert _chi2_ok(extra, VF.softmax(tl)[K])


def test_disjoint_supports_reject_at_once_and_resample_from_the_target():
    dl = np.full((K, V), -1e3); dl[:, :2] = [0.0, 0.5]
    tl = np.full((K + 1, V), -1e3); tl[:, 2:] = [0.3, -0.2, 1.0]
    x = _draft_tokens(dl, 6)
    n, extra = _run(dl, tl, x)
    assert np.all(n == 0)
    assert _chi2_ok(extra, VF.softmax(tl)[0])


def test_greedy_block():
    t = np.zeros((2, 4, 6))
    for k, v in enumerate([3, 1, 4, 2]):
        t[:, k, v] = 2.0
    t[1, 0, 5] = 2.0  # tie at position 0 of row 1: the lowest index (3) wins
    d = np.zeros((2, 3, 6))
    x = np.array([[3, 1, 0], [3, 1, 4]])
    n, extra = VF.verify(d, t, x, temperature=0.0)
    np.testing.assert_array_equal(n, [2, 3])
    np.testing.assert_array_equal(extra, [4, 2])
