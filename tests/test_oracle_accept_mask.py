"""Pins for the accept-rate / tau and eval-mask oracles (CPU only)."""

import numpy as np
import scipy.special
import torch

import workloads as W
from oracle import accept_rate as OR
from oracle import eval_mask as OE


# ------------------------------------------------------------- accept rate
def test_identical_logits_accept_exactly_one():
    d = np.random.default_rng(1).standard_normal((3, 4, 1000)) * 3
    assert np.all(OR.accept_rate(d, d) == 1.0)


def test_symmetry_and_shift_invariance():
    rng = np.random.default_rng(2)
    d = rng.standard_normal((5, 777)) * 3
    t = d + rng.standard_normal((5, 777))
    np.testing.assert_array_equal(OR.accept_rate(d, t), OR.accept_rate(t, d))
    np.testing.assert_allclose(OR.accept_rate(d, d + rng.standard_normal((5, 1)) * 10), 1.0,
                               atol=1e-12)


def test_two_token_closed_form():
    """V = 2: accept = 1 - |sigmoid(d1 - d0) - sigmoid(t1 - t0)|."""
    rng = np.random.default_rng(3)
    d = rng.standard_normal((100, 2)) * 4
    t = rng.standard_normal((100, 2)) * 4
    expect = 1 - np.abs(scipy.special.expit(d[:, 1] - d[:, 0]) - scipy.special.expit(t[:, 1] - t[:, 0]))
    np.testing.assert_allclose(OR.accept_rate(d, t), expect, atol=1e-14)


def test_min_identity_with_library_softmax():
    """1 - TV(p, q) = sum_v min(p_v, q_v) (an identity independent of the
    |p - q| form), with p, q from torch's float64 softmax."""
    rng = np.random.default_rng(4)
    d = rng.standard_normal((8, 3, 5000)) * 3
    t = d + rng.standard_normal((8, 3, 1)) * rng.standard_normal((8, 3, 5000))
    p = torch.softmax(torch.from_numpy(d), -1).numpy()
    q = torch.softmax(torch.from_numpy(t), -1).numpy()
    np.testing.assert_allclose(OR.accept_rate(d, t), np.minimum(p, q).sum(-1), atol=1e-13)


def test_disjoint_spikes_accept_zero():
    d = np.zeros((1, 8))
    t = np.zeros((1, 8))
    d[0, 2] = 50
    t[0, 5] = 50
    assert OR.accept_rate(d, t)[0] < 1e-20


def test_range():
    rng = np.random.default_rng(5)
    a = OR.accept_rate(rng.standard_normal((200, 50)) * 10, rng.standard_normal((200, 50)) * 10)
    assert np.all((a >= 0) & (a <= 1))


def test_tau_closed_forms():
    """tau = 1 + sum_k prod_{i<=k} acc_i m_i: zero mask -> 1; all ones ->
    1 + gamma; constant acc a over a valid prefix of length L ->
    1 + a + a^2 + ... + a^L."""
    g = 8
    assert OR.tau(np.full(g, 0.7), np.zeros(g)) == 1.0
    assert OR.tau(np.ones(g), np.ones(g)) == 1.0 + g
    for L in range(g + 1):
        m = np.array([1] * L + [0] * (g - L))
        a = 0.6
        np.testing.assert_allclose(OR.tau(np.full(g, a), m), 1 + sum(a ** k for k in range(1, L + 1)),
                                   rtol=1e-15)
    acc = np.array([[0.9, 0.5, 0.2], [1.0, 0.0, 1.0]])
    np.testing.assert_allclose(OR.tau(acc, np.ones((2, 3))), [1 + 0.9 + 0.45 + 0.09, 2.0])


# --------------------------------------------------------------- eval mask
def test_eval_mask_hand_example():
    """Worked by hand from the three conditions and the cumulative product:
    gamma = 4, seq_len 10, loss mask zero at index 5 only.
      block (anchor 0, kept): labels 1,2,3,4 all valid      -> 1 1 1 1
      block (anchor 2, kept): labels 3,4,5,6; 5 unsupervised -> 1 1 0 0
      block (anchor 6, kept): labels 7,8,9,10; 10 >= 10      -> 1 1 1 0
      block (anchor 3, keep 0)                              -> 0 0 0 0
      block (anchor 9, kept): label 10 out of the sequence   -> 0 0 0 0"""
    lm = np.ones((1, 12), dtype=np.uint8)
    lm[0, 5] = 0
    m = OE.eval_mask([[0, 2, 6, 3, 9]], [[1, 1, 1, 0, 1]], [10], lm, 4)
    assert m[0].tolist() == [[1, 1, 1, 1], [1, 1, 0, 0], [1, 1, 1, 0], [0, 0, 0, 0], [0, 0, 0, 0]]
    # no loss mask: only bounds and keep matter
    m = OE.eval_mask([[0, 2, 6, 3, 9]], [[1, 1, 1, 0, 1]], [10], None, 4)
    assert m[0].tolist() == [[1, 1, 1, 1], [1, 1, 1, 1], [1, 1, 1, 0], [0, 0, 0, 0], [0, 0, 0, 0]]
    # a negative anchor on a kept block is treated as invalid
    assert OE.eval_mask([[-1]], [[1]], [10], None, 3)[0].tolist() == [[0, 0, 0]]


def test_eval_mask_invariants_and_library_cumprod():
    mask, _ = W.config4_structure()
    # shrink for speed: two rows, 64 blocks
    anchor, keep = mask.anchor[:2, :64], mask.keep[:2, :64].copy()
    keep[0, 5] = 0
    seq = np.array([4096, 900], dtype=np.int32)
    m = OE.eval_mask(anchor, keep, seq, mask.loss_mask[:2], 8)
    # independent vectorised predicate + torch.cumprod (library routine)
    L = anchor[:, :, None] + 1 + np.arange(8)[None, None, :]
    inb = L < seq[:, None, None]
    Lc = np.minimum(L, mask.loss_mask.shape[1] - 1)
    sup = np.take_along_axis(mask.loss_mask[:2, None, :].repeat(64, 1), Lc, axis=2) != 0
    pred = (keep[:, :, None] != 0) & (anchor[:, :, None] >= 0) & inb & sup
    ref = torch.cumprod(torch.from_numpy(pred.astype(np.int64)), dim=-1).numpy()
    assert np.array_equal(m, ref.astype(np.uint8))
    assert np.all(np.diff(m.astype(int), axis=-1) <= 0)          # prefix-zeroing
    assert np.all(m[0, 5] == 0)                                    # keep = 0
    first_bad = np.argmin(np.concatenate([pred, np.zeros_like(pred[..., :1])], -1), axis=-1)
    assert np.array_equal(m.sum(-1), first_bad)                    # first zero at first invalid


def test_eval_mask_all_valid_is_all_ones():
    m = OE.eval_mask([[0, 3]], [[1, 1]], [100], None, 16)
    assert np.all(m == 1)
