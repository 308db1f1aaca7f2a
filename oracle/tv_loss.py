"""Teacher-forced Markov block logits, the L1 (total-variation) alignment
loss with its gradient, and tau_greedy — oracle.

Test infrastructure only (see ``oracle/__init__``).

What is computed:

* Teacher-forced block logits (page 1 §3.7: in training apply_block_logits
  takes every position's bias from that position's given previous token,
  not from a sampled one; page 4 §3.3 calls this teacher forcing): for row n
  with previous token prev[n], logits[n] = base[n] + W1[prev[n]] @ W2, with
  W1 [V, r] and W2 [r, V] as in ``oracle.markov``.  Optional soft cap
  (page 1 §3.12: the gemma4 backend's final logit soft-capping):
  c * tanh(logits / c) for c > 0.
* L1 distance of a row (page 1 §3.9, the paper's Eq. 10): sum over the
  vocabulary of |softmax(draft)_v - softmax(target)_v|, which is twice the
  total-variation distance.
* Loss: every draft position k = 0..gamma-1 of a block is weighted by
  w_k = exp(-k / decay) times its eval-mask bit, and the loss is the
  weighted sum of the row distances divided by the sum of the weights
  (page 1 §3.9: weights exp(-(k-1)/gamma) for 1-based k with
  loss_decay_gamma = 4; page 4 §4.1: e^{-k/gamma} with gamma = 4 — the same
  weights for a 0-based k; the pages divide by a global denominator and
  leave it unstated, read here as the sum of the weights of the valid
  positions).  With no valid position the loss is 0.
* Gradient of that loss with respect to the draft logits: a row with
  coefficient c_n = w_n m_n / sum(w m) contributes
  c_n * p_v * (s_v - sum_u s_u p_u), with p = softmax(draft),
  q = softmax(target) and s = sign(p - q) (sign(0) = 0: the subgradient
  that treats a tie as not moving).  This is the chain rule through the
  softmax: d p_u / d x_v = p_u (delta_uv - p_v).
* tau_greedy (page 1 §3.10: the greedy variant of tau uses argmax tokens):
  a position accepts when the draft's argmax token equals the target's
  (lowest index on ties), and tau_greedy = 1 + sum_k prod_{i<=k} a_i m_i.

All arithmetic is float64 on the exact stored values.
"""

from __future__ import annotations

import numpy as np

from .accept_rate import softmax


def block_logits(base, w1, w2, prev, softcap=0.0):
    """base [N, V] + W1[prev] @ W2, then c * tanh(l / c) when softcap c > 0."""
    e = np.asarray(w1, dtype=np.float64)[np.asarray(prev, dtype=np.int64)]  # [N, r]
    logits = np.asarray(base, dtype=np.float64) + e @ np.asarray(w2, dtype=np.float64)
    if softcap > 0:
        logits = softcap * np.tanh(logits / softcap)
    return logits


def l1_distance(draft, target):
    """Per row: sum_v |softmax(draft)_v - softmax(target)_v|."""
    return np.abs(softmax(draft) - softmax(target)).sum(axis=-1)


def position_weights(gamma, decay):
    """w_k = exp(-k / decay) for the block positions k = 0 .. gamma - 1."""
    return np.exp(-np.arange(gamma, dtype=np.float64) / decay)


def row_coefficients(eval_mask, decay):
    """c[b, a, k] = w_k * m[b, a, k] / sum(w * m) (all zeros if nothing is valid)."""
    m = np.asarray(eval_mask, dtype=np.float64)
    wm = m * position_weights(m.shape[-1], decay)
    den = wm.sum()
    return wm / den if den > 0 else np.zeros_like(wm)


def l1_loss(draft, target, eval_mask, decay=4.0):
    """draft, target [B, A, gamma, V]; eval_mask [B, A, gamma] -> scalar loss."""
    return float((row_coefficients(eval_mask, decay) * l1_distance(draft, target)).sum())


def l1_loss_grad(draft, target, eval_mask, decay=4.0):
    """d loss / d draft, [B, A, gamma, V]."""
    p, q = softmax(draft), softmax(target)
    s = np.sign(p - q)
    sp = (s * p).sum(axis=-1, keepdims=True)
    return row_coefficients(eval_mask, decay)[..., None] * p * (s - sp)


def greedy_accept(draft, target):
    """1.0 where argmax draft == argmax target (numpy argmax: lowest index on ties)."""
    return (np.argmax(draft, axis=-1) == np.argmax(target, axis=-1)).astype(np.float64)


def tau_greedy(draft, target, eval_mask):
    """[B, A]: 1 + sum_k prod_{i<=k} greedy_accept_i * m_i."""
    a = greedy_accept(draft, target) * np.asarray(eval_mask, dtype=np.float64)
    return 1.0 + np.cumprod(a, axis=-1).sum(axis=-1)
