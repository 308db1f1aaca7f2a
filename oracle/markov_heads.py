"""Gated and recurrent Markov heads: step bias, teacher-forced block logits
and the gamma-step sampler — oracle.

Test infrastructure only (see ``oracle/__init__``).

What is computed (page 1, "03 · DSpark 建模", §3.7; page 4, "DSpark 深度解读",
§3.3, the table of the three head variants):

* Both heads produce the rank-r row E that the vanilla head takes as W1[x]
  (x the previous token); the step bias is then E @ W2 exactly as for the
  vanilla head (``oracle.markov``), and so are the step logits, the soft cap
  of the block logits and the token choice.
* Gated head: gate = sigmoid(W_g [h; W1[x]]), E = gate * W1[x] (elementwise).
  W_g maps the concatenation of the backbone hidden state h (length d) and
  W1[x] (length r), in that order, to r gate values; it is stored [r, d + r].
  Reading: the gate has r entries because it multiplies W1[x]; page 4 lists
  the added parameters as d x d, which cannot hold for r != d, so the shape
  follows the formula.  Page 1 shows no bias term in the gate; none is used.
* Recurrent head (the paper's Eq. 6): z_k = [s_{k-1}; W1[x_{k-1}]; h_k]
  (length 2r + d, in that order); with three maps W_g, W_c, W_o, each
  [r, 2r + d] (page 4's added-parameter count 3r(2r + d) agrees):
      s_k = sigmoid(W_g z_k) * s_{k-1} + (1 - sigmoid(W_g z_k)) * tanh(W_c z_k)
      E_k = tanh(W_o z_k)          (the bias is W2^T tanh(W_o z_k))
  so the bias at position k sees the state before position k's update.
  Readings: the state starts at zero at the first position of every block
  (the pages give no initial state); no bias terms (none are shown).  The
  three maps are stored stacked as one array [3, r, 2r + d] in the order
  gate, candidate, output.
* Training (page 1 §3.7): teacher-forced, every position k takes x_{k-1}
  from the given previous tokens, but the recurrent state still runs along
  the block.  Sampling: the state passes from one sampling step to the next
  and x_{k-1} is the token just sampled (the first previous token for k = 0).

All arithmetic is float64 on the exact stored values.
"""

from __future__ import annotations

import numpy as np

from .markov import perturb

GATED = "gated"
RNN = "rnn"


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def gated_embedding(h, w1, wg, prev):
    """h [N, d]; W1 [V, r]; W_g [r, d + r]; prev [N].  Returns gate * W1[prev]
    [N, r]."""
    e = np.asarray(w1, dtype=np.float64)[np.asarray(prev, dtype=np.int64)]
    z = np.concatenate([np.asarray(h, dtype=np.float64), e], axis=-1)
    gate = sigmoid(z @ np.asarray(wg, dtype=np.float64).T)
    return gate * e


def rnn_cell(s, e, h, w):
    """One recurrent update.  s [N, r] (s_{k-1}), e [N, r] (W1[x_{k-1}]),
    h [N, d], w [3, r, 2r + d].  Returns (s_k, E_k)."""
    w = np.asarray(w, dtype=np.float64)
    z = np.concatenate([np.asarray(s, dtype=np.float64), np.asarray(e, dtype=np.float64),
                        np.asarray(h, dtype=np.float64)], axis=-1)
    g = sigmoid(z @ w[0].T)
    c = np.tanh(z @ w[1].T)
    out = np.tanh(z @ w[2].T)
    return g * s + (1.0 - g) * c, out


def _embedding(kind, s, h, w1, whead, prev):
    """The rank-r row of one position for every row, and the next state."""
    if kind == GATED:
        return s, gated_embedding(h, w1, whead, prev)
    e = np.asarray(w1, dtype=np.float64)[np.asarray(prev, dtype=np.int64)]
    return rnn_cell(s, e, h, whead)


def block_logits(kind, base, hidden, w1, w2, whead, prev, softcap=0.0):
    """Teacher-forced logits of whole blocks.

    base [R, gamma, V]; hidden [R, gamma, d]; prev [R, gamma] (prev[:, k] is
    x_{k-1} of position k).  Returns logits [R, gamma, V] float64, soft-capped
    as c * tanh(l / c) when softcap c > 0."""
    base = np.asarray(base, dtype=np.float64)
    R, G, V = base.shape
    r = np.asarray(w1).shape[1]
    s = np.zeros((R, r))
    out = np.zeros((R, G, V))
    for k in range(G):
        s, e = _embedding(kind, s, np.asarray(hidden)[:, k], w1, whead, np.asarray(prev)[:, k])
        l = base[:, k] + e @ np.asarray(w2, dtype=np.float64)
        out[:, k] = softcap * np.tanh(l / softcap) if softcap > 0 else l
    return out


def sample_block_tokens(kind, base, hidden, w1, w2, whead, first_prev, temperature=0.0, seed=0,
                        teacher=None, rows=None):
    """The gamma-step loop with the head's state carried between steps.

    Same conventions as ``oracle.markov.sample_block_tokens`` (teacher tokens
    replace the oracle's own samples as previous tokens; ``rows`` are the
    global row indices that key the Gumbel noise).  Returns (tokens [R, gamma],
    z [R, gamma, V], logits [R, gamma, V])."""
    base = np.asarray(base, dtype=np.float64)
    R, G, V = base.shape
    r = np.asarray(w1).shape[1]
    rows = np.arange(R) if rows is None else np.asarray(rows)
    prev = np.asarray(first_prev, dtype=np.int64).copy()
    s = np.zeros((R, r))
    tokens = np.zeros((R, G), dtype=np.int64)
    zs = np.zeros((R, G, V))
    ls = np.zeros((R, G, V))
    for i in range(G):
        s, e = _embedding(kind, s, np.asarray(hidden)[:, i], w1, whead, prev)
        l = base[:, i] + e @ np.asarray(w2, dtype=np.float64)
        z = perturb(l, temperature, seed, rows, i)
        tok = np.argmax(z, axis=1)
        tokens[:, i], zs[:, i], ls[:, i] = tok, z, l
        prev = np.asarray(teacher[:, i], dtype=np.int64) if teacher is not None else tok
    return tokens, zs, ls
