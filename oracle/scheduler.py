"""Confidence head, prefix survival and the hardware-aware verify-length
scheduler — oracle.

Test infrastructure only (see ``oracle/__init__``).

What is computed:

* Confidence head (page 1 §3.8: one linear layer to a single output; with
  the Markov variant its input is the backbone hidden state concatenated with
  the Markov head's embedding of the previous token; page 4 §3.4: trained
  with a binary cross entropy, so its probability is the sigmoid of that
  output): c_n = sigmoid(w_h . h_n + w_e . W1[prev_n] + b), the conditional
  acceptance probability of draft position n given that its prefix is
  accepted.  Without the Markov input w_e is absent.
* Prefix survival (page 4 §5.1, a_k the chance that the first k drafts are
  all accepted; reading: the running product of the conditional
  probabilities along the block, which is what makes the page's worked
  example come out): a_k = prod_{i <= k} c_i for the block positions
  k = 1 .. gamma.
* Scheduler (page 4 §5.1): Theta_l = (1 + sum_{k=1}^{l} a_k) * SPS(l + 1)
  for l = 0 .. gamma, where SPS(m) is the target model's measured steps per
  second when it verifies m tokens; the search is causal-greedy: l grows
  from 0 and stops at the first l whose Theta is below Theta_{l-1}; the
  chosen length is the last one before that drop (gamma if none).

All arithmetic is float64.
"""

from __future__ import annotations

import numpy as np


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def confidence(hidden, weight_h, bias, w1=None, prev=None, weight_e=None):
    """hidden [..., H]; weight_h [H]; optional Markov input W1[prev] with
    weight_e [r].  Returns c [...]."""
    z = np.asarray(hidden, dtype=np.float64) @ np.asarray(weight_h, dtype=np.float64) + bias
    if weight_e is not None:
        e = np.asarray(w1, dtype=np.float64)[np.asarray(prev, dtype=np.int64)]
        z = z + e @ np.asarray(weight_e, dtype=np.float64)
    return sigmoid(z)


def prefix_survival(c):
    """a[..., k] = prod_{i <= k} c[..., i] along the last (block) axis."""
    return np.cumprod(np.asarray(c, dtype=np.float64), axis=-1)


def thetas(a_block, sps):
    """Theta_l for l = 0 .. gamma of one block: (1 + sum_{k<=l} a_k) * SPS[l],
    with sps[l] = SPS(l + 1)."""
    a_block = np.asarray(a_block, dtype=np.float64)
    acc = np.concatenate([[1.0], 1.0 + np.cumsum(a_block)])
    return acc * np.asarray(sps, dtype=np.float64)[: len(acc)]


def verify_length(a_block, sps):
    """Causal-greedy choice: the last l before Theta first drops."""
    th = thetas(a_block, sps)
    l = 0
    while l + 1 < len(th) and not th[l + 1] < th[l]:
        l += 1
    return l
