"""TV-distance accept rate and the tau statistic — oracle.

Test infrastructure only (see ``oracle/__init__``).

What is computed:

* Accept rate (page 1 §3.9, the paper's Eq. 8; page 2 §3.5 and §3.8.3 show
  the expression): softmax of the draft logits and of the target logits over
  the vocabulary, the accept rate is 1 - 1/2 * sum_v |p_v - q_v| (one minus
  the total-variation distance), clamped to [0, 1] (the clamp is from
  page 1 §3.9; page 2's snippet omits it, and it only matters for rounding).
  Both softmaxes are taken in float64 here (the pages take them in float32,
  upcasting the stored logits).
* tau (page 1 §3.10): expected accepted drafts per block is the sum over k of
  the running product over i <= k of accept[i] * eval_mask[i]; tau adds one
  for the bonus token.
"""

from __future__ import annotations

import numpy as np


def softmax(x):
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


def accept_rate(draft, target):
    """draft, target [..., V] -> accept [...] (float64)."""
    p = softmax(draft)
    q = softmax(target)
    tv = 0.5 * np.abs(p - q).sum(axis=-1)
    return np.clip(1.0 - tv, 0.0, 1.0)


def tau(accept, eval_mask):
    """accept, eval_mask [..., gamma] -> tau [...]."""
    w = np.asarray(accept, dtype=np.float64) * np.asarray(eval_mask, dtype=np.float64)
    return 1.0 + np.cumprod(w, axis=-1).sum(axis=-1)
