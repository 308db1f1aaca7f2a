"""Lossless verify step: rejection sampling of a drafted block against the
target model — oracle.

Test infrastructure only (see ``oracle/__init__``).

What is computed (page 3, "如何评价 DeepSeek 发布 DSpark？哪些亮点值得关注？",
the speculative-decoding
primer: the target checks the K drafted positions in one pass, accepts from
left to right the prefix that agrees with its distribution P by rejection
sampling, cuts at the first failure and draws that position again from the
target, so that the output distribution is exactly the target's; page 4,
"DSpark 深度解读", §1.2 says the same).  The pages name the method but not
its steps; the reading here is the published speculative-sampling rule
(Leviathan, Kalman, Matias, "Fast Inference from Transformers via
Speculative Decoding", ICML 2023; Chen et al., "Accelerating Large Language
Model Decoding with Speculative Sampling", 2023), the one that makes the
output distribution the target's:

* q_k = softmax(draft_logits[k] / T), p_k = softmax(target_logits[k] / T)
  for the draft positions k = 0 .. K-1, and p_K for the position after them.
* Position k (all earlier ones accepted) keeps the drafted token x_k when
  u_k < p_k(x_k) / q_k(x_k) (so with probability min(1, p/q)); u_k is a
  uniform draw.
* At the first rejected k the output token is a draw from the residual
  max(0, p_k - q_k) (normalised); if all K are kept, one more token is drawn
  from p_K.  Either way n_acc drafted tokens plus one target token come out.
* T = 0 (greedy): x_k is kept when it is the argmax of the target logits
  (lowest index on ties) and the extra token is that argmax.

Random numbers (one counter-based generator, ``oracle.philox``, shared with
the device by its published definition): u_k is uniform_from_bits of word 0
of Philox4x32-10 at counter (k, 0, row, 2); the draws from the residual and
from p_K are Gumbel-max with the noise of counter (v >> 2, k, row, 1), word
v & 3 — streams 2 and 1, apart from the draft sampler's stream 0.

All arithmetic is float64.
"""

from __future__ import annotations

import numpy as np

from . import philox


def softmax(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def accept_uniform(seed, row, k):
    key = (int(seed) & 0xFFFFFFFF, (int(seed) >> 32) & 0xFFFFFFFF)
    w = philox.philox4x32(np.array([[k, 0, row, 2]], dtype=np.uint64), key)
    return float(philox.uniform_from_bits(w[0, 0]))


def verify_row(draft_logits, target_logits, draft_tokens, temperature, seed, row):
    """One request.  draft_logits [K, V], target_logits [K + 1, V],
    draft_tokens [K].  Returns (n_acc, the extra target token, the ratios
    p/q of the decided positions, the uniforms used)."""
    d = np.asarray(draft_logits, dtype=np.float64)
    t = np.asarray(target_logits, dtype=np.float64)
    K, V = d.shape
    ratios, us = [], []
    for k in range(K):
        x = int(draft_tokens[k])
        if temperature == 0:
            if x != int(np.argmax(t[k])):
                return k, int(np.argmax(t[k])), ratios, us
            continue
        q, p = softmax(d[k] / temperature), softmax(t[k] / temperature)
        u = accept_uniform(seed, row, k)
        ratio = p[x] / q[x]
        ratios.append(ratio)
        us.append(u)
        if not u < ratio:
            resid = np.maximum(p - q, 0.0)
            with np.errstate(divide="ignore"):
                z = np.log(resid) + philox.gumbel(seed, row, k, V, stream=1)
            return k, int(np.argmax(z)), ratios, us
    if temperature == 0:
        return K, int(np.argmax(t[K])), ratios, us
    z = t[K] / temperature + philox.gumbel(seed, row, K, V, stream=1)
    return K, int(np.argmax(z)), ratios, us


def verify(draft_logits, target_logits, draft_tokens, temperature=1.0, seed=0, rows=None):
    """draft_logits [R, K, V], target_logits [R, K + 1, V], draft_tokens
    [R, K].  Returns (n_acc [R], extra token [R])."""
    R = np.asarray(draft_tokens).shape[0]
    rows = np.arange(R) if rows is None else np.asarray(rows)
    n = np.zeros(R, dtype=np.int64)
    tok = np.zeros(R, dtype=np.int64)
    for i in range(R):
        n[i], tok[i], _, _ = verify_row(draft_logits[i], target_logits[i], draft_tokens[i], temperature, seed,
                                        int(rows[i]))
    return n, tok
