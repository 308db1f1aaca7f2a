"""Markov head: step logits and the gamma-step sequential sampler — oracle.

Test infrastructure only (see ``oracle/__init__``).

What is computed:

* Vanilla Markov head (page 1 §3.7, the paper's Eq. 5; page 2 §3.4 and
  §3.8.2 show the module): W1 is an embedding table [V, r], W2 a bias-free
  linear map from rank r to V; the step bias for previous token x is
  W2(W1[x]), i.e. the row W1[x] (length r) times the matrix W2 stored here as
  [r, V] (the math of nn.Linear(r, V) applied to a row vector).
* Step logits are the backbone's base logits for that block position plus
  that bias (page 2 §3.4, apply_step_logits).
* Sampling (page 2 §3.4 / §3.8.2, sample_block_tokens): left to right over the
  block positions; position 0 uses the supplied first previous token (the
  anchor token), every later position uses the token just sampled.
* Token choice (page 2 §3.4, sample_tokens; its body is not on the pages):
  temperature 0 -> argmax, lowest index on ties; temperature T > 0 ->
  Gumbel-max, argmax over v of l[v]/T + G[v] with G from ``oracle.philox``.

All arithmetic is float64 on the exact stored values of base, W1 and W2.
"""

from __future__ import annotations

import numpy as np

from . import philox


def step_logits(base_step, w1, w2, prev):
    """base_step [R, V] + W1[prev] @ W2 (float64).  prev [R] ints."""
    e = np.asarray(w1, dtype=np.float64)[np.asarray(prev, dtype=np.int64)]  # [R, r]
    return np.asarray(base_step, dtype=np.float64) + e @ np.asarray(w2, dtype=np.float64)


def perturb(logits, temperature, seed, rows, step):
    """The values whose argmax is the sampled token: logits themselves when
    temperature == 0, else logits / T + Gumbel(seed, row, step, v)."""
    if temperature == 0:
        return logits
    V = logits.shape[-1]
    g = np.stack([philox.gumbel(seed, int(r), step, V) for r in rows])
    return logits / temperature + g


def sample_block_tokens(base, w1, w2, first_prev, temperature=0.0, seed=0,
                        teacher=None, rows=None):
    """The gamma-step loop.

    base [R, gamma, V]; first_prev [R].  With ``teacher`` ([R, gamma] tokens,
    e.g. the device's own samples) step i uses teacher[:, i-1] as previous
    token instead of the oracle's own sample, so that each step can be
    compared on its own even after the two chains diverge.  ``rows`` are the
    global row indices of the R rows (the Philox key uses them; default
    0..R-1).

    Returns (tokens [R, gamma] int64, z [R, gamma, V] float64 where z are the
    values argmax'ed at each step, logits [R, gamma, V] float64)."""
    base = np.asarray(base)
    R, G, V = base.shape
    rows = np.arange(R) if rows is None else np.asarray(rows)
    prev = np.asarray(first_prev, dtype=np.int64).copy()
    tokens = np.zeros((R, G), dtype=np.int64)
    zs = np.zeros((R, G, V), dtype=np.float64)
    ls = np.zeros((R, G, V), dtype=np.float64)
    for i in range(G):
        l = step_logits(base[:, i, :], w1, w2, prev)
        z = perturb(l, temperature, seed, rows, i)
        tok = np.argmax(z, axis=1)  # first occurrence on ties
        tokens[:, i] = tok
        zs[:, i] = z
        ls[:, i] = l
        prev = np.asarray(teacher[:, i], dtype=np.int64) if teacher is not None else tok
    return tokens, zs, ls


def acceptable_tokens(z_row, margin):
    """Tokens a device may legitimately return for one step: every index whose
    value is within `margin` of the maximum (a unique index when the top-2
    margin exceeds `margin`)."""
    z_row = np.asarray(z_row)
    return np.flatnonzero(z_row >= z_row.max() - margin)
