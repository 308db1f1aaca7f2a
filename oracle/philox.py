"""Philox counter-based generator and the Gumbel noise the Markov sampler draws.

Test infrastructure only (see ``oracle/__init__``).

Philox-4xW-R is defined in Salmon, Moraes, Dror and Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3" (SC'11), Section 4.2: a counter of four W-bit
words is passed through R rounds.  Each round multiplies words 0 and 2 by two
fixed odd constants, keeps both halves (high and low W bits) of each 2W-bit
product, XORs the high halves with the two other counter words and the round
key, and permutes the words.  The round key starts at the user key and is
advanced by a Weyl increment (fixed constants) before every round but the
first.  The constants below are the ones that paper publishes for W = 32 and
W = 64.

The round structure is written once, generic over the word width, so that
the 64-bit instance can be checked against numpy's library implementation
(``numpy.random.Philox`` is Philox4x64-10) and the 32-bit instance against the
paper's published known-answer vectors.

Gumbel noise (the pages name temperature sampling but do not show its body,
page 2 §3.4 "sample_tokens"; the reading taken for the hot path is Gumbel-max
on a counter-based stream keyed by seed, row, step and vocabulary index):

* key     = (seed mod 2^32, seed >> 32)
* counter = (v >> 2, step, row, 0); the draw for vocabulary index v is output
  word (v & 3) of Philox4x32-10 at that counter;
* u       = ((x >> 9) + 1/2) * 2^-23, which lies in [2^-24, 1 - 2^-24] and is
  exactly representable in float32 and float64;
* G       = -ln(-ln u).
"""

from __future__ import annotations

import numpy as np

# Published Philox constants (SC'11 paper, Section 4.2 / its reference code).
_CONSTANTS = {
    32: dict(M0=0xD2511F53, M1=0xCD9E8D57, W0=0x9E3779B9, W1=0xBB67AE85),
    64: dict(M0=0xD2E7470EE14C6C93, M1=0xCA5A826395121157,
             W0=0x9E3779B97F4A7C15, W1=0xBB67AE8584CAA73B),
}


def _mulhilo32(a, m):
    """(high, low) 32-bit halves of the 64-bit product a*m; a is uint64 holding
    32-bit values, m a Python int below 2^32."""
    p = a * np.uint64(m)
    return p >> np.uint64(32), p & np.uint64(0xFFFFFFFF)


def _mulhilo64(a, m):
    """(high, low) 64-bit halves of the 128-bit product a*m using Python ints
    (object arrays).  Slow; used only by the width-64 instance."""
    p = a * m
    return p >> 64, p & ((1 << 64) - 1)


def _rounds(c0, c1, c2, c3, k0, k1, width, rounds):
    """Apply `rounds` Philox rounds to the counter words (c0..c3) under key
    (k0, k1).  Word arrays are numpy uint64 (width 32) or object arrays of
    Python ints (width 64)."""
    C = _CONSTANTS[width]
    mask = (1 << width) - 1
    if width == 32:
        mulhilo = _mulhilo32
        k0 = np.uint64(k0)
        k1 = np.uint64(k1)
        w0, w1, msk = np.uint64(C["W0"]), np.uint64(C["W1"]), np.uint64(mask)
    else:
        mulhilo = _mulhilo64
        w0, w1, msk = C["W0"], C["W1"], mask
    for r in range(rounds):
        if r > 0:  # Weyl key schedule: the key advances before every later round
            k0 = (k0 + w0) & msk
            k1 = (k1 + w1) & msk
        hi0, lo0 = mulhilo(c0, C["M0"])
        hi1, lo1 = mulhilo(c2, C["M1"])
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0), lo1, (hi0 ^ c3 ^ k1), lo0
    return c0, c1, c2, c3


def philox4x32(counter, key, rounds=10):
    """Philox4x32-R.  counter: array-like [..., 4] of uint32 words; key: two
    uint32 words.  Returns uint32 array [..., 4]."""
    ctr = np.asarray(counter, dtype=np.uint64)
    c = [ctr[..., i] & np.uint64(0xFFFFFFFF) for i in range(4)]
    out = _rounds(*c, int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF, 32, rounds)
    return np.stack(out, axis=-1).astype(np.uint32)


def philox4x64(counter, key, rounds=10):
    """Philox4x64-R on Python ints.  counter: sequence of four 64-bit words;
    key: two 64-bit words.  Returns a tuple of four ints."""
    c = [np.array(int(x), dtype=object) for x in counter]
    out = _rounds(*c, int(key[0]), int(key[1]), 64, rounds)
    return tuple(int(x) for x in out)


def gumbel_uniform_bits(seed, row, step, V, stream=0):
    """Raw 32-bit draws x[v], v in [0, V), for one (row, step); `stream` is
    the fourth counter word (0 for the draft sampler's noise; other values
    give streams independent of it)."""
    nblk = (V + 3) // 4
    ctr = np.zeros((nblk, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(nblk, dtype=np.uint64)
    ctr[:, 1] = step
    ctr[:, 2] = row
    ctr[:, 3] = stream
    key = (int(seed) & 0xFFFFFFFF, (int(seed) >> 32) & 0xFFFFFFFF)
    words = philox4x32(ctr, key)  # [nblk, 4]; word (v & 3) of block (v >> 2)
    return words.reshape(-1)[:V]


def uniform_from_bits(x):
    """u = ((x >> 9) + 1/2) * 2^-23 in float64 (exact)."""
    x = np.asarray(x, dtype=np.uint64)
    return ((x >> np.uint64(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def gumbel(seed, row, step, V, stream=0):
    """Gumbel(0,1) noise G[v] = -ln(-ln u[v]) for one (row, step), float64."""
    u = uniform_from_bits(gumbel_uniform_bits(seed, row, step, V, stream))
    return -np.log(-np.log(u))
