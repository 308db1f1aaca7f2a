"""Pins for the oracle's Philox generator and Gumbel noise (CPU only)."""

import math
import os

import numpy as np
import pytest

from oracle import philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox_kat.txt")


def _kat_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            t = line.split()
            rows.append((t[0], int(t[1]), [int(x, 16) for x in t[2:6]],
                         [int(x, 16) for x in t[6:8]], [int(x, 16) for x in t[8:12]]))
    return rows


@pytest.mark.parametrize("row", _kat_rows(), ids=lambda r: f"{r[0]}-{r[2][0]:x}")
def test_known_answer_vectors(row):
    """Published known-answer vectors of the generator's definition."""
    variant, rounds, ctr, key, expect = row
    if variant == "philox4x32":
        got = [int(x) for x in philox.philox4x32([ctr], key, rounds)[0]]
    else:
        got = list(philox.philox4x64(ctr, key, rounds))
    assert got == expect


def test_4x64_matches_numpy_library():
    """numpy.random.Philox is a library implementation of Philox4x64-10; with
    its counter state set to c it emits the block for counter c + 1.  The
    64-bit instance shares the round structure with the 32-bit one the
    sampler uses, so this pins the structure (product halves, XOR pattern,
    word permutation, key schedule) independently of the constants."""
    rng = np.random.default_rng(7)
    for _ in range(6):
        ctr = [int(x) for x in rng.integers(0, 2**63, size=4, dtype=np.int64)]
        ctr[0] = ctr[0] & ~1  # keep the +1 carry out of the high words
        key = [int(x) for x in rng.integers(0, 2**63, size=2, dtype=np.int64)]
        bg = np.random.Philox(counter=np.array(ctr, dtype=np.uint64),
                              key=np.array(key, dtype=np.uint64))
        lib = [int(x) for x in bg.random_raw(4)]
        ours = list(philox.philox4x64([ctr[0] + 1] + ctr[1:], key))
        assert ours == lib


def test_round_count_matters():
    """A dropped or extra round changes the output (the KAT is for 10)."""
    a = philox.philox4x32([[1, 2, 3, 4]], (5, 6), rounds=10)
    assert not np.array_equal(a, philox.philox4x32([[1, 2, 3, 4]], (5, 6), rounds=9))
    assert not np.array_equal(a, philox.philox4x32([[1, 2, 3, 4]], (5, 6), rounds=11))


def test_counter_layout():
    """Draw v is word (v & 3) of the block at counter (v >> 2, step, row, 0)
    under key (seed_lo, seed_hi)."""
    seed, row, step, V = 0x1234_5678_9ABC_DEF0, 5, 3, 23
    bits = philox.gumbel_uniform_bits(seed, row, step, V)
    for v in range(V):
        w = philox.philox4x32([[v >> 2, step, row, 0]],
                              (seed & 0xFFFFFFFF, seed >> 32))[0, v & 3]
        assert int(bits[v]) == int(w)


def test_uniform_range_and_exactness():
    x = np.array([0, 1, 511, 512, 2**31, 2**32 - 1], dtype=np.uint64)
    u = philox.uniform_from_bits(x)
    assert u[0] == 2.0 ** -24
    assert u[-1] == 1.0 - 2.0 ** -24
    assert np.all(u.astype(np.float32).astype(np.float64) == u)  # exact in fp32
    assert np.all((u > 0) & (u < 1))


def test_uniform_statistics():
    """Mean 1/2, variance 1/12 and a chi-square test over 64 buckets for
    2^20 draws spread over rows, steps and vocabulary indices."""
    u = np.concatenate([philox.uniform_from_bits(philox.gumbel_uniform_bits(99, r, s, 4096))
                        for r in range(16) for s in range(16)])
    n = u.size
    assert abs(u.mean() - 0.5) < 5 * math.sqrt(1 / 12 / n)
    assert abs(u.var() - 1 / 12) < 5 * math.sqrt(1 / 180 / n)
    counts = np.bincount((u * 64).astype(int), minlength=64)
    e = n / 64
    chi2 = ((counts - e) ** 2 / e).sum()
    assert chi2 < 63 + 5 * math.sqrt(2 * 63)  # 63 dof, ~5 sigma


def test_streams_differ_by_row_step_seed():
    a = philox.gumbel_uniform_bits(1, 0, 0, 64)
    assert not np.array_equal(a, philox.gumbel_uniform_bits(1, 1, 0, 64))
    assert not np.array_equal(a, philox.gumbel_uniform_bits(1, 0, 1, 64))
    assert not np.array_equal(a, philox.gumbel_uniform_bits(2, 0, 0, 64))
    assert not np.array_equal(a, philox.gumbel_uniform_bits(1 << 32, 0, 0, 64))


def test_gumbel_moments():
    """Gumbel(0,1): mean = Euler-Mascheroni constant, variance = pi^2 / 6."""
    g = np.concatenate([philox.gumbel(4242, r, s, 8192) for r in range(8) for s in range(8)])
    n = g.size
    assert abs(g.mean() - 0.5772156649015329) < 5 * math.sqrt(math.pi ** 2 / 6 / n)
    assert abs(g.var() - math.pi ** 2 / 6) < 0.02
    assert g.min() >= -math.log(-math.log(2.0 ** -24)) - 1e-12
    assert g.max() <= -math.log(-math.log1p(-2.0 ** -24)) + 1e-9
