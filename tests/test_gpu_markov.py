"""Markov-head sampler on the GPU vs the oracle.

Tokens must match exactly wherever the oracle's top-2 margin of the argmax'ed
values exceeds 1e-3 (elsewhere any token within 1e-3 of the maximum is
accepted).  Chains are compared teacher-forced: step i of the oracle uses the
device's token of step i-1, so one divergence cannot cascade.  Step logits
are compared at 1e-4 (float32 weights) / 2e-2 (bf16 weights; the device
multiplies the exact bf16 values with float32 accumulation, asserted far
tighter below)."""

import math

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import as_dtype, dev
from oracle import markov as OM

pytestmark = pytest.mark.gpu
MARGIN = 1e-3


@pytest.fixture(scope="module")
def dsp():
    import semi_autoregressive_block_amd as m
    return m


def _check(tok, base, w1v, w2v, first_prev, T, seed, rows=None):
    _, z, l = OM.sample_block_tokens(base, w1v, w2v, first_prev, T, seed, teacher=tok, rows=rows)
    R, G = tok.shape
    bad = [(r, i) for r in range(R) for i in range(G)
           if tok[r, i] not in OM.acceptable_tokens(z[r, i], MARGIN)]
    assert not bad, f"{len(bad)} mismatching tokens, first {bad[:5]}"
    return l


def _run_case(dsp, mk, want_logits=True):
    tok, sl = dsp.markov_sample(dev(mk.base), as_dtype(mk.w1, mk.wdtype), as_dtype(mk.w2, mk.wdtype),
                                dev(mk.first_prev), temperature=mk.temperature, seed=mk.seed,
                                want_step_logits=want_logits)
    return tok.cpu().numpy(), (sl.cpu().numpy() if sl is not None else None)


def test_config1_fp32(dsp):
    _, mk, _ = W.config1()
    tok, sl = _run_case(dsp, mk)
    l = _check(tok, mk.base, mk.vals("w1"), mk.vals("w2"), mk.first_prev, 0.0, mk.seed)
    assert np.abs(sl - l).max() < 1e-4


@pytest.mark.parametrize("R,G,V,r,T", [
    (37, 5, 10008, 64, 0.0),      # ragged rows and vocabulary sub-tiles, greedy
    (37, 5, 10008, 64, 0.7),      # Gumbel-max
    (130, 3, 4096, 256, 1.0),     # three row groups
    (20, 4, 2048, 512, 0.0),      # rank 512
    (9, 3, 1001, 40, 1.3),        # V not a multiple of 8: vector-ALU path, bf16 weights
    (64, 2, 4104, 72, 0.5),       # rank not a multiple of 32: zero-padded rank step
    (37, 3, 16384, 256, 0.0),     # one launch per step, ragged row blocks
    (37, 3, 16384, 256, 0.9),     # the same with Gumbel noise
    (37, 3, 49160, 256, 0.0),     # several tiles per workgroup, one partial tile
    (37, 4, 49160, 256, 0.9),     # the same with Gumbel noise
    (64, 4, 65536, 72, 0.5),      # rank zero-padded to 256, 64-row workgroups
    (128, 1, 60000, 256, 0.0),    # a single step
    (100, 6, 52000, 128, 1.0),    # rank 128, ragged last tile
    (81, 4, 40000, 256, 0.0),     # six row blocks, the last with one row: block-pipelined round kernel
    (96, 5, 40000, 256, 0.8),     # six full row blocks, Gumbel noise
    (120, 3, 30000, 64, 0.0),     # eight row blocks, rank 64
    (128, 6, 20000, 256, 1.0),    # eight full row blocks, Gumbel noise
])
def test_bf16_variants(dsp, R, G, V, r, T):
    mk = W.markov_case(R * 1000 + V, R, G, V, r, "bf16", base_std=2.0, w1_std=1.0,
                       w2_std=1.0 / math.sqrt(r), temperature=T, philox_seed=4242)
    tok, sl = _run_case(dsp, mk)
    l = _check(tok, mk.base, mk.vals("w1"), mk.vals("w2"), mk.first_prev, T, 4242)
    err = np.abs(sl - l).max()
    assert err < 2e-2 and err < 1e-4, err


def test_zero_w2_keeps_base_exactly(dsp):
    mk = W.markov_case(5, 16, 4, 4096, 256, "bf16", 3.0, 1.0, 0.0)
    mk.w2[:] = 0
    tok, sl = _run_case(dsp, mk)
    assert np.array_equal(sl, mk.base)
    assert np.array_equal(tok, np.argmax(mk.base, axis=2))


def test_permutation_chain(dsp):
    """W1 = c*I, W2 = c*P_pi (bf16-exact, c = 8): token_i = pi^(i+1)(first)."""
    rng = np.random.default_rng(3)
    V, r, R, G, c = 32, 32, 24, 12, 8.0
    pi = rng.permutation(V)
    w1 = np.zeros((V, r), np.float32)
    w1[np.arange(V), np.arange(V)] = c
    w2 = np.zeros((r, V), np.float32)
    w2[np.arange(V), pi] = c
    base = rng.standard_normal((R, G, V)).astype(np.float32)
    first = rng.integers(0, V, size=R).astype(np.int32)
    tok, _ = dsp.markov_sample(dev(base), as_dtype(W.to_bf16_bits(w1), "bf16"),
                               as_dtype(W.to_bf16_bits(w2), "bf16"), dev(first))
    tok = tok.cpu().numpy()
    cur = first.astype(np.int64)
    for i in range(G):
        cur = pi[cur]
        assert np.array_equal(tok[:, i], cur)


@pytest.mark.parametrize("R", [81, 100, 128])
def test_permutation_chain_row_blocks(dsp, R):
    """Tokens confined to the first 256 of V = 4096: W1[x] = c e_x and
    W2[k] = c e_pi(k) (bf16-exact, c = 8), so token_i = pi^(i+1)(first) for
    every row; with six to eight 16-row blocks every step's tokens come from
    the previous step's decoded keys of the same rows."""
    rng = np.random.default_rng(R)
    V, r, G, c = 4096, 256, 12, 8.0
    pi = rng.permutation(r)
    w1 = np.zeros((V, r), np.float32)
    w1[np.arange(r), np.arange(r)] = c
    w2 = np.zeros((r, V), np.float32)
    w2[np.arange(r), pi] = c
    base = rng.standard_normal((R, G, V)).astype(np.float32)
    first = rng.integers(0, r, size=R).astype(np.int32)
    tok, _ = dsp.markov_sample(dev(base), as_dtype(W.to_bf16_bits(w1), "bf16"),
                               as_dtype(W.to_bf16_bits(w2), "bf16"), dev(first))
    tok = tok.cpu().numpy()
    cur = first.astype(np.int64)
    for i in range(G):
        cur = pi[cur]
        assert np.array_equal(tok[:, i], cur), i


def test_gumbel_frequencies_on_device(dsp):
    """4096 rows with identical logits, W2 = 0, T = 1: the device's token
    frequencies follow softmax(l) (chi-square), and each row equals the
    oracle's Gumbel-max token where the margin allows."""
    V, R = 8, 4096
    l = np.array([0.3, -1.0, 1.2, 0.0, 0.5, -0.4, 2.0, 0.9], np.float32)
    base = np.tile(l, (R, 1, 1))
    w1 = np.zeros((V, 32), np.float32)
    w2 = np.zeros((32, V), np.float32)
    tok, _ = dsp.markov_sample(dev(base), dev(w1), dev(w2), dev(np.zeros(R, np.int32)),
                               temperature=1.0, seed=99)
    tok = tok.cpu().numpy()
    p = np.exp(l - l.max())
    p /= p.sum()
    counts = np.bincount(tok[:, 0], minlength=V)
    chi2 = ((counts - R * p) ** 2 / (R * p)).sum()
    assert chi2 < 7 + 5 * math.sqrt(14)
    _check(tok, base, w1, w2, np.zeros(R, np.int32), 1.0, 99)


def test_bad_first_token_is_flagged_not_faulting(dsp):
    mk = W.markov_case(6, 4, 2, 512, 32, "bf16", 1.0, 1.0, 0.1)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    fp = mk.first_prev.copy()
    fp[1] = 512 + 7
    fp[2] = -3
    tok, _ = dsp.markov_sample(dev(mk.base), as_dtype(mk.w1, "bf16"), as_dtype(mk.w2, "bf16"), dev(fp),
                               status=st)
    assert int(st.item()) & 2
    fp2 = fp.copy()
    fp2[1] = fp2[2] = 0  # out-of-range tokens read as token 0
    _check(tok.cpu().numpy(), mk.base, mk.vals("w1"), mk.vals("w2"), fp2, 0.0, 0)


def test_deterministic(dsp):
    mk = W.markov_case(7, 64, 4, 151936, 256, "bf16", 3.0, 0.02, 0.02, temperature=1.0, philox_seed=5)
    a = [dsp.markov_sample(dev(mk.base), as_dtype(mk.w1, "bf16"), as_dtype(mk.w2, "bf16"),
                           dev(mk.first_prev), temperature=1.0, seed=5)[0] for _ in range(2)]
    assert torch.equal(a[0], a[1])


def _full_size_check(dsp, inp, T, seed, rows):
    tok, _ = dsp.markov_sample(inp["base"], inp["w1"], inp["w2"], inp["first_prev"],
                               temperature=T, seed=seed)
    tok = tok.cpu().numpy()
    base = inp["base"][rows].cpu().numpy()
    w1 = inp["w1"].float().cpu().numpy()
    w2 = inp["w2"].float().cpu().numpy()
    fp = inp["first_prev"].cpu().numpy()[rows]
    _check(tok[rows], base, w1, w2, fp, T, seed, rows=np.asarray(rows))
    return tok


def test_config3_full_size(dsp):
    """R=64, gamma=16, V=151936, r=256, bf16 weights, T=1 Gumbel: the launch
    the bench times; every row checked step by step (teacher-forced)."""
    inp = W.config3_device(torch, torch.device("cuda:0"))
    tok = _full_size_check(dsp, inp, inp["temperature"], inp["seed"], list(range(64)))
    assert tok.min() >= 0 and tok.max() < 151936


def test_config5_markov_full_size(dsp):
    """R=128 rows, gamma=16, greedy: the round the bench times, every row."""
    inp = W.config5_device(torch, torch.device("cuda:0"))
    _full_size_check(dsp, inp, 0.0, 0, list(range(128)))

