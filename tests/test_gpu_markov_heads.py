"""Gated and recurrent Markov heads on the GPU vs the oracle: teacher-forced
block logits and the stateful sampler.

Bars: logits within 2e-2, and an RMS error under 2^-8 of the RMS of the
bias (logits - base), with bf16 W1/W2 (the rank-r row E is rounded to bf16
for the matrix cores, a relative error of at most 2^-9 per entry, about
2^-9 / sqrt(3) on average, so the bias moves by about that fraction; a
wrong index or term moves it by its own size); the hidden-state
products are exact bf16 values accumulated in float32), and within 1e-4
with float32 W1/W2 (E stays float32);
tokens equal the oracle's argmax wherever the oracle's top-2 margin exceeds
twice the logit bar, and otherwise lie within that margin of the oracle's
maximum.  The sampler is compared step by step with the oracle run on the
device's own tokens as previous tokens (its state then follows the same
path)."""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DEV, as_dtype, dev
from oracle import markov_heads as OH

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsp():
    import semi_autoregressive_block_amd as m
    return m


def _inputs(seed, kind, R, G, V, r, d, wdtype):
    rng = np.random.default_rng(seed)
    base = (rng.standard_normal((R, G, V)) * 3).astype(np.float32)
    hidden = W.to_bf16_bits(rng.standard_normal((R, G, d)).astype(np.float32))
    w1 = (rng.standard_normal((V, r)) * 0.5).astype(np.float32)
    w2 = (rng.standard_normal((r, V)) * 0.3).astype(np.float32)
    if wdtype == "bf16":
        w1, w2 = W.to_bf16_bits(w1), W.to_bf16_bits(w2)
    fan = d + r if kind == "gated" else 2 * r + d
    shape = (r, fan) if kind == "gated" else (3, r, fan)
    whead = W.to_bf16_bits((rng.standard_normal(shape) * 1.5 / np.sqrt(fan)).astype(np.float32))
    prev = rng.integers(0, V, size=(R, G)).astype(np.int32)
    return base, hidden, w1, w2, whead, prev


def _dev_args(base, hidden, w1, w2, whead, wdtype):
    return dev(base), as_dtype(hidden, "bf16"), as_dtype(w1, wdtype), as_dtype(w2, wdtype), as_dtype(whead, "bf16")


def _ref_args(hidden, w1, w2, whead, wdtype):
    return W.values(hidden, "bf16"), W.values(w1, wdtype), W.values(w2, wdtype), W.values(whead, "bf16")


def _bar(wdtype):
    return 2e-2 if wdtype == "bf16" else 1e-4


def _check_logits(got, ref, wdtype, base):
    err = np.abs(got - ref)
    assert err.max() < _bar(wdtype), err.max()
    if wdtype == "bf16":
        rms, bias = np.sqrt(np.mean(err ** 2)), np.sqrt(np.mean((ref - base) ** 2))
        assert rms < 2.0 ** -8 * bias, (rms, bias)


def _check_tokens(tok, z, margin):
    """tok [..] device tokens; z [.., V] oracle values they were chosen from."""
    z = z.reshape(-1, z.shape[-1])
    tok = tok.reshape(-1)
    best = z.max(axis=-1)
    chosen = z[np.arange(len(tok)), tok]
    assert np.all(chosen >= best - margin), np.max(best - chosen)
    top2 = np.sort(z, axis=-1)[:, -2:]
    sure = top2[:, 1] - top2[:, 0] > margin
    np.testing.assert_array_equal(tok[sure], np.argmax(z, axis=-1)[sure])
    assert sure.mean() >= 0.75


CASES = [
    # kind, B, gamma, V, r, d, wdtype, softcap
    ("gated", 3, 5, 4096, 64, 256, "bf16", 0.0),
    ("rnn", 3, 5, 4096, 64, 256, "bf16", 0.0),
    ("rnn", 37, 3, 2048, 40, 72, "bf16", 0.0),     # ragged rows, rank and hidden size off the tiles
    ("gated", 5, 4, 1001, 48, 96, "bf16", 0.0),    # V not a multiple of 8: vector-ALU vocabulary step
    ("rnn", 4, 6, 3000, 32, 64, "f32", 0.0),       # float32 W1/W2
    ("gated", 4, 4, 2048, 32, 64, "f32", 5.0),     # soft cap
    ("rnn", 2, 3, 1024, 512, 64, "bf16", 30.0),    # rank 512 (64 KB of staged state), soft cap
    ("rnn", 3, 2, 512, 8, 8, "bf16", 0.0),         # smallest rank and hidden size: the contraction is all tail
    ("gated", 1, 1, 64, 8, 24, "f32", 0.0),        # one position, d below one 32-wide slab
]


@pytest.mark.parametrize("kind,B,G,V,r,d,wdtype,softcap", CASES)
def test_block_logits(dsp, kind, B, G, V, r, d, wdtype, softcap):
    base, hidden, w1, w2, whead, prev = _inputs(B * G + V + r, kind, B, G, V, r, d, wdtype)
    logits, tok = dsp.markov_head_block_logits(kind, *_dev_args(base, hidden, w1, w2, whead, wdtype), dev(prev),
                                               softcap=softcap, want_tokens=True)
    ref = OH.block_logits(kind, base, *_ref_args(hidden, w1, w2, whead, wdtype), prev, softcap=softcap)
    _check_logits(logits.cpu().numpy(), ref, wdtype, base)
    _check_tokens(tok.cpu().numpy(), ref, 2 * _bar(wdtype))


@pytest.mark.parametrize("kind,temperature", [("gated", 0.0), ("rnn", 0.0), ("rnn", 0.8), ("gated", 1.3)])
def test_sampler_against_teacher_forced_oracle(dsp, kind, temperature):
    R, G, V, r, d = 37, 6, 4096, 64, 128
    base, hidden, w1, w2, whead, _ = _inputs(7 + R, kind, R, G, V, r, d, "bf16")
    first = np.random.default_rng(1).integers(0, V, size=R).astype(np.int32)
    tok, sl = dsp.markov_head_sample(kind, *_dev_args(base, hidden, w1, w2, whead, "bf16"), dev(first),
                                     temperature=temperature, seed=1234, want_step_logits=True)
    tok = tok.cpu().numpy().astype(np.int64)
    _, z, l = OH.sample_block_tokens(kind, base, *_ref_args(hidden, w1, w2, whead, "bf16"), first,
                                     temperature=temperature, seed=1234, teacher=tok)
    _check_logits(sl.cpu().numpy(), l, "bf16", base)
    margin = 2 * _bar("bf16") / (temperature if temperature > 0 else 1.0)
    _check_tokens(tok, z, margin)


def test_sampler_serving_shape_sampled_rows(dsp):
    """R = 128 requests, gamma = 16, V = 151936, r = 256, d = 4096 with the
    recurrent head; 17 rows (every eighth and the last) replayed by the
    oracle, tokens and step logits.

    At this size the bias is large (RMS about 3), so the fixed 2e-2 bar is
    replaced by the bound the arithmetic gives: E is rounded to bf16 (each
    entry moves by at most 2^-9 of itself) before the float32 product, so
    |l - l_oracle| <= 2^-9 sum_j |E_j W2[j, v]| plus float32 slack (1e-3
    covers the 256-term sums and the base add).  A token differs from the
    oracle's argmax only where the two logits are within the sum of their
    bounds."""
    R, G, V, r, d = 128, 16, 151936, 256, 4096
    rng = np.random.default_rng(21)
    base = torch.randn((R, G, V), generator=torch.Generator().manual_seed(5)).mul_(3).to(DEV)
    hid = W.to_bf16_bits(rng.standard_normal((R, G, d)).astype(np.float32))
    w1 = W.to_bf16_bits((rng.standard_normal((V, r)) * 0.5).astype(np.float32))
    w2 = W.to_bf16_bits((rng.standard_normal((r, V)) * 0.3).astype(np.float32))
    fan = 2 * r + d
    whead = W.to_bf16_bits((rng.standard_normal((3, r, fan)) * 1.5 / np.sqrt(fan)).astype(np.float32))
    first = rng.integers(0, V, size=R).astype(np.int32)
    tok, sl = dsp.markov_head_sample("rnn", base, as_dtype(hid, "bf16"), as_dtype(w1, "bf16"), as_dtype(w2, "bf16"),
                                     as_dtype(whead, "bf16"), dev(first), want_step_logits=True)
    tok = tok.cpu().numpy().astype(np.int64)
    rows = np.array(list(range(0, R, 8)) + [R - 1])
    sel = torch.as_tensor(rows, device=DEV)
    b = base[sel].cpu().numpy()
    got = sl[sel].cpu().numpy()
    del sl
    w1v, w2v, hv, whv = (W.values(w1, "bf16"), W.values(w2, "bf16").astype(np.float64),
                         W.values(hid[rows], "bf16"), W.values(whead, "bf16"))
    _, z, l = OH.sample_block_tokens("rnn", b, hv, w1v, w2v, whv, first[rows], teacher=tok[rows], rows=rows)
    # the oracle's E along the device's token path, for the rounding bound
    s_ = np.zeros((len(rows), r))
    prev = first[rows].astype(np.int64)
    aw2 = np.abs(w2v)
    mism = 0
    for k in range(G):
        s_, e = OH.rnn_cell(s_, w1v[prev], hv[:, k], whv)
        bound = 2.0 ** -9 * (np.abs(e) @ aw2) + 1e-3
        err = np.abs(got[:, k] - l[:, k])
        assert np.all(err <= bound), (k, float(err.max()), float((err - bound).max()))
        for j in range(len(rows)):
            a, t = int(np.argmax(z[j, k])), int(tok[rows[j], k])
            if a != t:
                mism += 1
                assert z[j, k, a] - z[j, k, t] <= bound[j, a] + bound[j, t], (rows[j], k, a, t)
        prev = tok[rows, k]
    res = got - l
    bias = l - b
    assert np.sqrt(np.mean(res ** 2)) < 2.0 ** -8 * np.sqrt(np.mean(bias ** 2))
    assert mism <= 0.05 * len(rows) * G, mism


def test_bad_previous_token_is_clamped_and_flagged(dsp):
    base, hidden, w1, w2, whead, prev = _inputs(3, "rnn", 2, 4, 512, 16, 32, "bf16")
    prev[0, 2] = -1
    prev[1, 0] = 512
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    logits, _ = dsp.markov_head_block_logits("rnn", *_dev_args(base, hidden, w1, w2, whead, "bf16"), dev(prev),
                                             status=st)
    from semi_autoregressive_block_amd import _lib
    assert int(st.item()) & _lib.STATUS_BAD_TOKEN
    fixed = prev.copy()
    fixed[0, 2] = fixed[1, 0] = 0
    ref = OH.block_logits("rnn", base, *_ref_args(hidden, w1, w2, whead, "bf16"), fixed)
    _check_logits(logits.cpu().numpy(), ref, "bf16", base)


def test_wrong_head_shape_is_rejected(dsp):
    base, hidden, w1, w2, whead, prev = _inputs(4, "gated", 2, 3, 256, 16, 32, "bf16")
    with pytest.raises(ValueError):
        dsp.markov_head_block_logits("rnn", *_dev_args(base, hidden, w1, w2, whead, "bf16"), dev(prev))


def test_empty_batch_is_a_no_op(dsp):
    base, hidden, w1, w2, whead, _ = _inputs(8, "rnn", 1, 4, 256, 16, 32, "bf16")
    args = _dev_args(base[:0], hidden[:0], w1, w2, whead, "bf16")
    tok, _ = dsp.markov_head_sample("rnn", *args, dev(np.zeros(0, dtype=np.int32)))
    assert tuple(tok.shape) == (0, 4)
    logits, _ = dsp.markov_head_block_logits("rnn", *args, dev(np.zeros((0, 4), dtype=np.int32)))
    assert tuple(logits.shape) == (0, 4, 256)


def test_workspace_reused_by_a_smaller_call(dsp):
    """One workspace, two calls in a row (the second on fewer rows and
    steps): the state, the projection and the key slots are rebuilt each
    call, so the second result matches the oracle too."""
    R, G, V, r, d = 40, 6, 2048, 32, 64
    ws = torch.empty(dsp.markov_head_sample_workspace_bytes("rnn", R, G, V, r), dtype=torch.uint8, device=DEV)
    for seed, (rr, gg) in ((11, (R, G)), (12, (17, 3))):
        base, hidden, w1, w2, whead, _ = _inputs(seed, "rnn", rr, gg, V, r, d, "bf16")
        first = np.random.default_rng(seed).integers(0, V, size=rr).astype(np.int32)
        tok, sl = dsp.markov_head_sample("rnn", *_dev_args(base, hidden, w1, w2, whead, "bf16"), dev(first),
                                         want_step_logits=True, workspace=ws)
        tok = tok.cpu().numpy().astype(np.int64)
        _, z, l = OH.sample_block_tokens("rnn", base, *_ref_args(hidden, w1, w2, whead, "bf16"), first, teacher=tok)
        _check_logits(sl.cpu().numpy(), l, "bf16", base)
        _check_tokens(tok, z, 2 * _bar("bf16"))
