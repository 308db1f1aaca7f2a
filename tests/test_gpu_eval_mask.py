"""Eval mask on the GPU vs the oracle: bit-exact (integer work)."""

import numpy as np
import pytest

import workloads as W
from gpu_util import dev
from oracle import eval_mask as OE

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsp():
    import semi_autoregressive_block_amd as m
    return m


def _run(dsp, anchor, keep, seq, lm, gamma, status=None):
    return dsp.eval_mask(dev(anchor), dev(keep), dev(seq), None if lm is None else dev(lm),
                         gamma=gamma, status=status).cpu().numpy()


def test_config1(dsp):
    _, _, m = W.config1()
    got = _run(dsp, m.anchor, m.keep, m.seq_lens, m.loss_mask, m.gamma)
    assert np.array_equal(got, OE.eval_mask(m.anchor, m.keep, m.seq_lens, m.loss_mask, m.gamma))


def test_config4_full_size(dsp):
    m, _ = W.config4_structure()
    got = _run(dsp, m.anchor, m.keep, m.seq_lens, m.loss_mask, m.gamma)
    assert np.array_equal(got, OE.eval_mask(m.anchor, m.keep, m.seq_lens, m.loss_mask, m.gamma))
    assert got.sum() > 0 and (got == 0).sum() > 0


def test_config5_full_size(dsp):
    m = W.config5_structure()["mask"]
    got = _run(dsp, m.anchor, m.keep, m.seq_lens, None, m.gamma)
    ref = OE.eval_mask(m.anchor, m.keep, m.seq_lens, None, m.gamma)
    assert np.array_equal(got, ref)
    assert 0.1 < (ref[:, 0].sum(-1) < 16).mean() < 0.45  # about a quarter truncated


def test_hand_example_and_edges(dsp):
    import torch
    lm = np.ones((1, 12), dtype=np.uint8)
    lm[0, 5] = 0
    got = _run(dsp, np.array([[0, 2, 6, 3, 9]], np.int32), np.array([[1, 1, 1, 0, 1]], np.uint8),
               np.array([10], np.int32), lm, 4)
    assert got[0].tolist() == [[1, 1, 1, 1], [1, 1, 0, 0], [1, 1, 1, 0], [0, 0, 0, 0], [0, 0, 0, 0]]
    # negative anchor on a kept block: invalid and flagged
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = _run(dsp, np.array([[-1, 0]], np.int32), np.array([[1, 1]], np.uint8),
               np.array([10], np.int32), None, 3, status=st)
    assert got[0].tolist() == [[0, 0, 0], [1, 1, 1]] and int(st.item()) & 1
    # sequence longer than the loss-mask stride: labels past it are invalid and flagged
    st.zero_()
    got = _run(dsp, np.array([[4]], np.int32), np.array([[1]], np.uint8), np.array([20], np.int32),
               np.ones((1, 7), np.uint8), 4, status=st)
    assert got[0].tolist() == [[1, 1, 0, 0]] and int(st.item()) & 8


def test_random_many(dsp):
    rng = np.random.default_rng(5)
    for trial in range(5):
        B, A, g, S = int(rng.integers(1, 9)), int(rng.integers(1, 40)), int(rng.integers(1, 20)), 300
        anchor = rng.integers(-2, S, size=(B, A)).astype(np.int32)
        keep = (rng.random((B, A)) < 0.8).astype(np.uint8)
        seq = rng.integers(1, S + 1, size=B).astype(np.int32)
        lm = (rng.random((B, S)) < 0.9).astype(np.uint8)
        got = _run(dsp, anchor, keep, seq, lm, g)
        assert np.array_equal(got, OE.eval_mask(anchor, keep, seq, lm, g))
