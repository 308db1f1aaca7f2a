"""Teacher-forced Markov block logits and the L1 (TV) loss, its gradient and
tau_greedy on the GPU vs the oracle.

Bars: logits within 1e-4 (float32 weights) / 2e-2 (bf16 weights: the device
multiplies the exact bf16 values with float32 accumulation, asserted far
tighter below); argmax tokens exact wherever the oracle's top-2 margin
exceeds 1e-3; loss and per-row L1 distances within 1e-4 (float32 softmaxes);
gradients within 1e-4 of the row's largest gradient magnitude, except at
elements whose p and q agree to 1e-5 relative (there the sign of p - q, and
so the subgradient, may differ between float32 and float64), plus the slack
those ties leave on S = sum s p (c p times 2 sum_ties p, and 1e-5 for
S's float32 summation); tau_greedy
exact (ties between equal logits go to the lowest index on both sides)."""

import math

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DEV, as_dtype, dev, host_bits
from oracle import accept_rate as OR
from oracle import tv_loss as OT

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsp():
    import semi_autoregressive_block_amd as m
    return m


def _markov_inputs(seed, N, V, r, wdtype, wscale=0.05):
    rng = np.random.default_rng(seed)
    base = (rng.standard_normal((N, V)) * 3).astype(np.float32)
    w1 = (rng.standard_normal((V, r)) * wscale).astype(np.float32)
    w2 = (rng.standard_normal((r, V)) * wscale).astype(np.float32)
    if wdtype == "bf16":
        w1, w2 = W.to_bf16_bits(w1), W.to_bf16_bits(w2)
    prev = rng.integers(0, V, size=N).astype(np.int32)
    return base, w1, w2, prev


def _check_tokens(tok, ref_logits):
    """Rows with a clear winner (top-2 margin above 1e-3) must pick it; the
    others must pick a logit within 1e-3 of the row's maximum."""
    best = ref_logits.max(axis=-1)
    chosen = ref_logits[np.arange(len(tok)), tok]
    assert np.all(chosen >= best - 1e-3), np.max(best - chosen)
    top2 = np.sort(ref_logits, axis=-1)[:, -2:]
    sure = top2[:, 1] - top2[:, 0] > 1e-3
    np.testing.assert_array_equal(tok[sure], np.argmax(ref_logits, axis=-1)[sure])
    assert sure.mean() >= 0.75  # most rows have a clear winner


@pytest.mark.parametrize("N,V,r,wdtype,softcap", [
    (37, 4096, 64, "bf16", 0.0),       # ragged rows, several 64-column tiles
    (200, 20000, 256, "bf16", 0.0),    # two 128-row groups, ragged vocabulary tail
    (200, 20000, 256, "bf16", 30.0),   # soft cap
    (45, 2048, 512, "bf16", 0.0),      # rank 512
    (300, 8192, 128, "bf16", 0.0),     # W2 held in registers: 19 row blocks, the last ragged
    (17, 16384, 96, "bf16", 12.0),     # the same with rank 96 (three rank steps) and a soft cap
    (19, 1001, 40, "bf16", 5.0),       # V not a multiple of 8: vector-ALU path, soft cap
    (23, 3000, 48, "f32", 0.0),        # float32 weights: vector-ALU path
])
def test_block_logits(dsp, N, V, r, wdtype, softcap):
    base, w1, w2, prev = _markov_inputs(N + V, N, V, r, wdtype, wscale=0.3)
    logits, tok = dsp.markov_block_logits(dev(base), as_dtype(w1, wdtype), as_dtype(w2, wdtype), dev(prev),
                                          softcap=softcap, want_tokens=True)
    ref = OT.block_logits(base, W.values(w1, wdtype), W.values(w2, wdtype), prev, softcap)
    err = np.abs(logits.cpu().numpy() - ref).max()
    assert err < (2e-2 if wdtype == "bf16" else 1e-4), err
    assert err < 2e-4
    _check_tokens(tok.cpu().numpy(), ref)


def test_block_logits_full_vocabulary_sampled_rows(dsp):
    """V = 151936, r = 256, 384 rows (three row groups), checked on a sample."""
    N, V, r = 384, 151936, 256
    base, w1, w2, prev = _markov_inputs(5, N, V, r, "bf16", wscale=0.05)
    logits, tok = dsp.markov_block_logits(dev(base), as_dtype(w1, "bf16"), as_dtype(w2, "bf16"), dev(prev),
                                          want_tokens=True)
    rows = np.array([0, 1, 127, 128, 200, 255, 256, 383])
    ref = OT.block_logits(base[rows], W.values(w1, "bf16"), W.values(w2, "bf16"), prev[rows])
    got = logits[torch.as_tensor(rows, device=DEV)].cpu().numpy()
    assert np.abs(got - ref).max() < 2e-4
    _check_tokens(tok.cpu().numpy()[rows], ref)


def test_block_logits_bad_token_is_clamped_and_flagged(dsp):
    base, w1, w2, prev = _markov_inputs(9, 10, 2048, 64, "bf16")
    prev[3] = -5
    prev[7] = 2048
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    logits, _ = dsp.markov_block_logits(dev(base), as_dtype(w1, "bf16"), as_dtype(w2, "bf16"), dev(prev), status=st)
    from semi_autoregressive_block_amd import _lib
    assert int(st.item()) & _lib.STATUS_BAD_TOKEN
    fixed = prev.copy()
    fixed[[3, 7]] = 0
    ref = OT.block_logits(base, W.values(w1, "bf16"), W.values(w2, "bf16"), fixed)
    assert np.abs(logits.cpu().numpy() - ref).max() < 2e-4


def test_block_logits_bad_token_register_path(dsp):
    """The W2-in-registers kernel (V / 16 >= compute units) clamps and flags bad tokens too."""
    base, w1, w2, prev = _markov_inputs(11, 40, 8192, 64, "bf16")
    prev[0] = -1
    prev[33] = 8192
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    logits, tok = dsp.markov_block_logits(dev(base), as_dtype(w1, "bf16"), as_dtype(w2, "bf16"), dev(prev),
                                          status=st, want_tokens=True)
    from semi_autoregressive_block_amd import _lib
    assert int(st.item()) & _lib.STATUS_BAD_TOKEN
    fixed = prev.copy()
    fixed[[0, 33]] = 0
    ref = OT.block_logits(base, W.values(w1, "bf16"), W.values(w2, "bf16"), fixed)
    assert np.abs(logits.cpu().numpy() - ref).max() < 2e-4
    _check_tokens(tok.cpu().numpy(), ref)


def _loss_inputs(seed, B, A, g, V, dtype):
    rng = np.random.default_rng(seed)
    d = (rng.standard_normal((B, A, g, V)) * 3).astype(np.float32)
    t = (d + rng.standard_normal(d.shape) * rng.uniform(0.2, 2.0, size=(B, A, g, 1))).astype(np.float32)
    # some rows whose argmax agrees, some with tied maxima (lowest index wins)
    t[0, 0, 0] = d[0, 0, 0]
    i1, i2 = V // 3, V // 2
    d[0, 0, 1, i1] = d[0, 0, 1, i2] = d[0, 0, 1].max() + 1.0
    t[0, 0, 1, i1] = t[0, 0, 1, i2] = t[0, 0, 1].max() + 1.0
    m = np.ones((B, A, g), dtype=np.uint8)
    for b in range(B):
        for a in range(A):
            m[b, a, rng.integers(1, g + 1):] = 0
    if dtype == "bf16":
        d, t = W.to_bf16_bits(d), W.to_bf16_bits(t)
    return d, t, m


def _check_grad(g, d, t, m, ref, decay=4.0):
    """Gradient within 1e-4 of the row's largest magnitude, except at near
    ties of p and q (1e-5 relative), whose sign float32 cannot resolve.  The
    same ties enter S = sum_u s_u p_u with either sign, so S is known only to
    within 2 sum_ties p, and each element's c p (s - S) to within c p times
    that; the bar includes this slack, and 1e-5 more for S as a float32 sum
    (it matters where s - S vanishes, e.g. every s = +1 on the support, so
    that the exact gradient and the row's scale are zero)."""
    p, q = OR.softmax(d), OR.softmax(t)
    tie = np.abs(p - q) <= 1e-5 * np.maximum(p, q)
    c = OT.row_coefficients(m, decay)[..., None]
    s_slack = 2.0 * np.where(tie, p, 0.0).sum(axis=-1, keepdims=True)
    scale = np.abs(ref).max(axis=-1, keepdims=True)
    bad = (np.abs(g - ref) > 1e-4 * scale + c * p * (s_slack + 1e-5) + 1e-12) & ~tie
    assert not bad.any(), (int(bad.sum()), np.abs(g - ref)[bad].max())


@pytest.mark.parametrize("B,A,g,V,dtype", [
    (2, 3, 4, 1001, "bf16"),     # V not a multiple of 8: row-wise kernel, element loads
    (2, 3, 4, 1000, "bf16"),     # cluster kernel with one (ragged) slice per row
    (2, 3, 4, 4096, "bf16"),     # two slices per row
    (1, 5, 8, 3000, "f32"),
    (1, 2, 3, 7, "f32"),         # tiny vocabulary, row-wise kernel
])
def test_l1_loss_small(dsp, B, A, g, V, dtype):
    d, t, m = _loss_inputs(B * 100 + V, B, A, g, V, dtype)
    dv, tv = W.values(d, dtype), W.values(t, dtype)
    loss, grad, rows, tau = dsp.l1_loss(as_dtype(d, dtype), as_dtype(t, dtype), eval_mask=dev(m), want_grad=True,
                                        want_rows=True, want_tau_greedy=True)
    assert abs(loss.item() - OT.l1_loss(dv, tv, m)) < 1e-5
    assert np.abs(rows.cpu().numpy() - OT.l1_distance(dv, tv)).max() < 1e-5
    np.testing.assert_array_equal(tau.cpu().numpy(), OT.tau_greedy(dv, tv, m))
    _check_grad(grad.cpu().numpy(), dv, tv, m, OT.l1_loss_grad(dv, tv, m))


def test_l1_loss_full_vocabulary(dsp):
    B, A, g, V = 1, 2, 8, 151936
    d, t, m = _loss_inputs(11, B, A, g, V, "bf16")
    dv, tv = W.values(d, "bf16"), W.values(t, "bf16")
    loss, grad, rows, tau = dsp.l1_loss(as_dtype(d, "bf16"), as_dtype(t, "bf16"), eval_mask=dev(m), want_grad=True,
                                        want_rows=True, want_tau_greedy=True)
    assert abs(loss.item() - OT.l1_loss(dv, tv, m)) < 1e-5
    assert np.abs(rows.cpu().numpy() - OT.l1_distance(dv, tv)).max() < 1e-5
    np.testing.assert_array_equal(tau.cpu().numpy(), OT.tau_greedy(dv, tv, m))
    _check_grad(grad.cpu().numpy(), dv, tv, m, OT.l1_loss_grad(dv, tv, m))


@pytest.mark.parametrize("B,A,g,V,dtype,want_grad", [
    (4, 16, 8, 20000, "bf16", True),    # 7 slices, the last ragged; several rows per cluster
    (4, 16, 8, 20000, "bf16", False),   # no gradient: the pipeline without the S exchange
    (2, 16, 8, 10000, "f32", True),     # float32: 4 slices, the last ragged
    (1, 16, 8, 151936, "bf16", True),   # full vocabulary, 50 slices, ~8 rows per cluster
])
def test_l1_loss_cluster_pipeline(dsp, B, A, g, V, dtype, want_grad):
    """Every row of a launch whose clusters each run several rows through the
    three-stage pipeline (statistics, L1/S shares, gradient) against the oracle."""
    d, t, m = _loss_inputs(B * 1000 + V + int(want_grad), B, A, g, V, dtype)
    dv, tv = W.values(d, dtype), W.values(t, dtype)
    loss, grad, rows, tau = dsp.l1_loss(as_dtype(d, dtype), as_dtype(t, dtype), eval_mask=dev(m),
                                        want_grad=want_grad, want_rows=True, want_tau_greedy=True)
    assert abs(loss.item() - OT.l1_loss(dv, tv, m)) < 1e-5
    assert np.abs(rows.cpu().numpy() - OT.l1_distance(dv, tv)).max() < 1e-5
    np.testing.assert_array_equal(tau.cpu().numpy(), OT.tau_greedy(dv, tv, m))
    if want_grad:
        _check_grad(grad.cpu().numpy(), dv, tv, m, OT.l1_loss_grad(dv, tv, m))
    else:
        assert grad is None


def test_l1_loss_masked_vocabulary(dsp):
    """-inf logits: a padded vocabulary tail in both tensors (p = q = 0, sign 0),
    tokens masked in one tensor only, and a slice that is -inf throughout."""
    B, A, g, V = 2, 8, 8, 16384
    d, t, m = _loss_inputs(77, B, A, g, V, "f32")
    d[..., 15000:] = -np.inf
    t[..., 15000:] = -np.inf
    d[..., 3072:6144] = -np.inf          # the whole second slice of the draft
    t[..., 100:200] = -np.inf            # the target only
    d[0, 1, 2, 0] = -np.inf              # index 0
    db, tb = W.to_bf16_bits(d), W.to_bf16_bits(t)
    dv, tv = W.values(db, "bf16"), W.values(tb, "bf16")
    loss, grad, rows, tau = dsp.l1_loss(as_dtype(db, "bf16"), as_dtype(tb, "bf16"), eval_mask=dev(m),
                                        want_grad=True, want_rows=True, want_tau_greedy=True)
    assert abs(loss.item() - OT.l1_loss(dv, tv, m)) < 1e-5
    assert np.abs(rows.cpu().numpy() - OT.l1_distance(dv, tv)).max() < 1e-5
    np.testing.assert_array_equal(tau.cpu().numpy(), OT.tau_greedy(dv, tv, m))
    gh = grad.cpu().numpy()
    assert np.isfinite(gh).all()
    assert not gh[..., 15000:].any()
    _check_grad(gh, dv, tv, m, OT.l1_loss_grad(dv, tv, m))


def test_l1_loss_wait_timeout_poisons_and_recovers(dsp):
    """A poll limit of one, set from the host, drives the bounded waits of the
    cluster kernel into their timeout path while every workgroup still exits
    normally: the rows a timed-out workgroup served read NaN.  The next call at
    the default limit matches the oracle again."""
    d, t, m = _loss_inputs(12, 2, 16, 8, 151936, "bf16")
    db, tb = as_dtype(d, "bf16"), as_dtype(t, "bf16")
    dsp.set_wait_limit(1)
    try:
        loss, _, rows, _ = dsp.l1_loss(db, tb, eval_mask=dev(m), want_grad=True, want_rows=True)
        torch.cuda.synchronize()
    finally:
        dsp.set_wait_limit(0)
    assert np.isnan(rows.cpu().numpy()).any()
    loss, _, rows, _ = dsp.l1_loss(db, tb, eval_mask=dev(m), want_grad=True, want_rows=True)
    dv, tv = W.values(d, "bf16"), W.values(t, "bf16")
    assert np.abs(rows.cpu().numpy() - OT.l1_distance(dv, tv)).max() < 1e-5
    assert abs(loss.item() - OT.l1_loss(dv, tv, m)) < 1e-5


def test_l1_loss_no_mask_and_all_masked(dsp):
    d, t, _ = _loss_inputs(3, 1, 2, 4, 512, "f32")
    loss, grad, _, tau = dsp.l1_loss(as_dtype(d, "f32"), as_dtype(t, "f32"), want_grad=True, want_tau_greedy=True)
    ones = np.ones((1, 2, 4), dtype=np.uint8)
    assert abs(loss.item() - OT.l1_loss(d, t, ones)) < 1e-5
    np.testing.assert_array_equal(tau.cpu().numpy(), OT.tau_greedy(d, t, ones))
    zeros = np.zeros((1, 2, 4), dtype=np.uint8)
    loss, grad, _, tau = dsp.l1_loss(as_dtype(d, "f32"), as_dtype(t, "f32"), eval_mask=dev(zeros), want_grad=True,
                                     want_tau_greedy=True)
    assert loss.item() == 0.0
    assert torch.count_nonzero(grad).item() == 0
    assert np.all(tau.cpu().numpy() == 1.0)


def test_l1_loss_identical_is_zero_and_deterministic(dsp):
    d, _, m = _loss_inputs(4, 2, 2, 4, 4096, "bf16")
    x = as_dtype(d, "bf16")
    loss, grad, rows, tau = dsp.l1_loss(x, x, eval_mask=dev(m), want_grad=True, want_rows=True, want_tau_greedy=True)
    assert loss.item() == 0.0 and torch.count_nonzero(rows).item() == 0
    np.testing.assert_array_equal(tau.cpu().numpy(), 1.0 + np.cumprod(m, axis=-1).sum(axis=-1))
    assert torch.count_nonzero(grad).item() == 0
    _, t, _ = _loss_inputs(5, 2, 2, 4, 4096, "bf16")
    y = as_dtype(t, "bf16")
    a = dsp.l1_loss(x, y, eval_mask=dev(m), want_grad=True)
    b = dsp.l1_loss(x, y, eval_mask=dev(m), want_grad=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_block_logits_training_batch_sampled_rows(dsp):
    """The launch the bench times: 16384 rows (workload 4's training batch) x
    V = 151936, rank 256, bf16 W1/W2 (W2 held in registers over the whole
    launch); 256 rows checked against the oracle (the first and last rows, rows
    on either side of 16-row block and 128-row group edges, and a random
    sample), logits and greedy tokens."""
    bl = W.config4_block_logits_device(torch, DEV)
    N, V, r = bl["N"], bl["V"], bl["r"]
    logits, tok = dsp.markov_block_logits(bl["base"], bl["w1"], bl["w2"], bl["prev"], want_tokens=True)
    edges = {0, 1, 15, 16, 127, 128, 8191, 8192, N - 17, N - 16, N - 1}
    rows = sorted(edges | set(np.random.default_rng(21).choice(N, size=256 - len(edges), replace=False).tolist()))
    sel = torch.as_tensor(rows, device=DEV)
    w1 = bl["w1"].double().cpu().numpy()
    w2 = bl["w2"].double().cpu().numpy()
    ref = OT.block_logits(bl["base"][sel].double().cpu().numpy(), w1, w2, bl["prev"][sel].cpu().numpy())
    got = logits[sel].cpu().numpy()
    assert np.abs(got - ref).max() < 2e-4
    _check_tokens(tok[sel].cpu().numpy(), ref)


def test_l1_loss_training_batch(dsp):
    """The launch the bench times: workload 4's 4 x 512 x 8 rows of V = 151936
    bf16 with its eval mask.  Every row's L1 distance and greedy agreement
    (hence the loss and tau_greedy) against the oracle, 32 blocks at a time;
    the gradient on 16 blocks (128 rows), including the first and last."""
    inp = W.config4_device(torch, DEV)
    m = inp["mask"]
    em = dsp.eval_mask(dev(m.anchor), dev(m.keep), dev(m.seq_lens), dev(m.loss_mask), gamma=8)
    loss, grad, rows, tau = dsp.l1_loss(inp["draft"], inp["target"], eval_mask=em, want_grad=True,
                                        want_rows=True, want_tau_greedy=True)
    em_h, rows_h, tau_h = em.cpu().numpy(), rows.cpu().numpy(), tau.cpu().numpy()
    grad_blocks = {0, 4 * 512 - 1} | set(np.random.default_rng(31).choice(4 * 512, size=14, replace=False).tolist())
    w = OT.position_weights(8, 4.0)
    den_all = float((em_h * w).sum())
    l1 = np.zeros((4, 512, 8))
    agree = np.zeros((4, 512, 8))
    for c in range(0, 4 * 512, 32):
        idx = torch.arange(c, c + 32, device=DEV)
        bs, as_ = (idx // 512).cpu().numpy(), (idx % 512).cpu().numpy()
        dv = W.bf16_to_f32(host_bits(inp["draft"][idx // 512, idx % 512]))
        tv = W.bf16_to_f32(host_bits(inp["target"][idx // 512, idx % 512]))
        l1[bs, as_] = OT.l1_distance(dv, tv)
        agree[bs, as_] = OT.greedy_accept(dv, tv)
        for j in range(32):
            if c + j in grad_blocks:
                # the loss normalises its row weights over the whole batch, the
                # oracle over the block it is given: compare in the block's units
                b, a = int(bs[j]), int(as_[j])
                g = grad[b, a].cpu().numpy()[None, None].astype(np.float64)
                d1, t1, m1 = dv[j][None, None], tv[j][None, None], em_h[b, a][None, None]
                den_block = float((m1 * w).sum())
                if den_block == 0.0:
                    assert not g.any()
                    continue
                _check_grad(g * (den_all / den_block), d1, t1, m1, OT.l1_loss_grad(d1, t1, m1))
    assert np.abs(rows_h - l1).max() < 1e-5
    ref_loss = float((OT.row_coefficients(em_h, 4.0) * l1).sum())
    assert abs(loss.item() - ref_loss) < 1e-5 * max(1.0, abs(ref_loss))
    ref_tau = 1.0 + np.cumprod(agree * em_h, axis=-1).sum(axis=-1)
    np.testing.assert_array_equal(tau_h, ref_tau)
