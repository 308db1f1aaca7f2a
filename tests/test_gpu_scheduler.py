"""Confidence head, prefix survival and the verify-length scheduler on the
GPU vs the oracle.

Bars: confidences, survivals and throughputs within 1e-5 (float32 dot
products and products); verify lengths exact except where the oracle's
decisive throughput comparison is within 1e-5 relative (a float32 near-tie);
the page's worked example reproduced to the two decimals it prints."""

import os

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DEV, as_dtype, dev
from oracle import scheduler as OS

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def dsp():
    import semi_autoregressive_block_amd as m
    return m


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def test_worked_example_on_device(dsp):
    vals = {}
    for line in open(os.path.join(HERE, "golden", "scheduler_worked_example.txt")):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            vals[k] = [float(x) for x in v]
    c = np.array(vals["confidence"] + [0.3])
    hidden = np.log(c / (1 - c)).reshape(1, 1, 3, 1)  # sigmoid^-1, weight 1, bias 0
    vlen, conf, surv, theta = dsp.confidence_schedule(_f32(hidden), _f32([1.0]), 0.0, _f32(vals["sps"]),
                                                      want_theta=True)
    np.testing.assert_allclose(conf.cpu().numpy().ravel(), c, atol=1e-6)
    np.testing.assert_array_equal(np.round(theta.cpu().numpy().astype(np.float64).ravel()[:3], 2), vals["theta"])
    assert int(vlen.item()) == int(vals["chosen_length"][0])


def _check(vlen, conf, surv, theta, ref_c, sps):
    ref_a = OS.prefix_survival(ref_c)
    np.testing.assert_allclose(conf, ref_c, atol=1e-5)
    np.testing.assert_allclose(surv, ref_a, atol=1e-5)
    B, A, g = ref_c.shape
    for b in range(B):
        for a in range(A):
            th = OS.thetas(ref_a[b, a], sps)
            np.testing.assert_allclose(theta[b, a], th, rtol=1e-5)
            l = OS.verify_length(ref_a[b, a], sps)
            if vlen[b, a] != l:  # only a float32 near-tie at the decisive comparison may differ
                k = min(l, vlen[b, a]) + 1
                assert abs(th[k] - th[k - 1]) <= 1e-5 * th[k - 1], (b, a, vlen[b, a], l)


@pytest.mark.parametrize("B,A,g,H,hdtype,markov", [
    (3, 5, 8, 300, "bf16", True),
    (2, 4, 16, 1000, "f32", True),
    (128, 1, 16, 4096, "bf16", False),   # serving shape: one block per request
    (1, 1, 1, 7, "f32", False),
])
def test_random_blocks(dsp, B, A, g, H, hdtype, markov):
    rng = np.random.default_rng(B * 1000 + H)
    hidden = rng.standard_normal((B, A, g, H)).astype(np.float32)
    wh = (rng.standard_normal(H) / np.sqrt(H) * 2).astype(np.float32)
    bias = 1.5
    sps = np.sort(rng.uniform(0.3, 1.0, g + 1))[::-1].astype(np.float32)
    sps[g // 2 + 1:] *= 0.6  # a hardware cliff
    if hdtype == "bf16":
        hidden = W.to_bf16_bits(hidden)
    hv = W.values(hidden, hdtype)
    kw = {}
    if markov:
        V, r = 1000, 40
        w1 = W.to_bf16_bits(rng.standard_normal((V, r)).astype(np.float32) * 0.5)
        prev = rng.integers(0, V, size=(B, A, g)).astype(np.int32)
        we = rng.standard_normal(r).astype(np.float32) * 0.3
        kw = dict(w1=as_dtype(w1, "bf16"), prev=dev(prev), weight_e=_f32(we))
        ref_c = OS.confidence(hv, wh, bias, W.values(w1, "bf16"), prev, we)
    else:
        ref_c = OS.confidence(hv, wh, bias)
    vlen, conf, surv, theta = dsp.confidence_schedule(as_dtype(hidden, hdtype), _f32(wh), bias, _f32(sps),
                                                      want_theta=True, **kw)
    _check(vlen.cpu().numpy(), conf.cpu().numpy(), surv.cpu().numpy(), theta.cpu().numpy(), ref_c, sps)


def test_bad_previous_token_is_clamped_and_flagged(dsp):
    rng = np.random.default_rng(3)
    hidden = rng.standard_normal((1, 2, 4, 64)).astype(np.float32)
    wh = rng.standard_normal(64).astype(np.float32) * 0.1
    V, r = 50, 16
    w1 = rng.standard_normal((V, r)).astype(np.float32)
    we = rng.standard_normal(r).astype(np.float32) * 0.2
    prev = rng.integers(0, V, size=(1, 2, 4)).astype(np.int32)
    prev[0, 1, 2] = V + 3
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    sps = np.linspace(1.0, 0.8, 5).astype(np.float32)
    vlen, conf, surv, _ = dsp.confidence_schedule(_f32(hidden), _f32(wh), 0.0, _f32(sps), w1=_f32(w1),
                                                  prev=dev(prev), weight_e=_f32(we), status=st)
    from semi_autoregressive_block_amd import _lib
    assert int(st.item()) & _lib.STATUS_BAD_TOKEN
    fixed = prev.copy()
    fixed[0, 1, 2] = 0
    np.testing.assert_allclose(conf.cpu().numpy(), OS.confidence(hidden, wh, 0.0, w1, fixed, we), atol=1e-5)
