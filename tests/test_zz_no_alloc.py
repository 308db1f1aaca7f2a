"""The allocation-free Markov sampler entry point against the workspace one.

dspark_markov_sample_noalloc runs the same kernels as dspark_markov_sample
with its per-step keys in the library's fixed device array, so tokens and
step logits must be identical.  Two calls in a row, the second smaller (the
array keeps the first call's keys; the call must clear what it reads), then
the workspace entry point on the same inputs; plus the host-side rejection
of sizes beyond the array."""

import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DEV

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsp():
    import semi_autoregressive_block_amd as m
    return m


def _case(seed, R, gamma, V, r, wstd):
    g = torch.Generator(device=DEV).manual_seed(seed)
    base = torch.randn((R, gamma, V), generator=g, device=DEV).mul_(3)
    w1 = (torch.randn((V, r), generator=g, device=DEV) * wstd).to(torch.bfloat16)
    w2 = (torch.randn((r, V), generator=g, device=DEV) * wstd).to(torch.bfloat16)
    first = torch.randint(0, V, (R,), generator=g, device=DEV, dtype=torch.int32)
    return base, w1, w2, first


def _noalloc(dsp, base, w1, w2, first, T, seed):
    """One call of the C entry point with caller-owned outputs."""
    from semi_autoregressive_block_amd import _lib
    R, gamma, V = base.shape
    r = w1.shape[1]
    tok = torch.full((R, gamma), -7, dtype=torch.int32, device=DEV)
    sl = torch.full_like(base, float("nan"))
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    rc = dsp._LIB.dspark_markov_sample_noalloc(
        base.data_ptr(), w1.data_ptr(), w2.data_ptr(), first.data_ptr(), tok.data_ptr(), sl.data_ptr(),
        R, gamma, V, r, _lib.BF16, float(T), seed, st.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, dsp.last_error()
    return tok, sl, st


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_workspace_entry_point(dsp, order):
    cases = [
        # seed, R, gamma, V, r, weight std, temperature, philox seed
        (1, 128, 16, 151936, 256, 0.02, 0.0, 0),        # the serving round's sampler
        (2, 37, 5, 4096, 64, 0.5, 0.8, 1234),           # smaller, Gumbel, chain-moving weights
    ]
    for seed, R, gamma, V, r, wstd, T, ps in cases:
        base, w1, w2, first = _case(seed, R, gamma, V, r, wstd)
        tok_n, sl_n, st_n = _noalloc(dsp, base, w1, w2, first, T, ps)
        tok_w, sl_w = dsp.markov_sample(base, w1, w2, first, temperature=T, seed=ps, want_step_logits=True)
        torch.cuda.synchronize()
        assert int(st_n.item()) == 0
        assert torch.equal(tok_n, tok_w), (R, gamma, (tok_n != tok_w).sum().item())
        assert torch.equal(sl_n, sl_w), (R, gamma)
        assert int(tok_n.min()) >= 0 and int(tok_n.max()) < V
        del base, w1, w2, sl_n, sl_w
        torch.cuda.empty_cache()


def test_noalloc_binding_repeat_and_limit(dsp):
    """The binding's wrapper on a third, mid-size call after the others, and
    the fixed limit: R = 128 rows allow gamma <= 64, gamma = 65 is refused
    before anything is enqueued."""
    base, w1, w2, first = _case(3, 64, 8, 8192, 128, 0.3)
    tok = torch.empty((64, 8), dtype=torch.int32, device=DEV)
    a, _ = dsp.markov_sample_noalloc(base, w1, w2, first, temperature=1.1, seed=5, tokens=tok)
    b, _ = dsp.markov_sample(base, w1, w2, first, temperature=1.1, seed=5)
    assert a.data_ptr() == tok.data_ptr() and torch.equal(a, b)
    from semi_autoregressive_block_amd import _lib
    assert dsp.markov_sample_workspace_bytes(128, 64, 151936, 256) <= _lib.NOALLOC_SCRATCH_BYTES
    assert dsp.markov_sample_workspace_bytes(128, 65, 151936, 256) > _lib.NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(1)
    rc = dsp._LIB.dspark_markov_sample_noalloc(p, p, p, p, p, None, 128, 65, 151936, 256, _lib.BF16, 0.0, 0,
                                               None, None)
    assert rc == _lib.ERR_WORKSPACE and b"above the fixed" in dsp._LIB.dspark_last_error()
