"""Checks of the shared input generator (CPU only)."""

import numpy as np
import torch

import workloads as W


def test_bf16_rounding_matches_library_cast():
    """The host bf16 conversion rounds to nearest even exactly like torch's
    float32 -> bfloat16 cast (a library routine), ties included."""
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 0.0, -0.0,
                                  65504.0, 1e-40], dtype=np.float32)])
    ours = W.to_bf16_bits(x)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, lib)
    assert np.array_equal(W.bf16_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_structures_have_the_stated_shapes():
    a, k = W.config2_structure()
    assert a.shape == (1, 512) and k.sum() == 472 and np.all(k[0, 472:] == 0)
    assert np.all(np.diff(a[0, :472]) > 0) and a[0, :472].max() <= 4094
    mask, sigma = W.config4_structure()
    assert mask.anchor.shape == (4, 512) and sigma.min() >= 0.1 and sigma.max() <= 3.0
    for b in range(4):
        P = np.argmax(mask.loss_mask[b])
        assert 64 <= P <= 1024
        assert np.all(mask.anchor[b, :472] >= P)
    s = W.config5_structure()
    assert s["ctx_lens"].min() >= 1024 and s["ctx_lens"].max() <= 8192
    assert np.array_equal(s["anchor"][:, 0], s["ctx_lens"])
    trunc = (s["mask"].seq_lens - s["ctx_lens"] - 1) < 16
    assert 0.1 < trunc.mean() < 0.45
    assert (s["keep"] == 0).sum() == 6 and s["keep"].shape == (128, 1)  # about 5 % finished requests


def test_config1_shapes():
    attn, mk, mask = W.config1()
    assert attn.q.shape == (2, 64, 4, 64) and attn.k_ctx.shape == (256, 2, 64)
    assert mk.base.shape == (16, 8, 4096) and mk.w2.shape == (32, 4096)
    assert (attn.keep == 0).sum() == 4
