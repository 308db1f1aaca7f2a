"""Pins for the block-attention oracle (CPU only)."""

import numpy as np
import pytest
import scipy.special
import torch

import workloads as W
from oracle import attention as OA


def test_mask_rules_hand_enumerated():
    """The three rules written out by hand for a 4-token context and two
    2-row blocks (page 1 §3.4): causal context, each block sees the context
    strictly before its anchor plus its own block, a keep=0 block sees
    nothing."""
    # anchors (1, 3), keep (1, 0)
    expect = np.array([
        [1, 0, 0, 0, 0, 0, 0, 0],
        [1, 1, 0, 0, 0, 0, 0, 0],
        [1, 1, 1, 0, 0, 0, 0, 0],
        [1, 1, 1, 1, 0, 0, 0, 0],
        [1, 0, 0, 0, 1, 1, 0, 0],
        [1, 0, 0, 0, 1, 1, 0, 0],
        [0, 0, 0, 0, 0, 0, 0, 0],
        [0, 0, 0, 0, 0, 0, 0, 0]], dtype=bool)
    assert np.array_equal(OA.full_mask(4, 2, [1, 3], [1, 0]), expect)
    # anchors (2, 0), keep (1, 1): the second block sees only itself
    expect2 = expect.copy()
    expect2[4:6] = [1, 1, 0, 0, 1, 1, 0, 0]
    expect2[6:8] = [0, 0, 0, 0, 0, 0, 1, 1]
    assert np.array_equal(OA.full_mask(4, 2, [2, 0], [1, 1]), expect2)
    # anchor at the end of the context: the whole context is visible
    m = OA.full_mask(3, 2, [3], [1])
    assert m[3].tolist() == [1, 1, 1, 1, 1] and m[4].tolist() == [1, 1, 1, 1, 1]


def _tiny_cases():
    out = []
    for seed, ctx, A, gamma, Hq, Hkv, D in [
            (1, [5, 9], 3, 2, 4, 2, 8), (2, [7], 4, 3, 2, 2, 4),
            (3, [1, 0, 6], 2, 4, 6, 3, 8), (4, [12], 5, 2, 4, 1, 4)]:
        c = W.attention_case(seed, ctx, A, gamma, Hq, Hkv, D, "f32")
        c.keep[0, -1] = 0  # a masked block
        c.anchor[0, 0] = 0  # a block that sees no context
        out.append(c)
    return out


@pytest.mark.parametrize("case", _tiny_cases())
def test_set_definition_equals_full_mask_brute_force(case):
    args = [case.vals("q"), case.vals("k_ctx"), case.vals("v_ctx"), case.ctx_offsets,
            case.vals("k_blk"), case.vals("v_blk"), case.anchor, case.keep, case.gamma,
            case.scale]
    o1, l1 = OA.block_attention(*args)
    o2, l2 = OA.block_attention_dense(*args)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)
    assert np.all(o1[0, -case.gamma:] == 0) and np.all(np.isneginf(l1[0, :, -case.gamma:]))


def test_library_sdpa_per_block():
    """Each kept block equals torch's scaled_dot_product_attention (CPU,
    float64) over [context keys before the anchor; own-block keys], with the
    key/value heads repeated to the query heads; also for scale = 1."""
    for scale in (None, 1.0):
        c = W.attention_case(11, [40, 17], 4, 8, 8, 2, 16, "f32", scale=scale)
        c.keep[1, 2] = 0
        out, lse = OA.block_attention(c.vals("q"), c.vals("k_ctx"), c.vals("v_ctx"),
                                      c.ctx_offsets, c.vals("k_blk"), c.vals("v_blk"),
                                      c.anchor, c.keep, c.gamma, c.scale)
        g, rep = c.gamma, 8 // 2
        for b in range(2):
            c0 = c.ctx_offsets[b]
            for a in range(4):
                rows = slice(a * g, (a + 1) * g)
                if not c.keep[b, a]:
                    assert np.all(out[b, rows] == 0)
                    continue
                p = c.anchor[b, a]
                k = np.concatenate([c.vals("k_ctx")[c0:c0 + p], c.vals("k_blk")[b, rows]])
                v = np.concatenate([c.vals("v_ctx")[c0:c0 + p], c.vals("v_blk")[b, rows]])
                qt = torch.from_numpy(c.vals("q")[b, rows].astype(np.float64)).transpose(0, 1)
                kt = torch.from_numpy(k.astype(np.float64)).transpose(0, 1).repeat_interleave(rep, 0)
                vt = torch.from_numpy(v.astype(np.float64)).transpose(0, 1).repeat_interleave(rep, 0)
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qt[None], kt[None], vt[None], scale=c.scale)[0].transpose(0, 1).numpy()
                np.testing.assert_allclose(out[b, rows], ref, atol=1e-12)
                s = c.scale * np.einsum("ghd,jhd->hgj", qt.numpy().transpose(1, 0, 2),
                                        kt.numpy().transpose(1, 0, 2))
                np.testing.assert_allclose(lse[b, :, rows], scipy.special.logsumexp(s, axis=-1),
                                           atol=1e-12)


def test_zero_query_closed_forms():
    """Q = 0 gives uniform weights over the visible set.  With V_ctx[j] = j and
    V_blk[a, k] = 1000 + k in dimension 0 the output is the mean of the
    visible indices: (p(p-1)/2 + 1000*gamma + gamma(gamma-1)/2) / (p + gamma);
    with V = 1 everywhere it is 1 for kept blocks and 0 for masked ones."""
    S, A, g, Hq, Hkv, D = 30, 5, 4, 4, 2, 8
    c = W.attention_case(5, [S], A, g, Hq, Hkv, D, "f32")
    c.keep[0, 3] = 0
    c.anchor[0, :] = [0, 7, 30, 12, 29]
    q = np.zeros_like(c.q)
    vctx = np.zeros_like(c.v_ctx)
    vctx[:, :, 0] = np.arange(S)[:, None]
    vctx[:, :, 1] = 1
    vblk = np.zeros_like(c.v_blk)
    vblk[0, :, :, 0] = (1000 + np.arange(A * g) % g)[:, None]
    vblk[0, :, :, 1] = 1
    out, _ = OA.block_attention(q, c.k_ctx, vctx, c.ctx_offsets, c.k_blk, vblk,
                                c.anchor, c.keep, g, c.scale)
    for a in range(A):
        rows = out[0, a * g:(a + 1) * g]
        if not c.keep[0, a]:
            assert np.all(rows == 0)
            continue
        p = c.anchor[0, a]
        mean = (p * (p - 1) / 2 + 1000 * g + g * (g - 1) / 2) / (p + g)
        np.testing.assert_allclose(rows[:, :, 0], mean, rtol=1e-13)
        np.testing.assert_allclose(rows[:, :, 1], 1.0, rtol=1e-13)


def test_one_hot_value_probe():
    """Q = 0 and V_j = e_j over the concatenated index space: each output row
    is 1/|vis| exactly on the visible set (enumerates the mask position by
    position through the attention itself)."""
    S, A, g, D = 20, 3, 4, 32
    c = W.attention_case(6, [S], A, g, 2, 1, D, "f32")
    c.anchor[0] = [0, 13, 20]
    c.keep[0] = [1, 1, 1]
    vctx = np.zeros_like(c.v_ctx)
    vctx[np.arange(S), 0, np.arange(S)] = 1
    vblk = np.zeros_like(c.v_blk)
    # own-block row k of every block is e_{S+k}: distinct from the context columns
    for j in range(A * g):
        vblk[0, j, 0, S + (j % g)] = 1
    out, _ = OA.block_attention(np.zeros_like(c.q), c.k_ctx, vctx, c.ctx_offsets, c.k_blk,
                                vblk, c.anchor, c.keep, g, c.scale)
    for a in range(A):
        p = c.anchor[0, a]
        expect = np.zeros(D)
        expect[:p] = 1.0 / (p + g)
        expect[S:S + g] = 1.0 / (p + g)
        for k in range(g):
            for h in range(2):
                np.testing.assert_allclose(out[0, a * g + k, h], expect, atol=1e-15)


def test_invisible_keys_do_not_matter():
    """Changing context K/V at positions >= anchor, or any other block's
    K/V, leaves a block's output unchanged."""
    c = W.attention_case(8, [25], 3, 4, 4, 2, 8, "f32")
    c.anchor[0] = [10, 3, 20]
    args = lambda kc, vc, kb, vb: OA.block_attention(c.q, kc, vc, c.ctx_offsets, kb, vb,
                                                      c.anchor, c.keep, 4, c.scale)[0]
    base = args(c.k_ctx, c.v_ctx, c.k_blk, c.v_blk)
    kc, vc = c.k_ctx.copy(), c.v_ctx.copy()
    kc[10:] += 5.0
    vc[10:] -= 3.0
    pert = args(kc, vc, c.k_blk, c.v_blk)
    np.testing.assert_array_equal(pert[0, 0:4], base[0, 0:4])   # block 0, anchor 10
    np.testing.assert_array_equal(pert[0, 4:8], base[0, 4:8])   # block 1, anchor 3
    assert not np.allclose(pert[0, 8:12], base[0, 8:12])       # block 2 sees 10..19
    kb, vb = c.k_blk.copy(), c.v_blk.copy()
    kb[0, 4:12] += 2.0
    vb[0, 4:12] += 2.0
    pert = args(c.k_ctx, c.v_ctx, kb, vb)
    np.testing.assert_array_equal(pert[0, 0:4], base[0, 0:4])
    assert not np.allclose(pert[0, 4:8], base[0, 4:8])


def test_rows_helper_matches_full():
    c = W.attention_case(9, [33, 50], 3, 8, 8, 2, 16, "bf16")
    c.keep[1, 1] = 0
    full, lse = OA.block_attention(c.vals("q"), c.vals("k_ctx"), c.vals("v_ctx"),
                                   c.ctx_offsets, c.vals("k_blk"), c.vals("v_blk"),
                                   c.anchor, c.keep, 8, c.scale)
    picks = [(0, 0, 3), (1, 1, 0), (1, 2, 7)]
    got = OA.block_attention_rows(c.vals("q"), c.vals("k_ctx"), c.vals("v_ctx"),
                                  c.ctx_offsets, c.vals("k_blk"), c.vals("v_blk"),
                                  c.anchor, c.keep, 8, c.scale, picks)
    for (b, a, h), (o, l) in got.items():
        np.testing.assert_allclose(o, full[b, a * 8:(a + 1) * 8, h], atol=1e-12)
        np.testing.assert_allclose(l, lse[b, h, a * 8:(a + 1) * 8], atol=1e-12)
