"""Block-masked dual-source attention on the GPU vs the oracle.

Outputs and log-sum-exps within 2e-2 absolute for bf16 inputs and 1e-4 for
float32 inputs.  Small cases span several 64-row tiles, ragged tails,
several 1024-key context chunks, both head dims and GQA groupings; the
full-size workloads are checked on sampled (block, head) outputs in the
launch configuration the bench times."""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DEV, as_dtype, dev, host_bits
from oracle import attention as OA

pytestmark = pytest.mark.gpu
TOL = {"bf16": 2e-2, "f32": 1e-4}


@pytest.fixture(scope="module")
def dsp():
    import semi_autoregressive_block_amd as m
    return m


def _run(dsp, c, max_ctx=None, status=None, total_ctx=None):
    dt = c.dtype
    kc = as_dtype(c.k_ctx, dt)
    out, lse = dsp.block_attention(
        as_dtype(c.q, dt), kc, as_dtype(c.v_ctx, dt), dev(c.ctx_offsets), as_dtype(c.k_blk, dt),
        as_dtype(c.v_blk, dt), dev(c.anchor), dev(c.keep),
        max_ctx=int(np.diff(c.ctx_offsets).max(initial=0)) if max_ctx is None else max_ctx,
        scale=c.scale, want_lse=True, status=status)
    return out.float().cpu().numpy(), lse.cpu().numpy()


def _ref(c):
    return OA.block_attention(c.vals("q"), c.vals("k_ctx"), c.vals("v_ctx"), c.ctx_offsets,
                              c.vals("k_blk"), c.vals("v_blk"), c.anchor, c.keep, c.gamma, c.scale)


def _compare(got, ref, tol):
    o, l = got
    ro, rl = ref
    assert np.abs(o - ro).max() < tol, np.abs(o - ro).max()
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(l), fin)
    assert np.all(l[~fin] == -np.inf)
    assert np.abs(l[fin] - rl[fin]).max(initial=0) < tol


def test_config1_fp32(dsp):
    c, _, _ = W.config1()
    _compare(_run(dsp, c), _ref(c), TOL["f32"])


CASES = [
    # seed, ctx lens, A, gamma, Hq, Hkv, D
    (1, [300, 700], 5, 8, 8, 2, 128),
    (2, [0, 37, 2100], 3, 16, 4, 4, 64),
    (3, [1500], 7, 5, 6, 2, 128),       # group 3, gamma 5: tiles cut through blocks
    (4, [64, 3000, 1], 2, 16, 32, 8, 128),
    (5, [2500, 900], 20, 8, 8, 8, 64),
    (6, [4100], 3, 64, 2, 1, 128),      # gamma 64: own keys span two slabs
    (7, [3000, 260], 40, 8, 16, 4, 128),  # ten 128-row tiles per (request, KV head), four blocks each
    (8, [1800], 37, 8, 8, 2, 128),      # 128-row tiles over blocks of 32 rows, a ragged last tile (32 rows)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_bf16_cases(dsp, case):
    seed, ctx, A, g, Hq, Hkv, D = case
    c = W.attention_case(seed, ctx, A, g, Hq, Hkv, D, "bf16")
    if c.keep.size > 1:
        c.keep.flat[1] = 0
    _compare(_run(dsp, c), _ref(c), TOL["bf16"])


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 8, 2), (64, 4, 4)])
def test_streaming_tiles_long_contexts(dsp, D, Hq, Hkv):
    """Streaming tiles (one 16-position block per request) over contexts of
    130 to 8193 keys: odd numbers of 32-key slabs and of slab pairs, a long
    request with keep = 0, and anchors inside and at the end of the context."""
    ctx = [4096, 4097, 4200, 6001, 8193, 130, 7000, 5000]
    anchor = np.array([[4096], [4097], [4200], [3000], [8193], [130], [6999], [5000]], dtype=np.int32)
    keep = np.ones((len(ctx), 1), dtype=np.uint8)
    keep[7, 0] = 0
    c = W.attention_case(31 + D, ctx, 1, 16, Hq, Hkv, D, "bf16", anchor=anchor, keep=keep)
    _compare(_run(dsp, c), _ref(c), TOL["bf16"])


def test_fp32_vector_path_multichunk(dsp):
    c = W.attention_case(21, [1200, 50], 3, 8, 4, 2, 64, "f32")
    _compare(_run(dsp, c), _ref(c), TOL["f32"])


def test_anchor_extremes_and_masked_blocks(dsp):
    c = W.attention_case(31, [2048], 6, 16, 8, 2, 128, "bf16")
    c.anchor[0] = [0, 2048, 1024, 1023, 1, 2047]
    c.keep[0] = [1, 1, 0, 1, 1, 1]
    got = _run(dsp, c)
    _compare(got, _ref(c), TOL["bf16"])
    o, l = got
    assert np.all(o[0, 32:48] == 0) and np.all(np.isneginf(l[0, :, 32:48]))


def test_zero_query_one_hot_probe(dsp):
    """Q = 0 and V_j = e_j: each output row is 1/|vis| on exactly the visible
    set — the mask enumerated position by position through the kernel."""
    S, A, g, D = 40, 3, 8, 64
    c = W.attention_case(41, [S], A, g, 4, 2, D, "bf16")
    c.anchor[0] = [0, 17, 40]
    c.keep[0] = [1, 1, 1]
    c.q[:] = 0
    vctx = np.zeros((S, 2, D), np.float32)
    vctx[np.arange(S), :, np.arange(S)] = 1.0
    vblk = np.zeros((1, A * g, 2, D), np.float32)
    for j in range(A * g):
        vblk[0, j, :, S + (j % g)] = 1.0
    c.v_ctx, c.v_blk = W.to_bf16_bits(vctx), W.to_bf16_bits(vblk)
    o, _ = _run(dsp, c)
    for a in range(A):
        p = c.anchor[0, a]
        vis = np.zeros(D, bool)
        vis[:p] = True
        vis[S:S + g] = True
        rows = o[0, a * g:(a + 1) * g]
        assert np.all(rows[..., ~vis] == 0)
        assert np.abs(rows[..., vis] - 1.0 / (p + g)).max() < 4e-3


def test_bad_anchor_and_offsets_are_clamped_and_flagged(dsp):
    c = W.attention_case(51, [100, 60], 2, 8, 4, 2, 128, "bf16")
    c.anchor[0, 0] = 500     # beyond the context: clamped to 100
    c.anchor[1, 1] = -4      # clamped to 0
    c.keep[:] = 1
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = _run(dsp, c, status=st)
    assert int(st.item()) & 1
    c2 = W.AttentionCase(**{**c.__dict__})
    c2.anchor = c.anchor.copy()
    c2.anchor[0, 0], c2.anchor[1, 1] = 100, 0
    _compare(got, _ref(c2), TOL["bf16"])
    # offsets beyond the K/V allocation: reads are clamped into it and flagged
    st.zero_()
    bad = c.ctx_offsets.copy()
    bad[2] = 10_000
    out, _ = dsp.block_attention(as_dtype(c.q, "bf16"), as_dtype(c.k_ctx, "bf16"),
                                 as_dtype(c.v_ctx, "bf16"), dev(bad), as_dtype(c.k_blk, "bf16"),
                                 as_dtype(c.v_blk, "bf16"), dev(c2.anchor), dev(c.keep),
                                 max_ctx=100, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & 4


def _offset_view(a, dtype, shift):
    """The same values in a contiguous view whose data pointer sits `shift`
    elements past an allocation boundary (bf16: 2 bytes per element), so it
    is not 16-byte aligned."""
    t = as_dtype(a, dtype)
    buf = torch.empty(t.numel() + shift, dtype=t.dtype, device=DEV)
    v = buf[shift:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("which", ["all", "out", "k_ctx"])
def test_bf16_unaligned_views(dsp, which):
    """bf16 tensors that are not 16-byte aligned (e.g. views that start one
    element into an allocation) take the vector-ALU kernel; it must agree
    with the oracle like the matrix-core kernel."""
    c = W.attention_case(71, [700, 130], 3, 8, 8, 2, 128, "bf16")
    c.keep[1, 2] = 0
    names = ["q", "k_ctx", "v_ctx", "k_blk", "v_blk"]
    shift = {n: (1 if which in ("all", n) else 0) for n in names + ["out"]}
    ts = {n: _offset_view(getattr(c, n), "bf16", shift[n]) for n in names}
    assert which != "all" or all(ts[n].data_ptr() % 16 for n in names)
    out = _offset_view(np.zeros(c.q.shape, np.uint16), "bf16", shift["out"])
    o, lse = dsp.block_attention(ts["q"], ts["k_ctx"], ts["v_ctx"], dev(c.ctx_offsets), ts["k_blk"],
                                 ts["v_blk"], dev(c.anchor), dev(c.keep), max_ctx=700, out=out, want_lse=True)
    assert o.data_ptr() == out.data_ptr()
    _compare((o.float().cpu().numpy(), lse.cpu().numpy()), _ref(c), TOL["bf16"])


def test_deterministic(dsp):
    c = W.attention_case(61, [3000, 5000], 2, 16, 32, 8, 128, "bf16")
    args = (as_dtype(c.q, "bf16"), as_dtype(c.k_ctx, "bf16"), as_dtype(c.v_ctx, "bf16"),
            dev(c.ctx_offsets), as_dtype(c.k_blk, "bf16"), as_dtype(c.v_blk, "bf16"),
            dev(c.anchor), dev(c.keep))
    a = dsp.block_attention(*args, max_ctx=5000)[0]
    b = dsp.block_attention(*args, max_ctx=5000)[0]
    assert torch.equal(a, b)


def _sampled(dsp, inp, picks, gamma):
    out, lse = dsp.block_attention(inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"],
                                   inp["k_blk"], inp["v_blk"], inp["anchor"], inp["keep"],
                                   max_ctx=inp["max_ctx"], want_lse=True)
    torch.cuda.synchronize()
    offs = inp["ctx_offsets"].cpu().numpy()
    anchor, keep = inp["anchor"].cpu().numpy(), inp["keep"].cpu().numpy()
    f = lambda t: W.bf16_to_f32(host_bits(t))
    Hkv = inp["k_ctx"].shape[1]
    group = inp["q"].shape[2] // Hkv
    for (b, a, h) in picks:
        kvh = h // group
        c0, c1 = int(offs[b]), int(offs[b + 1])
        rows = slice(a * gamma, (a + 1) * gamma)
        q = f(inp["q"][b, rows, h])[None, :, None, :]
        kc = f(inp["k_ctx"][c0:c1, kvh])[:, None, :]
        vc = f(inp["v_ctx"][c0:c1, kvh])[:, None, :]
        kb = f(inp["k_blk"][b, rows, kvh])[None, :, None, :]
        vb = f(inp["v_blk"][b, rows, kvh])[None, :, None, :]
        ro, rl = OA.block_attention(q, kc, vc, np.array([0, c1 - c0]), kb, vb,
                                    anchor[b:b + 1, a:a + 1], keep[b:b + 1, a:a + 1], gamma,
                                    1.0 / np.sqrt(q.shape[-1]))
        go = out[b, rows, h].float().cpu().numpy()
        gl = lse[b, h, rows].cpu().numpy()
        assert np.abs(go - ro[0, :, 0]).max() < TOL["bf16"], (b, a, h)
        if keep[b, a]:
            assert np.abs(gl - rl[0, 0]).max() < TOL["bf16"], (b, a, h)
        else:
            assert np.all(go == 0) and np.all(np.isneginf(gl))


def test_config2_full_size_sampled(dsp):
    """The training-shaped launch the bench times: every query head of five
    anchors (the first, a middle one, the last kept, the first padded one and
    the one with the longest context; all heads of an anchor span its blocks'
    eight KV-head workgroups) plus 24 random (anchor, head) pairs."""
    inp = W.config2_device(torch, DEV)
    anchor, keep = inp["anchor"].cpu().numpy()[0], inp["keep"].cpu().numpy()[0]
    longest = int(np.argmax(np.where(keep != 0, anchor, -1)))
    rng = np.random.default_rng(7)
    picks = [(0, int(a), int(h)) for a, h in zip(rng.integers(0, 512, 24), rng.integers(0, 32, 24))]
    picks += [(0, a, h) for a in sorted({0, 255, 471, 472, longest}) for h in range(32)]
    _sampled(dsp, inp, picks, 8)


def test_config5_full_size_sampled(dsp):
    """384 of the 4096 (request, head) outputs: every query head of the 8
    requests with the longest contexts (all their workgroups) and one random
    head of every request, in the launch configuration the bench times."""
    inp = W.config5_device(torch, DEV)
    lens = np.diff(inp["ctx_offsets"].cpu().numpy())
    longest = np.argsort(lens, kind="stable")[-8:]
    rng = np.random.default_rng(8)
    picks = [(int(b), 0, h) for b in longest for h in range(32)]
    picks += [(b, 0, int(h)) for b, h in zip(range(128), rng.integers(0, 32, 128))]
    _sampled(dsp, inp, picks, 16)
