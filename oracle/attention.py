"""Block-masked dual-source attention — oracle.

Test infrastructure only (see ``oracle/__init__``).

What is computed (page 1, "03 · DSpark 建模", §3.4 block attention mask and
§3.5 custom attention; page 4, "DSpark 深度解读", §3.2 parallel backbone):

* Queries come only from the draft blocks (anchor + gamma-1 mask embeddings).
* Keys/values are the concatenation, along the sequence axis, of the context
  projections (from the target's hidden states) and the draft blocks' own
  projections.
* Mask rules: (1) standard causal attention inside the context; (2) a draft
  block sees only the context strictly before its anchor plus the keys of its
  own block; (3) a block whose keep flag is 0 is fully masked.

Readings taken where the pages are silent (all listed in the design doc):

* "before its anchor" is strict: context key j is visible iff j < anchor;
* keys inside one block are visible to every query of that block
  (bidirectional inside the block);
* a fully masked query row outputs zeros, and its log-sum-exp is -inf;
* query head h uses key/value head h // (Hq // Hkv) (contiguous grouping);
* logits are scale * <q, k>, with scale an argument (1/sqrt(D) by default).

Shapes (row-major, the same as the C-ABI):
  q            [B, A*gamma, Hq, D]
  k_ctx, v_ctx [sum_b S_b, Hkv, D], request b owns rows ctx_offsets[b]..ctx_offsets[b+1]
  k_blk, v_blk [B, A*gamma, Hkv, D]
  anchor       [B, A] int, keep [B, A] (nonzero = kept)
  out          [B, A*gamma, Hq, D], lse [B, Hq, A*gamma]
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def block_attention(q, k_ctx, v_ctx, ctx_offsets, k_blk, v_blk, anchor, keep,
                    gamma, scale):
    """Set definition: for block (b, a) the visible keys are context rows
    [0, anchor[b,a]) of request b followed by the gamma own-block rows; softmax
    over them in float64 (max-subtracted), weighted sum of the values."""
    q, k_ctx, v_ctx, k_blk, v_blk = map(_f64, (q, k_ctx, v_ctx, k_blk, v_blk))
    anchor = np.asarray(anchor)
    keep = np.asarray(keep)
    B, AG, Hq, D = q.shape
    A = anchor.shape[1]
    assert AG == A * gamma
    Hkv = k_ctx.shape[1]
    group = Hq // Hkv
    out = np.zeros((B, AG, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq, AG), -np.inf, dtype=np.float64)
    for b in range(B):
        c0 = int(ctx_offsets[b])
        for a in range(A):
            if not keep[b, a]:
                continue  # rule (3): the whole block is masked
            p = int(anchor[b, a])
            rows = slice(a * gamma, (a + 1) * gamma)
            keys = np.concatenate([k_ctx[c0:c0 + p], k_blk[b, rows]], axis=0)
            vals = np.concatenate([v_ctx[c0:c0 + p], v_blk[b, rows]], axis=0)
            for h in range(Hq):
                kvh = h // group
                s = scale * (q[b, rows, h, :] @ keys[:, kvh, :].T)  # [gamma, p+gamma]
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(axis=1, keepdims=True)
                out[b, rows, h, :] = (e @ vals[:, kvh, :]) / l
                lse[b, h, rows] = (m + np.log(l))[:, 0]
    return out, lse


def mask_mod(q_idx, kv_idx, S, gamma, anchor_b, keep_b):
    """The visibility predicate over the conceptual sequence of one request:
    positions [0, S) are the context, position S + a*gamma + k is row k of
    draft block a.  Returns True where query q_idx may attend to kv_idx."""
    if q_idx < S:                         # a context position
        return kv_idx < S and kv_idx <= q_idx          # rule (1): causal
    a_q = (q_idx - S) // gamma
    if not keep_b[a_q]:                   # rule (3): masked block
        return False
    if kv_idx < S:                        # rule (2a): context before the anchor
        return kv_idx < anchor_b[a_q]
    return (kv_idx - S) // gamma == a_q   # rule (2b): own block only


def full_mask(S, gamma, anchor_b, keep_b):
    """Materialise the whole [S + A*gamma, S + A*gamma] boolean mask by
    evaluating the predicate position by position."""
    A = len(anchor_b)
    n = S + A * gamma
    M = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for j in range(n):
            M[i, j] = mask_mod(i, j, S, gamma, anchor_b, keep_b)
    return M


def block_attention_dense(q, k_ctx, v_ctx, ctx_offsets, k_blk, v_blk, anchor,
                          keep, gamma, scale):
    """Brute force: per request, lay out the full conceptual key/value
    sequence (context followed by all draft blocks), build the full mask with
    ``full_mask`` and run a dense masked softmax for every draft query row.
    Only for tiny shapes (the mask is built element by element)."""
    q, k_ctx, v_ctx, k_blk, v_blk = map(_f64, (q, k_ctx, v_ctx, k_blk, v_blk))
    anchor = np.asarray(anchor)
    keep = np.asarray(keep)
    B, AG, Hq, D = q.shape
    Hkv = k_ctx.shape[1]
    group = Hq // Hkv
    out = np.zeros((B, AG, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq, AG), -np.inf, dtype=np.float64)
    for b in range(B):
        c0, c1 = int(ctx_offsets[b]), int(ctx_offsets[b + 1])
        S = c1 - c0
        K = np.concatenate([k_ctx[c0:c1], k_blk[b]], axis=0)  # [S + A*gamma, Hkv, D]
        Vv = np.concatenate([v_ctx[c0:c1], v_blk[b]], axis=0)
        M = full_mask(S, gamma, anchor[b], keep[b])
        for i in range(AG):
            vis = M[S + i]
            if not vis.any():
                continue
            for h in range(Hq):
                kvh = h // group
                s = scale * (K[:, kvh, :] @ q[b, i, h, :])
                s = np.where(vis, s, -np.inf)
                m = s.max()
                e = np.where(vis, np.exp(s - m), 0.0)
                out[b, i, h, :] = (e @ Vv[:, kvh, :]) / e.sum()
                lse[b, h, i] = m + np.log(e.sum())
    return out, lse


def block_attention_rows(q, k_ctx, v_ctx, ctx_offsets, k_blk, v_blk, anchor,
                         keep, gamma, scale, picks):
    """The set definition evaluated only for selected outputs.

    picks: iterable of (b, a, h); returns {(b, a, h): (out [gamma, D],
    lse [gamma])}.  Used to check full-size launches one block at a time;
    the arrays may be any indexable (e.g. host copies of only what is read)."""
    res = {}
    Hq = q.shape[2]
    Hkv = k_ctx.shape[1]
    group = Hq // Hkv
    for (b, a, h) in picks:
        rows = slice(a * gamma, (a + 1) * gamma)
        D = q.shape[3]
        if not keep[b, a]:
            res[(b, a, h)] = (np.zeros((gamma, D)), np.full(gamma, -np.inf))
            continue
        c0 = int(ctx_offsets[b])
        p = int(anchor[b, a])
        kvh = h // group
        keys = np.concatenate([_f64(k_ctx[c0:c0 + p, kvh]), _f64(k_blk[b, rows, kvh])], 0)
        vals = np.concatenate([_f64(v_ctx[c0:c0 + p, kvh]), _f64(v_blk[b, rows, kvh])], 0)
        s = scale * (_f64(q[b, rows, h]) @ keys.T)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        res[(b, a, h)] = ((e @ vals) / l, (m + np.log(l))[:, 0])
    return res
