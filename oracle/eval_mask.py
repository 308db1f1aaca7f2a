"""Cumulative-product eval mask — oracle.

Test infrastructure only (see ``oracle/__init__``).

What is computed (page 1 §3.1 and §3.6): three per-position conditions are
ANDed and then a cumulative product runs along the block, so once a position
is invalid every later position of the block is zero — only the contiguous
valid prefix counts, as in speculative decoding's longest accepted prefix.

The pages do not list the three conditions.  Reading taken (the design doc lists
it): for block (b, a) and block position k, the predicted token's index is
L = anchor[b, a] + 1 + k (position 0 is the anchor itself and predicts the
next token, page 1 §3.3 and §3.11), and the position is valid iff

1. the block is kept (keep[b, a] != 0) and its anchor is non-negative,
2. the label index is inside the sequence: L < seq_lens[b],
3. the label is a supervised position: loss_mask[b, L] != 0 (when a loss
   mask is given; with none, condition 3 always holds).

Output is 0/1 (uint8).
"""

from __future__ import annotations

import numpy as np


def position_valid(anchor, keep, seq_len, loss_mask_row, k):
    """The three conditions for one block position (plain Python)."""
    if not keep or anchor < 0:
        return False
    L = anchor + 1 + k
    if L >= seq_len:
        return False
    if loss_mask_row is not None:
        if L >= len(loss_mask_row) or not loss_mask_row[L]:
            return False
    return True


def eval_mask(anchor, keep, seq_lens, loss_mask, gamma):
    """anchor, keep [B, A]; seq_lens [B]; loss_mask [B, S_stride] or None.
    Returns uint8 [B, A, gamma]."""
    anchor = np.asarray(anchor)
    keep = np.asarray(keep)
    seq_lens = np.asarray(seq_lens)
    B, A = anchor.shape
    out = np.zeros((B, A, gamma), dtype=np.uint8)
    for b in range(B):
        lm = None if loss_mask is None else np.asarray(loss_mask[b])
        for a in range(A):
            running = 1
            for k in range(gamma):
                v = position_valid(int(anchor[b, a]), bool(keep[b, a]),
                                   int(seq_lens[b]), lm, k)
                running = running * int(v)  # the cumulative product along the block
                out[b, a, k] = running
    return out
