"""DSpark draft-round hot path on MI355X: Python binding of libdspark.so.

Each function marshals torch tensors (device memory, the current HIP stream)
into one call of the C ABI declared in include/dspark.h and allocates the
outputs and workspace it needs through torch's allocator.  All arithmetic
runs in the library's HIP kernels; if the library is missing the import
fails.

Functions (same names and argument meaning as the C entry points; each
``*_workspace_bytes`` mirrors the C size query):

* ``block_attention``  — block-masked dual-source attention
* ``markov_sample``    — Markov-head gamma-step sampler
* ``markov_sample_noalloc`` — the same through the allocation-free entry point
* ``accept_rate``      — TV accept rate (+ tau); ``set_wait_limit``
* ``eval_mask``        — cumulative-product eval mask
* ``markov_block_logits`` — teacher-forced Markov logits of a whole block
* ``markov_head_sample`` / ``markov_head_block_logits`` — the same for the
  gated and recurrent heads
* ``l1_loss``          — L1 (TV) alignment loss, its gradient, tau_greedy
* ``confidence_schedule`` — confidence head, prefix survival, verify length
* ``verify``           — lossless verify (rejection sampling) of drafted blocks
"""

from __future__ import annotations

import math

import torch

from . import _lib

_LIB = _lib.load()

__all__ = ["block_attention", "block_attention_workspace_bytes",
           "markov_sample", "markov_sample_noalloc", "markov_sample_workspace_bytes",
           "accept_rate", "accept_rate_workspace_bytes", "set_wait_limit",
           "eval_mask",
           "markov_block_logits", "markov_block_logits_workspace_bytes",
           "markov_head_sample", "markov_head_sample_workspace_bytes",
           "markov_head_block_logits", "markov_head_block_logits_workspace_bytes",
           "l1_loss", "l1_loss_workspace_bytes",
           "confidence_schedule",
           "verify", "verify_workspace_bytes",
           "last_error", "version", "DSparkError"]


class DSparkError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = _LIB.dspark_last_error().decode(errors="replace")
        super().__init__(f"{where}: status {code}: {msg}")
        self.code = code


def last_error() -> str:
    return _LIB.dspark_last_error().decode(errors="replace")


def version() -> int:
    return int(_LIB.dspark_version())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(t, name, dtype=None, device=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _dt(t):
    if t.dtype == torch.bfloat16:
        return _lib.BF16
    if t.dtype == torch.float32:
        return _lib.F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def block_attention_workspace_bytes(B, A, gamma, Hq, Hkv, D, max_ctx) -> int:
    return int(_LIB.dspark_block_attention_workspace_bytes(B, A, gamma, Hq, Hkv, D, max_ctx))


def block_attention(q, k_ctx, v_ctx, ctx_offsets, k_blk, v_blk, anchor, keep, *, max_ctx,
                    scale=None, out=None, lse=None, want_lse=False, status=None,
                    workspace=None):
    """q [B, A*gamma, Hq, D]; k_ctx/v_ctx [T, Hkv, D]; ctx_offsets [B+1] int32;
    k_blk/v_blk [B, A*gamma, Hkv, D]; anchor [B, A] int32; keep [B, A] uint8.
    Returns (out [B, A*gamma, Hq, D], lse [B, Hq, A*gamma] or None)."""
    dev = q.device
    _check(q, "q", (torch.bfloat16, torch.float32), ndim=4)
    B, AG, Hq, D = q.shape
    A = anchor.shape[1]
    if A == 0 or AG % A:
        raise ValueError("q rows must be A * gamma")
    gamma = AG // A
    for name, t in (("k_ctx", k_ctx), ("v_ctx", v_ctx)):
        _check(t, name, q.dtype, dev, 3)
    Hkv = k_ctx.shape[1]
    for name, t in (("k_blk", k_blk), ("v_blk", v_blk)):
        _check(t, name, q.dtype, dev, 4)
        if tuple(t.shape) != (B, AG, Hkv, D):
            raise ValueError(f"{name} shape {tuple(t.shape)} != {(B, AG, Hkv, D)}")
    if tuple(k_ctx.shape[1:]) != (Hkv, D) or v_ctx.shape != k_ctx.shape:
        raise ValueError("k_ctx / v_ctx must be [T, Hkv, D]")
    _check(ctx_offsets, "ctx_offsets", torch.int32, dev, 1)
    _check(anchor, "anchor", torch.int32, dev, 2)
    _check(keep, "keep", torch.uint8, dev, 2)
    if ctx_offsets.shape[0] != B + 1 or tuple(anchor.shape) != (B, A) or tuple(keep.shape) != (B, A):
        raise ValueError("ctx_offsets / anchor / keep shapes do not match q")
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", q.dtype, dev, 4)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, AG), dtype=torch.float32, device=dev)
    if lse is not None:
        _check(lse, "lse", torch.float32, dev, 3)
    if status is not None:
        _check(status, "status", torch.int32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    nbytes = block_attention_workspace_bytes(B, A, gamma, Hq, Hkv, D, max_ctx)
    ws, wsb = _workspace(nbytes, dev, workspace)
    rc = _LIB.dspark_block_attention(
        _ptr(q), _ptr(k_ctx), _ptr(v_ctx), _ptr(ctx_offsets), _ptr(k_blk), _ptr(v_blk),
        _ptr(anchor), _ptr(keep), _ptr(out), _ptr(lse), B, A, gamma, Hq, Hkv, D, int(max_ctx),
        int(k_ctx.shape[0]), float(scale), _dt(q), _ptr(ws), wsb, _ptr(status), _stream(dev))
    if rc != 0:
        raise DSparkError(rc, "block_attention")
    return out, lse


def markov_sample_workspace_bytes(R, gamma, V, r, wdtype=_lib.BF16) -> int:
    return int(_LIB.dspark_markov_sample_workspace_bytes(R, gamma, V, r, wdtype))


def _markov_sample_args(base, w1, w2, first_prev, tokens, step_logits, want_step_logits, status):
    dev = base.device
    _check(base, "base", torch.float32, ndim=3)
    R, gamma, V = base.shape
    _check(w1, "w1", (torch.bfloat16, torch.float32), dev, 2)
    _check(w2, "w2", w1.dtype, dev, 2)
    r = w1.shape[1]
    if tuple(w1.shape) != (V, r) or tuple(w2.shape) != (r, V):
        raise ValueError(f"w1 must be [V, r] and w2 [r, V]; got {tuple(w1.shape)}, {tuple(w2.shape)}")
    _check(first_prev, "first_prev", torch.int32, dev, 1)
    if first_prev.shape[0] != R:
        raise ValueError("first_prev must have R entries")
    if tokens is None:
        tokens = torch.empty((R, gamma), dtype=torch.int32, device=dev)
    _check(tokens, "tokens", torch.int32, dev, 2)
    if step_logits is None and want_step_logits:
        step_logits = torch.empty_like(base)
    if step_logits is not None:
        _check(step_logits, "step_logits", torch.float32, dev, 3)
    if status is not None:
        _check(status, "status", torch.int32, dev)
    return dev, R, gamma, V, r, _dt(w1), tokens, step_logits


def markov_sample(base, w1, w2, first_prev, *, temperature=0.0, seed=0, tokens=None,
                  step_logits=None, want_step_logits=False, status=None, workspace=None):
    """base [R, gamma, V] float32; w1 [V, r]; w2 [r, V] (same dtype, bf16 or
    float32); first_prev [R] int32.  Returns (tokens [R, gamma] int32,
    step_logits [R, gamma, V] float32 or None)."""
    dev, R, gamma, V, r, wdt, tokens, step_logits = _markov_sample_args(
        base, w1, w2, first_prev, tokens, step_logits, want_step_logits, status)
    nbytes = markov_sample_workspace_bytes(R, gamma, V, r, wdt)
    ws, wsb = _workspace(nbytes, dev, workspace)
    rc = _LIB.dspark_markov_sample(
        _ptr(base), _ptr(w1), _ptr(w2), _ptr(first_prev), _ptr(tokens), _ptr(step_logits),
        R, gamma, V, r, wdt, float(temperature), int(seed) & (2**64 - 1), _ptr(ws), wsb,
        _ptr(status), _stream(dev))
    if rc != 0:
        raise DSparkError(rc, "markov_sample")
    return tokens, step_logits


def markov_sample_noalloc(base, w1, w2, first_prev, *, temperature=0.0, seed=0, tokens=None,
                          step_logits=None, want_step_logits=False, status=None):
    """markov_sample through the library's allocation-free entry point: no
    workspace (the per-step keys live in the library's fixed device array,
    shared by every call on the GPU: calls must not overlap).  Pass `tokens`
    (and `step_logits`) to keep this wrapper from allocating them."""
    dev, R, gamma, V, r, wdt, tokens, step_logits = _markov_sample_args(
        base, w1, w2, first_prev, tokens, step_logits, want_step_logits, status)
    rc = _LIB.dspark_markov_sample_noalloc(
        _ptr(base), _ptr(w1), _ptr(w2), _ptr(first_prev), _ptr(tokens), _ptr(step_logits),
        R, gamma, V, r, wdt, float(temperature), int(seed) & (2**64 - 1), _ptr(status), _stream(dev))
    if rc != 0:
        raise DSparkError(rc, "markov_sample_noalloc")
    return tokens, step_logits


def accept_rate_workspace_bytes(B, A, gamma, V, dtype=_lib.BF16) -> int:
    return int(_LIB.dspark_accept_rate_workspace_bytes(B, A, gamma, V, dtype))


def accept_rate(draft, target, *, eval_mask=None, want_tau=False, accept=None, tau=None,
                status=None, workspace=None):
    """draft, target [B, A, gamma, V] (bf16 or float32); eval_mask [B, A, gamma]
    uint8 (optional, used for tau); status: int32 device word that receives
    STATUS_WAIT_TIMEOUT (optional).  Returns (accept [B, A, gamma] float32,
    tau [B, A] float32 or None)."""
    dev = draft.device
    _check(draft, "draft", (torch.bfloat16, torch.float32), ndim=4)
    _check(target, "target", draft.dtype, dev, 4)
    if target.shape != draft.shape:
        raise ValueError("draft and target shapes differ")
    B, A, gamma, V = draft.shape
    if accept is None:
        accept = torch.empty((B, A, gamma), dtype=torch.float32, device=dev)
    _check(accept, "accept", torch.float32, dev, 3)
    if eval_mask is not None:
        _check(eval_mask, "eval_mask", torch.uint8, dev, 3)
    if tau is None and want_tau:
        tau = torch.empty((B, A), dtype=torch.float32, device=dev)
    if tau is not None:
        _check(tau, "tau", torch.float32, dev, 2)
    if status is not None:
        _check(status, "status", torch.int32, dev)
    dt = _dt(draft)
    nbytes = accept_rate_workspace_bytes(B, A, gamma, V, dt)
    ws, wsb = _workspace(nbytes, dev, workspace)
    rc = _LIB.dspark_accept_rate(_ptr(draft), _ptr(target), _ptr(accept), _ptr(eval_mask),
                                 _ptr(tau), B, A, gamma, V, dt, _ptr(ws), wsb, _ptr(status),
                                 _stream(dev))
    if rc != 0:
        raise DSparkError(rc, "accept_rate")
    return accept, tau


def markov_block_logits_workspace_bytes(N, V, r, wdtype=_lib.BF16) -> int:
    return int(_LIB.dspark_markov_block_logits_workspace_bytes(N, V, r, wdtype))


def markov_block_logits(base, w1, w2, prev, *, softcap=0.0, logits=None, want_tokens=False, tokens=None,
                        status=None, workspace=None):
    """Teacher-forced Markov logits.  base [N, V] float32; w1 [V, r]; w2 [r, V]
    (bf16 or float32); prev [N] int32.  Returns (logits [N, V] float32,
    argmax tokens [N] int32 or None)."""
    dev = base.device
    _check(base, "base", torch.float32, ndim=2)
    N, V = base.shape
    _check(w1, "w1", (torch.bfloat16, torch.float32), dev, 2)
    _check(w2, "w2", w1.dtype, dev, 2)
    r = w1.shape[1]
    if tuple(w1.shape) != (V, r) or tuple(w2.shape) != (r, V):
        raise ValueError(f"w1 must be [V, r] and w2 [r, V]; got {tuple(w1.shape)}, {tuple(w2.shape)}")
    _check(prev, "prev", torch.int32, dev, 1)
    if prev.shape[0] != N:
        raise ValueError("prev must have N entries")
    if logits is None:
        logits = torch.empty_like(base)
    _check(logits, "logits", torch.float32, dev, 2)
    if tokens is None and want_tokens:
        tokens = torch.empty((N,), dtype=torch.int32, device=dev)
    if tokens is not None:
        _check(tokens, "tokens", torch.int32, dev, 1)
    if status is not None:
        _check(status, "status", torch.int32, dev)
    wdt = _dt(w1)
    ws, wsb = _workspace(markov_block_logits_workspace_bytes(N, V, r, wdt), dev, workspace)
    rc = _LIB.dspark_markov_block_logits(_ptr(base), _ptr(w1), _ptr(w2), _ptr(prev), _ptr(logits), _ptr(tokens),
                                         N, V, r, wdt, float(softcap), _ptr(ws), wsb, _ptr(status), _stream(dev))
    if rc != 0:
        raise DSparkError(rc, "markov_block_logits")
    return logits, tokens


_HEAD_KINDS = {"gated": _lib.HEAD_GATED, "rnn": _lib.HEAD_RNN}


def _head_kind(kind):
    if kind not in _HEAD_KINDS:
        raise ValueError(f"head kind must be one of {sorted(_HEAD_KINDS)}; got {kind!r}")
    return _HEAD_KINDS[kind]


def _check_head(kind, base, hidden, w1, w2, whead):
    """Shapes of the gated / recurrent head inputs; returns (R, gamma, V, r, d)."""
    dev = base.device
    _check(base, "base", torch.float32, ndim=3)
    R, gamma, V = base.shape
    _check(hidden, "hidden", torch.bfloat16, dev, 3)
    if tuple(hidden.shape[:2]) != (R, gamma):
        raise ValueError("hidden must be [R, gamma, d] matching base")
    d = hidden.shape[2]
    _check(w1, "w1", (torch.bfloat16, torch.float32), dev, 2)
    _check(w2, "w2", w1.dtype, dev, 2)
    r = w1.shape[1]
    if tuple(w1.shape) != (V, r) or tuple(w2.shape) != (r, V):
        raise ValueError(f"w1 must be [V, r] and w2 [r, V]; got {tuple(w1.shape)}, {tuple(w2.shape)}")
    want = (r, d + r) if kind == "gated" else (3, r, 2 * r + d)
    _check(whead, "whead", torch.bfloat16, dev)
    if tuple(whead.shape) != want:
        raise ValueError(f"{kind} head weights must be {want}; got {tuple(whead.shape)}")
    return R, gamma, V, r, d


def markov_head_sample_workspace_bytes(kind, R, gamma, V, r) -> int:
    return int(_LIB.dspark_markov_head_sample_workspace_bytes(_head_kind(kind), R, gamma, V, r))


def markov_head_sample(kind, base, hidden, w1, w2, whead, first_prev, *, temperature=0.0, seed=0, tokens=None,
                       step_logits=None, want_step_logits=False, status=None, workspace=None):
    """Gated ("gated") or recurrent ("rnn") Markov-head sampler.  base
    [R, gamma, V] float32; hidden [R, gamma, d] bf16; w1 [V, r], w2 [r, V];
    whead [r, d + r] (gated) or [3, r, 2r + d] (rnn) bf16; first_prev [R]
    int32.  Returns (tokens [R, gamma] int32, step_logits or None)."""
    k = _head_kind(kind)
    R, gamma, V, r, d = _check_head(kind, base, hidden, w1, w2, whead)
    dev = base.device
    _check(first_prev, "first_prev", torch.int32, dev, 1)
    if first_prev.shape[0] != R:
        raise ValueError("first_prev must have R entries")
    if tokens is None:
        tokens = torch.empty((R, gamma), dtype=torch.int32, device=dev)
    _check(tokens, "tokens", torch.int32, dev, 2)
    if step_logits is None and want_step_logits:
        step_logits = torch.empty_like(base)
    if step_logits is not None:
        _check(step_logits, "step_logits", torch.float32, dev, 3)
    if status is not None:
        _check(status, "status", torch.int32, dev)
    ws, wsb = _workspace(markov_head_sample_workspace_bytes(kind, R, gamma, V, r), dev, workspace)
    rc = _LIB.dspark_markov_head_sample(
        k, _ptr(base), _ptr(hidden), _ptr(w1), _ptr(w2), _ptr(whead), _ptr(first_prev), _ptr(tokens),
        _ptr(step_logits), R, gamma, V, r, d, _dt(w1), float(temperature), int(seed) & (2**64 - 1), _ptr(ws), wsb,
        _ptr(status), _stream(dev))
    if rc != 0:
        raise DSparkError(rc, "markov_head_sample")
    return tokens, step_logits


def markov_head_block_logits_workspace_bytes(kind, B, gamma, V, r) -> int:
    return int(_LIB.dspark_markov_head_block_logits_workspace_bytes(_head_kind(kind), B, gamma, V, r))


def markov_head_block_logits(kind, base, hidden, w1, w2, whead, prev, *, softcap=0.0, logits=None,
                             want_tokens=False, tokens=None, status=None, workspace=None):
    """Teacher-forced gated / recurrent head logits of B blocks.  base
    [B, gamma, V] float32; hidden [B, gamma, d] bf16; prev [B, gamma] int32
    (x_{k-1} of position k).  Returns (logits [B, gamma, V] float32, argmax
    tokens [B, gamma] int32 or None)."""
    k = _head_kind(kind)
    B, gamma, V, r, d = _check_head(kind, base, hidden, w1, w2, whead)
    dev = base.device
    _check(prev, "prev", torch.int32, dev, 2)
    if tuple(prev.shape) != (B, gamma):
        raise ValueError("prev must be [B, gamma]")
    if logits is None:
        logits = torch.empty_like(base)
    _check(logits, "logits", torch.float32, dev, 3)
    if tokens is None and want_tokens:
        tokens = torch.empty((B, gamma), dtype=torch.int32, device=dev)
    if tokens is not None:
        _check(tokens, "tokens", torch.int32, dev, 2)
    if status is not None:
        _check(status, "status", torch.int32, dev)
    ws, wsb = _workspace(markov_head_block_logits_workspace_bytes(kind, B, gamma, V, r), dev, workspace)
    rc = _LIB.dspark_markov_head_block_logits(
        k, _ptr(base), _ptr(hidden), _ptr(w1), _ptr(w2), _ptr(whead), _ptr(prev), _ptr(logits), _ptr(tokens), B,
        gamma, V, r, d, _dt(w1), float(softcap), _ptr(ws), wsb, _ptr(status), _stream(dev))
    if rc != 0:
        raise DSparkError(rc, "markov_head_block_logits")
    return logits, tokens


def verify_workspace_bytes(R, K) -> int:
    return int(_LIB.dspark_verify_workspace_bytes(R, K))


def verify(draft_logits, target_logits, draft_tokens, *, temperature=1.0, seed=0, n_accepted=None,
           next_token=None, status=None, workspace=None):
    """Lossless verify of R drafted blocks.  draft_logits [R, K, V] float32;
    target_logits [R, K + 1, V] float32; draft_tokens [R, K] int32.  Returns
    (n_accepted [R] int32, next_token [R] int32)."""
    dev = target_logits.device
    _check(target_logits, "target_logits", torch.float32, ndim=3)
    R, K1, V = target_logits.shape
    K = K1 - 1
    _check(draft_logits, "draft_logits", torch.float32, dev, 3)
    _check(draft_tokens, "draft_tokens", torch.int32, dev, 2)
    if tuple(draft_logits.shape) != (R, K, V) or tuple(draft_tokens.shape) != (R, K):
        raise ValueError("draft_logits must be [R, K, V] and draft_tokens [R, K] for target_logits [R, K + 1, V]")
    if n_accepted is None:
        n_accepted = torch.empty((R,), dtype=torch.int32, device=dev)
    if next_token is None:
        next_token = torch.empty((R,), dtype=torch.int32, device=dev)
    _check(n_accepted, "n_accepted", torch.int32, dev, 1)
    _check(next_token, "next_token", torch.int32, dev, 1)
    if status is not None:
        _check(status, "status", torch.int32, dev)
    ws, wsb = _workspace(verify_workspace_bytes(R, K), dev, workspace)
    rc = _LIB.dspark_verify(_ptr(draft_logits), _ptr(target_logits), _ptr(draft_tokens), _ptr(n_accepted),
                            _ptr(next_token), R, K, V, float(temperature), int(seed) & (2**64 - 1), _ptr(ws), wsb,
                            _ptr(status), _stream(dev))
    if rc != 0:
        raise DSparkError(rc, "verify")
    return n_accepted, next_token


def l1_loss_workspace_bytes(B, A, gamma, V, dtype=_lib.BF16) -> int:
    return int(_LIB.dspark_l1_loss_workspace_bytes(B, A, gamma, V, dtype))


def l1_loss(draft, target, *, eval_mask=None, decay=4.0, want_grad=False, want_rows=False,
            want_tau_greedy=False, loss=None, grad=None, row_l1=None, tau_greedy=None, workspace=None):
    """L1 (TV) alignment loss.  draft, target [B, A, gamma, V] (bf16 or
    float32); eval_mask [B, A, gamma] uint8 (optional).  Returns (loss [1],
    grad [B, A, gamma, V] float32 or None, row_l1 [B, A, gamma] or None,
    tau_greedy [B, A] or None)."""
    dev = draft.device
    _check(draft, "draft", (torch.bfloat16, torch.float32), ndim=4)
    _check(target, "target", draft.dtype, dev, 4)
    if target.shape != draft.shape:
        raise ValueError("draft and target shapes differ")
    B, A, gamma, V = draft.shape
    if eval_mask is not None:
        _check(eval_mask, "eval_mask", torch.uint8, dev, 3)
    if loss is None:
        loss = torch.empty((1,), dtype=torch.float32, device=dev)
    _check(loss, "loss", torch.float32, dev, 1)
    if grad is None and want_grad:
        grad = torch.empty((B, A, gamma, V), dtype=torch.float32, device=dev)
    if grad is not None:
        _check(grad, "grad", torch.float32, dev, 4)
    if row_l1 is None and want_rows:
        row_l1 = torch.empty((B, A, gamma), dtype=torch.float32, device=dev)
    if row_l1 is not None:
        _check(row_l1, "row_l1", torch.float32, dev, 3)
    if tau_greedy is None and want_tau_greedy:
        tau_greedy = torch.empty((B, A), dtype=torch.float32, device=dev)
    if tau_greedy is not None:
        _check(tau_greedy, "tau_greedy", torch.float32, dev, 2)
    ws, wsb = _workspace(l1_loss_workspace_bytes(B, A, gamma, V, _dt(draft)), dev, workspace)
    rc = _LIB.dspark_l1_loss(_ptr(draft), _ptr(target), _ptr(eval_mask), float(decay), _ptr(loss), _ptr(row_l1),
                             _ptr(grad), _ptr(tau_greedy), B, A, gamma, V, _dt(draft), _ptr(ws), wsb, _stream(dev))
    if rc != 0:
        raise DSparkError(rc, "l1_loss")
    return loss, grad, row_l1, tau_greedy


def confidence_schedule(hidden, weight_h, bias, sps, *, w1=None, prev=None, weight_e=None, want_confidence=True,
                        want_survival=True, want_theta=False, status=None):
    """hidden [B, A, gamma, H] (bf16 or float32); weight_h [H] float32; bias
    float; sps [gamma + 1] float32; optional Markov input w1 [V, r], prev
    [B, A, gamma] int32, weight_e [r] float32.  Returns (verify_len [B, A]
    int32, confidence, survival [B, A, gamma] float32 or None, theta
    [B, A, gamma + 1] or None)."""
    dev = hidden.device
    _check(hidden, "hidden", (torch.bfloat16, torch.float32), ndim=4)
    B, A, gamma, H = hidden.shape
    _check(weight_h, "weight_h", torch.float32, dev, 1)
    _check(sps, "sps", torch.float32, dev, 1)
    if weight_h.shape[0] != H or sps.shape[0] != gamma + 1:
        raise ValueError("weight_h must have H entries and sps gamma + 1")
    r = V = 0
    wdt = _lib.BF16
    if weight_e is not None:
        _check(weight_e, "weight_e", torch.float32, dev, 1)
        _check(w1, "w1", (torch.bfloat16, torch.float32), dev, 2)
        _check(prev, "prev", torch.int32, dev, 3)
        V, r = w1.shape
        if weight_e.shape[0] != r or tuple(prev.shape) != (B, A, gamma):
            raise ValueError("weight_e must have r entries and prev be [B, A, gamma]")
        wdt = _dt(w1)
    conf = torch.empty((B, A, gamma), dtype=torch.float32, device=dev) if want_confidence else None
    surv = torch.empty((B, A, gamma), dtype=torch.float32, device=dev) if want_survival else None
    theta = torch.empty((B, A, gamma + 1), dtype=torch.float32, device=dev) if want_theta else None
    vlen = torch.empty((B, A), dtype=torch.int32, device=dev)
    if status is not None:
        _check(status, "status", torch.int32, dev)
    rc = _LIB.dspark_confidence_schedule(_ptr(hidden), _dt(hidden), _ptr(weight_h), float(bias), _ptr(w1), wdt,
                                         _ptr(prev), _ptr(weight_e), r, V, _ptr(sps), _ptr(conf), _ptr(surv),
                                         _ptr(vlen), _ptr(theta), B, A, gamma, H, _ptr(status), _stream(dev))
    if rc != 0:
        raise DSparkError(rc, "confidence_schedule")
    return vlen, conf, surv, theta


def set_wait_limit(polls: int) -> None:
    """Poll limit of the cooperative grids' bounded waits (0 = the default).
    Process-wide; meant for tests of the timeout path."""
    _LIB.dspark_set_wait_limit(int(polls))


def eval_mask(anchor, keep, seq_lens, loss_mask=None, *, gamma, out=None, status=None):
    """anchor [B, A] int32; keep [B, A] uint8; seq_lens [B] int32; loss_mask
    [B, S_stride] uint8 or None.  Returns uint8 [B, A, gamma]."""
    dev = anchor.device
    _check(anchor, "anchor", torch.int32, ndim=2)
    B, A = anchor.shape
    _check(keep, "keep", torch.uint8, dev, 2)
    _check(seq_lens, "seq_lens", torch.int32, dev, 1)
    if tuple(keep.shape) != (B, A) or seq_lens.shape[0] != B:
        raise ValueError("keep / seq_lens shapes do not match anchor")
    S_stride = 0
    if loss_mask is not None:
        _check(loss_mask, "loss_mask", torch.uint8, dev, 2)
        if loss_mask.shape[0] != B:
            raise ValueError("loss_mask must have B rows")
        S_stride = loss_mask.shape[1]
    if out is None:
        out = torch.empty((B, A, gamma), dtype=torch.uint8, device=dev)
    _check(out, "out", torch.uint8, dev, 3)
    if status is not None:
        _check(status, "status", torch.int32, dev)
    rc = _LIB.dspark_eval_mask(_ptr(anchor), _ptr(keep), _ptr(seq_lens), _ptr(loss_mask),
                               _ptr(out), B, A, gamma, S_stride, _ptr(status), _stream(dev))
    if rc != 0:
        raise DSparkError(rc, "eval_mask")
    return out
