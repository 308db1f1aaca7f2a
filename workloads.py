"""Seeded synthetic inputs for the DSpark draft-round hot path.

This module only draws inputs; it holds none of the method's arithmetic.  It
is the one module that both the oracle-side tests and the device-side tests,
bench and smoke use, so that both sides consume the same bytes.

Conventions (the full recipe per workload is written out below and in
the design doc):

* Structural choices (anchor positions, keep flags, context lengths, prompt
  lengths, per-block noise levels, tokens) are drawn on the host with numpy's
  PCG64, ``numpy.random.default_rng(seed)``.
* Dense tensors of small cases are drawn on the host with the same generator
  as float32 normals; bf16 tensors are the float32 draw rounded to nearest
  even (``to_bf16_bits``).
* Dense tensors of the full-size workloads (gigabytes) are drawn on the GPU
  with ``torch.Generator(device).manual_seed(seed)`` float32 normals, scaled,
  then cast (round to nearest even) to bf16.  Tests copy back exactly the
  stored bytes they hand to the oracle.

bf16 tensors on the host are carried as uint16 bit patterns; ``bf16_to_f32``
gives their exact values.
"""

from __future__ import annotations

import dataclasses

import numpy as np

SEED_BASE = 1000  # workload c uses seed 1000 + c


# ----------------------------------------------------------------- bf16 bits
def to_bf16_bits(x):
    """float32 array -> uint16 bf16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_to_f32(bits):
    """uint16 bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(rng, shape, std, dtype):
    """float32 N(0, std^2) draw; returns float32 values or bf16 bits."""
    x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return to_bf16_bits(x) if dtype == "bf16" else x


def values(x, dtype):
    """Exact float32 values of a host array stored as `dtype`."""
    return bf16_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


# ------------------------------------------------------------ anchor helpers
def sample_anchors(rng, loss_mask_row, n_real, A):
    """Anchor sampling for one sequence (the harness's stand-in for the
    reference's anchor sampler): candidates are positions p with
    loss_mask[p] and loss_mask[p+1] set; draw up to `n_real` of them without
    replacement, sort ascending, pad to A slots with anchor 0 / keep 0."""
    lm = np.asarray(loss_mask_row, dtype=bool)
    cand = np.flatnonzero(lm[:-1] & lm[1:])
    n = min(n_real, len(cand))
    pick = np.sort(rng.choice(cand, size=n, replace=False))
    anchor = np.zeros(A, dtype=np.int32)
    keep = np.zeros(A, dtype=np.uint8)
    anchor[:n] = pick
    keep[:n] = 1
    return anchor, keep


@dataclasses.dataclass
class AttentionCase:
    """Host-side inputs of one block-attention call."""
    q: np.ndarray          # [B, A*gamma, Hq, D]  (uint16 bf16 bits or float32)
    k_ctx: np.ndarray      # [sum S_b, Hkv, D]
    v_ctx: np.ndarray
    ctx_offsets: np.ndarray  # [B+1] int32
    k_blk: np.ndarray      # [B, A*gamma, Hkv, D]
    v_blk: np.ndarray
    anchor: np.ndarray     # [B, A] int32
    keep: np.ndarray       # [B, A] uint8
    gamma: int
    scale: float
    dtype: str             # "f32" or "bf16"

    def vals(self, name):
        return values(getattr(self, name), self.dtype)


def attention_case(seed, ctx_lens, A, gamma, Hq, Hkv, D, dtype, anchor=None,
                   keep=None, std=1.0, scale=None):
    """Random block-attention inputs with i.i.d. N(0, std^2) Q/K/V.  Anchors
    default to sorted distinct positions in [0, S_b] (A of them, or fewer
    if the context is short; the rest padded keep=0)."""
    rng = np.random.default_rng(seed)
    B = len(ctx_lens)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    offsets = np.zeros(B + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(ctx_lens)
    T = int(offsets[-1])
    if anchor is None:
        anchor = np.zeros((B, A), dtype=np.int32)
        keep = np.zeros((B, A), dtype=np.uint8)
        for b in range(B):
            n = min(A, int(ctx_lens[b]) + 1)
            pick = np.sort(rng.choice(int(ctx_lens[b]) + 1, size=n, replace=False))
            anchor[b, :n] = pick
            keep[b, :n] = 1
    anchor = np.asarray(anchor, dtype=np.int32)
    keep = np.asarray(keep, dtype=np.uint8)
    return AttentionCase(
        q=normal(rng, (B, A * gamma, Hq, D), std, dtype),
        k_ctx=normal(rng, (T, Hkv, D), std, dtype),
        v_ctx=normal(rng, (T, Hkv, D), std, dtype),
        ctx_offsets=offsets,
        k_blk=normal(rng, (B, A * gamma, Hkv, D), std, dtype),
        v_blk=normal(rng, (B, A * gamma, Hkv, D), std, dtype),
        anchor=anchor, keep=keep, gamma=gamma,
        scale=float(1.0 / np.sqrt(D)) if scale is None else float(scale),
        dtype=dtype)


@dataclasses.dataclass
class MarkovCase:
    base: np.ndarray        # [R, gamma, V] float32
    w1: np.ndarray          # [V, r] (bf16 bits or float32)
    w2: np.ndarray          # [r, V]
    first_prev: np.ndarray  # [R] int32
    temperature: float
    seed: int
    wdtype: str

    def vals(self, name):
        return values(getattr(self, name), self.wdtype) if name in ("w1", "w2") \
            else getattr(self, name)


def markov_case(seed, R, gamma, V, r, wdtype, base_std, w1_std, w2_std,
                temperature=0.0, philox_seed=None, first_prev=None):
    rng = np.random.default_rng(seed)
    base = rng.standard_normal(size=(R, gamma, V), dtype=np.float32) * np.float32(base_std)
    w1 = normal(rng, (V, r), w1_std, wdtype)
    w2 = normal(rng, (r, V), w2_std, wdtype)
    if first_prev is None:
        first_prev = rng.integers(0, V, size=R, dtype=np.int32)
    return MarkovCase(base=base, w1=w1, w2=w2,
                      first_prev=np.asarray(first_prev, dtype=np.int32),
                      temperature=float(temperature),
                      seed=int(seed if philox_seed is None else philox_seed),
                      wdtype=wdtype)


@dataclasses.dataclass
class MaskCase:
    anchor: np.ndarray      # [B, A] int32
    keep: np.ndarray        # [B, A] uint8
    seq_lens: np.ndarray    # [B] int32
    loss_mask: np.ndarray   # [B, S_stride] uint8 or None
    gamma: int


# ------------------------------------------------------------- workload 1
def config1():
    """Tiny fp32 draft round.

    B=2, context 128, gamma=8, A=8; anchors: 8 distinct positions drawn
    uniformly from the candidates (loss mask all ones, so p in [0, 126]),
    sorted; 2 of the 8 blocks per row (seeded choice) get keep=0.  Hidden
    states: context [2,128,256] and draft [2,64,256], N(0,1); projection
    weights N(0, 1/256) (std 1/sqrt(fan_in)); 4 query heads, 2 KV heads,
    head dim 64, scale 1/8.  The projections (part of the out-of-scope dense
    backbone) are done here in float64 and rounded to float32; both sides
    consume the projected Q/K/V.
    Markov: V=4096, r=32, base [16, 8, 4096] N(0, 2^2), W1 N(0,1),
    W2 N(0, 1/32), float32 weights; sequence tokens uniform in [0, V);
    first previous token = the token at the anchor; greedy.
    Eval mask: seq_len 128, loss mask all ones."""
    seed = SEED_BASE + 1
    rng = np.random.default_rng(seed)
    B, S, gamma, A, H, Hq, Hkv, D = 2, 128, 8, 8, 256, 4, 2, 64
    V, r = 4096, 32
    loss_mask = np.ones((B, S), dtype=np.uint8)
    anchor = np.zeros((B, A), dtype=np.int32)
    keep = np.zeros((B, A), dtype=np.uint8)
    for b in range(B):
        anchor[b], keep[b] = sample_anchors(rng, loss_mask[b], A, A)
        off = rng.choice(A, size=2, replace=False)
        keep[b, off] = 0
    tokens = rng.integers(0, V, size=(B, S), dtype=np.int32)
    h_ctx = rng.standard_normal((B, S, H)).astype(np.float64)
    h_drf = rng.standard_normal((B, A * gamma, H)).astype(np.float64)
    wq = rng.standard_normal((H, Hq * D)) / np.sqrt(H)
    wk = rng.standard_normal((H, Hkv * D)) / np.sqrt(H)
    wv = rng.standard_normal((H, Hkv * D)) / np.sqrt(H)
    f32 = lambda x: np.ascontiguousarray(x, dtype=np.float32)
    attn = AttentionCase(
        q=f32((h_drf @ wq).reshape(B, A * gamma, Hq, D)),
        k_ctx=f32((h_ctx @ wk).reshape(B * S, Hkv, D)),
        v_ctx=f32((h_ctx @ wv).reshape(B * S, Hkv, D)),
        ctx_offsets=np.array([0, S, 2 * S], dtype=np.int32),
        k_blk=f32((h_drf @ wk).reshape(B, A * gamma, Hkv, D)),
        v_blk=f32((h_drf @ wv).reshape(B, A * gamma, Hkv, D)),
        anchor=anchor, keep=keep, gamma=gamma, scale=1.0 / 8.0, dtype="f32")
    mrng = np.random.default_rng(seed + 100)
    markov = MarkovCase(
        base=mrng.standard_normal((B * A, gamma, V), dtype=np.float32) * np.float32(2.0),
        w1=mrng.standard_normal((V, r), dtype=np.float32),
        w2=mrng.standard_normal((r, V), dtype=np.float32) * np.float32(1.0 / np.sqrt(r)),
        first_prev=tokens[np.arange(B)[:, None], anchor].reshape(-1).astype(np.int32),
        temperature=0.0, seed=seed, wdtype="f32")
    mask = MaskCase(anchor=anchor, keep=keep,
                    seq_lens=np.full(B, S, dtype=np.int32), loss_mask=loss_mask,
                    gamma=gamma)
    return attn, markov, mask


# ------------------------------------------------------- full-size shapes
CONFIG2 = dict(B=1, S=4096, A=512, n_real=472, gamma=8, Hq=32, Hkv=8, D=128)
CONFIG3 = dict(R=64, gamma=16, V=151936, r=256, temperature=1.0)
CONFIG4 = dict(B=4, A=512, n_real=472, gamma=8, V=151936, S=4096)
CONFIG5 = dict(B=128, S_lo=1024, S_hi=8192, gamma=16, Hq=32, Hkv=8, D=128,
               V=151936, r=256, n_hi=63, n_finished=6)


def config2_structure():
    """Anchors of the training-style attention workload: 472 positions drawn
    without replacement from [0, 4094] (every position is a candidate when
    the loss mask is all ones), sorted; slots 472..511 padded anchor=0,
    keep=0."""
    c = CONFIG2
    rng = np.random.default_rng(SEED_BASE + 2)
    anchor, keep = sample_anchors(rng, np.ones(c["S"], dtype=np.uint8), c["n_real"], c["A"])
    return anchor[None, :], keep[None, :]


def config4_structure():
    """Eval-mask inputs and per-block noise levels of the accept-rate
    workload: prompt length P_b ~ U[64, 1024], loss_mask[b, t] = 1 for
    t >= P_b (the response region); 472 anchors from the candidates, sorted,
    40 pads with keep=0; seq_lens = 4096; sigma[b, a] ~ U[0.1, 3]."""
    c = CONFIG4
    rng = np.random.default_rng(SEED_BASE + 4)
    B, A, S = c["B"], c["A"], c["S"]
    loss_mask = np.zeros((B, S), dtype=np.uint8)
    anchor = np.zeros((B, A), dtype=np.int32)
    keep = np.zeros((B, A), dtype=np.uint8)
    for b in range(B):
        P = int(rng.integers(64, 1025))
        loss_mask[b, P:] = 1
        anchor[b], keep[b] = sample_anchors(rng, loss_mask[b], c["n_real"], A)
    sigma = rng.uniform(0.1, 3.0, size=(B, A)).astype(np.float32)
    mask = MaskCase(anchor=anchor, keep=keep, seq_lens=np.full(B, S, dtype=np.int32),
                    loss_mask=loss_mask, gamma=c["gamma"])
    return mask, sigma


def config5_structure():
    """Serving round structure: 128 requests with context lengths
    S_b ~ U{1024..8192}; one block per request anchored at the end of its
    context (anchor = S_b: the block sees the whole context); 6 of the 128
    requests (about 5 %, drawn without replacement from their own seeded
    stream) are finished and get keep = 0, the rest are kept; remaining
    generation budget n_b ~ U{0..63} so seq_lens_b = S_b + 1 + n_b and
    about a quarter of the blocks are truncated by the eval mask; first
    previous tokens uniform in [0, V)."""
    c = CONFIG5
    rng = np.random.default_rng(SEED_BASE + 5)
    B = c["B"]
    S = rng.integers(c["S_lo"], c["S_hi"] + 1, size=B).astype(np.int64)
    offsets = np.zeros(B + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(S)
    anchor = S.astype(np.int32)[:, None]
    keep = np.ones((B, 1), dtype=np.uint8)
    fin = np.random.default_rng(SEED_BASE + 55).choice(B, size=c["n_finished"], replace=False)
    keep[fin, 0] = 0
    n = rng.integers(0, c["n_hi"] + 1, size=B)
    seq_lens = (S + 1 + n).astype(np.int32)
    first_prev = rng.integers(0, c["V"], size=B, dtype=np.int32)
    mask = MaskCase(anchor=anchor, keep=keep, seq_lens=seq_lens, loss_mask=None,
                    gamma=c["gamma"])
    return dict(ctx_lens=S, ctx_offsets=offsets, anchor=anchor, keep=keep,
                first_prev=first_prev, mask=mask)


def config3_structure():
    rng = np.random.default_rng(SEED_BASE + 3)
    return rng.integers(0, CONFIG3["V"], size=CONFIG3["R"], dtype=np.int32)


# ----------------------------------------------- device draws (full sizes)
def device_normal(torch, gen, shape, std, dtype, device, chunk=1 << 27):
    """float32 N(0, std^2) drawn on `device` with generator `gen`, cast to
    `dtype` (torch dtype).  Drawn in chunks of `chunk` elements so the
    float32 temporary stays small."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[s:e].copy_(x)
    return out


def _gen(torch, device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def config2_device(torch, device):
    """Training-style attention inputs at full size: Q [1, 4096, 32, 128],
    K/V context [4096, 8, 128], K/V own blocks [1, 4096, 8, 128], all i.i.d.
    N(0, 1) rounded to bf16, drawn on `device`; anchors from
    config2_structure()."""
    c = CONFIG2
    anchor, keep = config2_structure()
    g = _gen(torch, device, SEED_BASE + 2)
    bf = torch.bfloat16
    AG = c["A"] * c["gamma"]
    out = dict(
        q=device_normal(torch, g, (c["B"], AG, c["Hq"], c["D"]), 1.0, bf, device),
        k_ctx=device_normal(torch, g, (c["S"], c["Hkv"], c["D"]), 1.0, bf, device),
        v_ctx=device_normal(torch, g, (c["S"], c["Hkv"], c["D"]), 1.0, bf, device),
        k_blk=device_normal(torch, g, (c["B"], AG, c["Hkv"], c["D"]), 1.0, bf, device),
        v_blk=device_normal(torch, g, (c["B"], AG, c["Hkv"], c["D"]), 1.0, bf, device),
        ctx_offsets=torch.tensor([0, c["S"]], dtype=torch.int32, device=device),
        anchor=torch.from_numpy(anchor).to(device), keep=torch.from_numpy(keep).to(device),
        anchor_host=anchor, keep_host=keep, max_ctx=c["S"])
    return out


def config3_device(torch, device):
    """Markov sampling inputs at full size: base [64, 16, 151936] float32
    N(0, 3^2); W1 [151936, 256] and W2 [256, 151936] bf16 N(0, 0.02^2);
    first previous tokens uniform in [0, V); temperature 1, Philox seed 1003."""
    c = CONFIG3
    g = _gen(torch, device, SEED_BASE + 3)
    return dict(
        base=device_normal(torch, g, (c["R"], c["gamma"], c["V"]), 3.0, torch.float32, device),
        w1=device_normal(torch, g, (c["V"], c["r"]), 0.02, torch.bfloat16, device),
        w2=device_normal(torch, g, (c["r"], c["V"]), 0.02, torch.bfloat16, device),
        first_prev=torch.from_numpy(config3_structure()).to(device),
        temperature=c["temperature"], seed=SEED_BASE + 3)


def config4_device(torch, device):
    """Accept-rate inputs at full size: draft [4, 512, 8, 151936] bf16
    N(0, 3^2); target = draft + N(0, sigma[b, a]^2) formed in float32 and
    rounded to bf16, sigma from config4_structure(); eval-mask inputs as
    there."""
    c = CONFIG4
    mask, sigma = config4_structure()
    g = _gen(torch, device, SEED_BASE + 4)
    shape = (c["B"], c["A"], c["gamma"], c["V"])
    draft = device_normal(torch, g, shape, 3.0, torch.bfloat16, device)
    target = torch.empty_like(draft)
    sig = torch.from_numpy(sigma).to(device)
    for b in range(c["B"]):
        for a0 in range(0, c["A"], 64):
            a1 = min(c["A"], a0 + 64)
            x = draft[b, a0:a1].float()
            x.add_(torch.randn(x.shape, generator=g, device=device, dtype=torch.float32)
                   * sig[b, a0:a1, None, None])
            target[b, a0:a1].copy_(x)
    return dict(draft=draft, target=target, mask=mask, sigma=sigma)


def config4_block_logits_device(torch, device):
    """Teacher-forced Markov block logits at the shape of workload 4's training
    batch: N = 4 x 512 x 8 = 16384 rows, base [N, 151936] float32 N(0, 3^2),
    W1 [151936, 256] and W2 [256, 151936] bf16 N(0, 0.02^2) (as workload 3),
    previous tokens uniform in [0, V)."""
    c = CONFIG4
    N, V, r = c["B"] * c["A"] * c["gamma"], c["V"], 256
    g = _gen(torch, device, SEED_BASE + 40)
    return dict(
        base=device_normal(torch, g, (N, V), 3.0, torch.float32, device),
        w1=device_normal(torch, g, (V, r), 0.02, torch.bfloat16, device),
        w2=device_normal(torch, g, (r, V), 0.02, torch.bfloat16, device),
        prev=torch.randint(0, V, (N,), generator=g, device=device, dtype=torch.int32),
        N=N, V=V, r=r)


def config5_device(torch, device):
    """Serving round inputs at full size (structure from config5_structure()):
    Q [128, 16, 32, 128], K/V context [sum S_b, 8, 128] and own-block K/V
    [128, 16, 8, 128], i.i.d. N(0, 1) bf16; Markov base [128, 16, 151936]
    float32 N(0, 3^2), W1/W2 bf16 N(0, 0.02^2), greedy."""
    c = CONFIG5
    st = config5_structure()
    g = _gen(torch, device, SEED_BASE + 5)
    bf = torch.bfloat16
    T = int(st["ctx_offsets"][-1])
    B, G = c["B"], c["gamma"]
    return dict(
        q=device_normal(torch, g, (B, G, c["Hq"], c["D"]), 1.0, bf, device),
        k_ctx=device_normal(torch, g, (T, c["Hkv"], c["D"]), 1.0, bf, device),
        v_ctx=device_normal(torch, g, (T, c["Hkv"], c["D"]), 1.0, bf, device),
        k_blk=device_normal(torch, g, (B, G, c["Hkv"], c["D"]), 1.0, bf, device),
        v_blk=device_normal(torch, g, (B, G, c["Hkv"], c["D"]), 1.0, bf, device),
        ctx_offsets=torch.from_numpy(st["ctx_offsets"]).to(device),
        anchor=torch.from_numpy(st["anchor"]).to(device),
        keep=torch.from_numpy(st["keep"]).to(device),
        base=device_normal(torch, g, (B, G, c["V"]), 3.0, torch.float32, device),
        w1=device_normal(torch, g, (c["V"], c["r"]), 0.02, bf, device),
        w2=device_normal(torch, g, (c["r"], c["V"]), 0.02, bf, device),
        first_prev=torch.from_numpy(st["first_prev"]).to(device),
        seq_lens=torch.from_numpy(st["mask"].seq_lens).to(device),
        structure=st, max_ctx=c["S_hi"])
