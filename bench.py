"""Throughput of one DSpark draft round on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one serving-shaped draft round over one batch resident in HBM:
eval mask, block-masked dual-source attention (one draft layer's attention
core) and the gamma-step Markov sampler, all through the C ABI on one
stream.  Workload: 128 requests with context lengths U{1024..8192}, one block
per request anchored at the end of its context, gamma = 16, 32 query / 8 KV
heads, head dim 128, V = 151936, Markov rank 256, greedy; bf16 inputs,
float32 accumulation.  The TV accept rate (with tau), which needs target
logits and so is not part of a serving round, is timed beside it on the
4 x 512 x 8-row training-shaped workload and reported under "accept_rate";
the training-shaped all-anchor attention (1 x 4096 context, 512 anchors,
gamma = 8; MFMA-bound) is timed too and reported under "attention_training"
against the bf16 matrix-core peak.  So are the two training-side neighbours
on the same 4 x 512 x 8-row shape: the L1 (TV) loss with its float32
gradient and tau_greedy ("l1_loss") and the teacher-forced Markov block
logits ("block_logits"), and, at the serving shape, the confidence head with
the verify-length scheduler ("confidence_schedule"), and the gated and
recurrent Markov-head samplers ("markov_heads") and the lossless verify
step ("verify").

Prints ONE JSON line: metric, value (drafted tokens/s), ms_per_step, the
per-operation breakdown, the roofline of the dominant kernel (achieved
algorithmic GB/s from HIP events on the launch stream vs the 8 TB/s HBM
peak) and the CPU oracle timed on a bounded sample of the same workload.

--only {round,attention,markov,accept,train_attention,copy,block_logits,l1_loss,schedule,heads,verify,config1,config3}
restricts the run to one part
(for profiler runs); --no-cpu skips the CPU baseline.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["round", "attention", "markov", "accept", "train_attention", "copy",
                                       "block_logits", "l1_loss", "schedule", "heads", "verify", "config1",
                                       "config3"],
                    default=None)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    return ap.parse_args()


KERNEL_SOURCES = {
    "block_attn_mfma<128,2,2,2>": "semi_autoregressive_block_amd/csrc/attention.hip",
    "markov_round_mfma<false>": "semi_autoregressive_block_amd/csrc/markov_round.hip",
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def source_digest(kernel):
    import hashlib
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES[kernel], "semi_autoregressive_block_amd/csrc/common.h"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary: FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what the
    same counter reads for a copy of known size.  None when there is no
    summary or the kernel's source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest(kernel):
        return None
    fetch = rec["fetch_kib"] * rec["copy_bytes"] / rec["copy_fetch_kib"]
    write = rec["write_kib"] * rec["copy_bytes"] / rec["copy_write_kib"]
    return fetch + write


def timed(torch, fn, steps, warmup):
    """Average ms of fn() over `steps` runs after `warmup`, bracketed by
    device synchronisation; events recorded on the current stream (the
    stream every library call is launched on)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def round_inputs(torch, dsp, W, dev):
    inp = W.config5_device(torch, dev)
    st = inp["structure"]
    c = W.CONFIG5
    B, G, Hq, Hkv, D, V, r = c["B"], c["gamma"], c["Hq"], c["Hkv"], c["D"], c["V"], c["r"]
    bufs = dict(
        out=torch.empty_like(inp["q"]),
        tokens=torch.empty((B, G), dtype=torch.int32, device=dev),
        mask=torch.empty((B, 1, G), dtype=torch.uint8, device=dev),
        ws_attn=torch.empty(max(1, dsp.block_attention_workspace_bytes(B, 1, G, Hq, Hkv, D, inp["max_ctx"])),
                            dtype=torch.uint8, device=dev),
        ws_mk=torch.empty(dsp.markov_sample_workspace_bytes(B, G, V, r), dtype=torch.uint8, device=dev),
    )
    kept = st["keep"][:, 0] != 0
    ctx_kept = int(st["ctx_lens"][kept].sum())
    nk = int(kept.sum())
    # algorithmic bytes: every input byte the definition reads once (a
    # finished request's block, keep = 0, reads nothing), every output
    # written once
    attn_bytes = (ctx_kept * Hkv * D * 2 * 2           # context K and V of kept blocks
                  + nk * G * Hq * D * 2 + B * G * Hq * D * 2  # Q of kept blocks in, every out row
                  + nk * G * Hkv * D * 2 * 2          # own-block K and V of kept blocks
                  + (B + 1) * 4 + B * 5)              # offsets, anchors, keep
    attn_flops = 4.0 * D * G * Hq * float(sum(int(s) + G for s in st["ctx_lens"][kept]))
    step_bytes = r * V * 2 + B * V * 4 + B * r * 2 + B * 8  # W2, base slice, W1 rows, keys
    # the sampler runs all G steps in one launch and reads W2 from memory once (it stays in the
    # compute units' registers): the least traffic a round needs
    round_min_bytes = r * V * 2 + G * (B * V * 4 + B * r * 2 + B * 8)
    return inp, bufs, dict(attn_bytes=attn_bytes, attn_flops=attn_flops,
                           markov_step_bytes=step_bytes, markov_steps=G, markov_min_bytes=round_min_bytes,
                           tokens=B * G)


def run_round(dsp, inp, bufs):
    st = inp["structure"]
    dsp.eval_mask(inp["anchor"], inp["keep"], inp["seq_lens"], gamma=16, out=bufs["mask"])
    dsp.block_attention(inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"], inp["k_blk"],
                        inp["v_blk"], inp["anchor"], inp["keep"], max_ctx=inp["max_ctx"],
                        out=bufs["out"], workspace=bufs["ws_attn"])
    dsp.markov_sample(inp["base"], inp["w1"], inp["w2"], inp["first_prev"], tokens=bufs["tokens"],
                      workspace=bufs["ws_mk"])


def cpu_baseline(W, inp, budget_s):
    """The oracle, as it is, on the first requests of the same round until
    about `budget_s` of CPU time has been spent (at least two requests)."""
    import numpy as np
    from oracle import attention as OA
    from oracle import eval_mask as OE
    from oracle import markov as OM

    f = lambda t: W.bf16_to_f32(t.contiguous().view(__import__("torch").int16).cpu().numpy().view(np.uint16))
    st = inp["structure"]
    offs = st["ctx_offsets"]
    w1 = f(inp["w1"]).astype(np.float64)
    w2 = f(inp["w2"]).astype(np.float64)
    t0 = time.perf_counter()
    n = 0
    while n < 2 or (time.perf_counter() - t0 < budget_s and n < 128):
        b = n
        c0, c1 = int(offs[b]), int(offs[b + 1])
        q = f(inp["q"][b:b + 1])
        kc, vc = f(inp["k_ctx"][c0:c1]), f(inp["v_ctx"][c0:c1])
        kb, vb = f(inp["k_blk"][b:b + 1]), f(inp["v_blk"][b:b + 1])
        OE.eval_mask(st["anchor"][b:b + 1], st["keep"][b:b + 1], st["mask"].seq_lens[b:b + 1], None, 16)
        OA.block_attention(q, kc, vc, np.array([0, c1 - c0]), kb, vb, st["anchor"][b:b + 1],
                           st["keep"][b:b + 1], 16, 1.0 / np.sqrt(128))
        base = inp["base"][b:b + 1].cpu().numpy()
        OM.sample_block_tokens(base, w1, w2, st["first_prev"][b:b + 1], 0.0, 0)
        n += 1
    el = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    return dict(value=n * 16 / el, unit="drafted tokens/s", cores=int(cores), kind="oracle",
                sample=f"first {n} of 128 requests of the same round (attention over their "
                       f"contexts, 16 Markov steps over V=151936, eval mask); {el:.1f} s; "
                       "float64 numpy, BLAS threads = cores")


def _oracle_threads(n):
    """Context manager limiting the oracle's BLAS threads to n (None: as is)."""
    import contextlib
    if n is None:
        return contextlib.nullcontext()
    from threadpoolctl import threadpool_limits
    return threadpool_limits(n)


def _cores():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return 1


def config1_part(torch, dsp, W, dev, K, Wm, cpu):
    """Tiny float32 draft round: eval mask + attention (2 rows x 8 blocks of
    8, 4/2 heads, D = 64, context 128) + Markov sampling (16 rows, V = 4096,
    r = 32, float32 weights, greedy).  Latency per round and 128 drafted
    positions / t; the oracle on the same inputs, single-threaded and with
    every BLAS thread."""
    import numpy as np
    attn, mk, mask = W.config1()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q, kc, vc, kb, vb = (t(getattr(attn, n)) for n in ("q", "k_ctx", "v_ctx", "k_blk", "v_blk"))
    offs, anc, keep = t(attn.ctx_offsets), t(attn.anchor), t(attn.keep)
    seq = t(mask.seq_lens)
    lm = t(mask.loss_mask)
    base, w1, w2, fp = t(mk.base), t(mk.w1), t(mk.w2), t(mk.first_prev)
    out = torch.empty_like(q)
    em = torch.empty((2, 8, 8), dtype=torch.uint8, device=dev)
    tok = torch.empty((16, 8), dtype=torch.int32, device=dev)
    wsa = torch.empty(max(1, dsp.block_attention_workspace_bytes(2, 8, 8, 4, 2, 64, 128)), dtype=torch.uint8,
                      device=dev)
    wsm = torch.empty(dsp.markov_sample_workspace_bytes(16, 8, 4096, 32, 0), dtype=torch.uint8, device=dev)

    def rnd():
        dsp.eval_mask(anc, keep, seq, lm, gamma=8, out=em)
        dsp.block_attention(q, kc, vc, offs, kb, vb, anc, keep, max_ctx=128, scale=attn.scale, out=out,
                            workspace=wsa)
        dsp.markov_sample(base, w1, w2, fp, tokens=tok, workspace=wsm)

    ms = timed(torch, rnd, K, Wm) if K > 0 else None
    res = dict(ms=ms, tokens=128)
    if cpu:
        from oracle import attention as OA
        from oracle import eval_mask as OE
        from oracle import markov as OM

        def oracle_round():
            OE.eval_mask(mask.anchor, mask.keep, mask.seq_lens, mask.loss_mask, 8)
            OA.block_attention(attn.q, attn.k_ctx, attn.v_ctx, attn.ctx_offsets, attn.k_blk, attn.v_blk,
                               attn.anchor, attn.keep, 8, attn.scale)
            OM.sample_block_tokens(mk.base, mk.w1, mk.w2, mk.first_prev, 0.0, 0)

        for label, n in (("cpu_1thread", 1), ("cpu", None)):
            with _oracle_threads(n):
                oracle_round()
                reps, t0 = 0, time.perf_counter()
                while reps < 3 or time.perf_counter() - t0 < 2.0:
                    oracle_round()
                    reps += 1
                el = (time.perf_counter() - t0) / reps
                res[label] = dict(value=128 / el, unit="drafted tokens/s", ms=el * 1e3,
                                  cores=1 if n == 1 else _cores(), kind="oracle",
                                  sample=f"the whole round, {reps} repetitions")
    return res


def config3_part(torch, dsp, W, dev, K, Wm, cpu, budget_s=10.0):
    """Markov sampling at the full configuration: 64 rows, gamma = 16,
    V = 151936, rank 256, bf16 weights, temperature 1 Gumbel-max.  Time per
    round, 1024 drafted tokens / t, algorithmic bytes per round vs the HBM
    peak; the oracle on the first rows of the same inputs for about
    budget_s."""
    import numpy as np
    c = W.CONFIG3
    inp = W.config3_device(torch, dev)
    R, G, V, r = c["R"], c["gamma"], c["V"], c["r"]
    tok = torch.empty((R, G), dtype=torch.int32, device=dev)
    ws = torch.empty(dsp.markov_sample_workspace_bytes(R, G, V, r), dtype=torch.uint8, device=dev)
    f = lambda: dsp.markov_sample(inp["base"], inp["w1"], inp["w2"], inp["first_prev"],
                                  temperature=inp["temperature"], seed=inp["seed"], tokens=tok, workspace=ws)
    ms = timed(torch, f, K, Wm)
    step_bytes = r * V * 2 + R * V * 4 + R * r * 2 + R * 4  # W2, base slice, W1 rows, prev
    res = dict(ms=ms, tokens=R * G, bytes=G * step_bytes)
    if cpu:
        from oracle import markov as OM
        fb = lambda x: W.bf16_to_f32(x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
        w1 = fb(inp["w1"]).astype(np.float64)
        w2 = fb(inp["w2"]).astype(np.float64)
        fp = inp["first_prev"].cpu().numpy()
        n, t0 = 0, time.perf_counter()
        while n < 1 or (time.perf_counter() - t0 < budget_s and n < R):
            OM.sample_block_tokens(inp["base"][n:n + 1].cpu().numpy(), w1, w2, fp[n:n + 1],
                                   inp["temperature"], inp["seed"], rows=np.array([n]))
            n += 1
        el = time.perf_counter() - t0
        res["cpu"] = dict(value=n * G / el, unit="drafted tokens/s", cores=_cores(), kind="oracle",
                          sample=f"first {n} of {R} rows, all 16 steps; {el:.1f} s; float64 numpy")
    del inp, ws
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the bench runs on one GPU: --gpus must be 1 (the path has no multi-GPU mode)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import semi_autoregressive_block_amd as dsp
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    K, Wm = args.steps, args.warmup
    result = {}

    if args.only == "copy":
        # plain copy of a known size: the scale factor for the HBM counters
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        ms = timed(torch, lambda: b.copy_(a), K, Wm)
        print(json.dumps({"copy_bytes": n, "ms": ms, "GBps": 2 * n / ms / 1e6}))
        return

    if args.only in (None, "round", "attention", "markov"):
        inp, bufs, alg = round_inputs(torch, dsp, W, dev)
        f_attn = lambda: dsp.block_attention(
            inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"], inp["k_blk"], inp["v_blk"],
            inp["anchor"], inp["keep"], max_ctx=inp["max_ctx"], out=bufs["out"],
            workspace=bufs["ws_attn"])
        f_mk = lambda: dsp.markov_sample(inp["base"], inp["w1"], inp["w2"], inp["first_prev"],
                                         tokens=bufs["tokens"], workspace=bufs["ws_mk"])
        f_mask = lambda: dsp.eval_mask(inp["anchor"], inp["keep"], inp["seq_lens"], gamma=16,
                                       out=bufs["mask"])
        if args.only == "attention":
            ms = timed(torch, f_attn, K, Wm)
            print(json.dumps({"attention_ms": ms, "GBps": alg["attn_bytes"] / ms / 1e6}))
            return
        if args.only == "markov":
            ms = timed(torch, f_mk, K, Wm)
            print(json.dumps({"markov_ms": ms,
                              "GBps": alg["markov_step_bytes"] * 16 / ms / 1e6}))
            return
        round_ms = timed(torch, lambda: run_round(dsp, inp, bufs), K, Wm)
        if args.only == "round":
            print(json.dumps({"round_ms": round_ms}))
            return
        attn_ms = timed(torch, f_attn, K, Wm)
        mk_ms = timed(torch, f_mk, K, Wm)
        mask_ms = timed(torch, f_mask, K, Wm)
        result["round"] = dict(ms=round_ms, attn_ms=attn_ms, markov_ms=mk_ms, mask_ms=mask_ms, **alg)
        round_inp = inp  # the CPU baseline runs last: seconds of host work would idle the GPU in between
        del bufs
        torch.cuda.empty_cache()

    if args.only in (None, "config1"):
        result["config1"] = config1_part(torch, dsp, W, dev, K, Wm, cpu=args.only == "config1" and not args.no_cpu)
        if args.only == "config1":
            print(json.dumps(result["config1"]))
            return

    if args.only in (None, "config3"):
        result["config3"] = config3_part(torch, dsp, W, dev, K, Wm, cpu=False)
        if args.only == "config3":
            print(json.dumps(result["config3"]))
            return

    if args.only in (None, "train_attention"):
        # training-shaped all-anchor attention: 472 kept blocks of 8 rows
        # over one 4096-token context, 32 query / 8 KV heads, D = 128
        t2 = W.config2_device(torch, dev)
        c2 = W.CONFIG2
        out2 = torch.empty_like(t2["q"])
        ws2 = torch.empty(max(1, dsp.block_attention_workspace_bytes(1, c2["A"], c2["gamma"], c2["Hq"], c2["Hkv"],
                                                                     c2["D"], c2["S"])),
                          dtype=torch.uint8, device=dev)
        f_t2 = lambda: dsp.block_attention(t2["q"], t2["k_ctx"], t2["v_ctx"], t2["ctx_offsets"], t2["k_blk"],
                                           t2["v_blk"], t2["anchor"], t2["keep"], max_ctx=t2["max_ctx"],
                                           out=out2, workspace=ws2)
        t2_ms = timed(torch, f_t2, K, Wm)
        a2, k2 = t2["anchor_host"], t2["keep_host"]
        # QK^T and PV over the visible pairs only
        t2_flops = 4.0 * c2["gamma"] * c2["D"] * c2["Hq"] * float(((a2 + c2["gamma"]) * (k2 != 0)).sum())
        if args.only == "train_attention":
            print(json.dumps({"train_attention_ms": t2_ms, "TFLOPs": t2_flops / t2_ms / 1e9}))
            return
        # draft positions: kept blocks x gamma query positions (each over all query heads)
        t2_pos = c2["gamma"] * int((k2 != 0).sum())
        result["train_attention"] = dict(ms=t2_ms, flops=t2_flops, positions=t2_pos)
        del t2, out2, ws2
        torch.cuda.empty_cache()

    if args.only in (None, "accept"):
        a4 = W.config4_device(torch, dev)
        m = a4["mask"]
        em = dsp.eval_mask(torch.from_numpy(m.anchor).to(dev), torch.from_numpy(m.keep).to(dev),
                           torch.from_numpy(m.seq_lens).to(dev), torch.from_numpy(m.loss_mask).to(dev),
                           gamma=8)
        acc = torch.empty((4, 512, 8), dtype=torch.float32, device=dev)
        tau = torch.empty((4, 512), dtype=torch.float32, device=dev)
        ws = torch.empty(dsp.accept_rate_workspace_bytes(4, 512, 8, 151936), dtype=torch.uint8, device=dev)
        f_acc = lambda: dsp.accept_rate(a4["draft"], a4["target"], eval_mask=em, accept=acc, tau=tau,
                                        workspace=ws)
        acc_ms = timed(torch, f_acc, K, Wm)
        acc_bytes = 2 * a4["draft"].numel() * 2 + 16384 * 4 + 16384 + 2048 * 4
        if args.only == "accept":
            print(json.dumps({"accept_ms": acc_ms, "GBps": acc_bytes / acc_ms / 1e6}))
            return
        result["accept"] = dict(ms=acc_ms, bytes=acc_bytes)
        del a4
        torch.cuda.empty_cache()

    if args.only in (None, "l1_loss"):
        # L1 (TV) loss with its gradient on workload 4's draft / target logits
        a4 = W.config4_device(torch, dev)
        m = a4["mask"]
        em = dsp.eval_mask(torch.from_numpy(m.anchor).to(dev), torch.from_numpy(m.keep).to(dev),
                           torch.from_numpy(m.seq_lens).to(dev), torch.from_numpy(m.loss_mask).to(dev),
                           gamma=8)
        grad = torch.empty(a4["draft"].shape, dtype=torch.float32, device=dev)
        loss = torch.empty((1,), dtype=torch.float32, device=dev)
        ws = torch.empty(dsp.l1_loss_workspace_bytes(4, 512, 8, 151936), dtype=torch.uint8, device=dev)
        f_l1 = lambda: dsp.l1_loss(a4["draft"], a4["target"], eval_mask=em, loss=loss, grad=grad, workspace=ws)
        l1_ms = timed(torch, f_l1, K, Wm)
        l1_bytes = 2 * a4["draft"].numel() * 2 + grad.numel() * 4  # both logit tensors once + the gradient
        # streaming ceiling of the same traffic mix (as many bytes read as written, 19.9 GB in all) on
        # this GPU: the runtime's copy of a gradient-sized float32 tensor into the gradient
        src = torch.empty_like(grad)
        ceil_ms = timed(torch, lambda: grad.copy_(src), K, Wm)
        del src
        if args.only == "l1_loss":
            print(json.dumps({"l1_loss_ms": l1_ms, "GBps": l1_bytes / l1_ms / 1e6,
                              "stream_ceiling_GBps": l1_bytes / ceil_ms / 1e6}))
            return
        result["l1_loss"] = dict(ms=l1_ms, bytes=l1_bytes, ceil_ms=ceil_ms)
        del a4, grad
        torch.cuda.empty_cache()

    if args.only in (None, "block_logits"):
        # teacher-forced Markov block logits, 16384 rows x V = 151936, rank 256
        bl = W.config4_block_logits_device(torch, dev)
        out = torch.empty_like(bl["base"])
        ws = torch.empty(dsp.markov_block_logits_workspace_bytes(bl["N"], bl["V"], bl["r"]), dtype=torch.uint8,
                         device=dev)
        f_bl = lambda: dsp.markov_block_logits(bl["base"], bl["w1"], bl["w2"], bl["prev"], logits=out,
                                               workspace=ws)
        bl_ms = timed(torch, f_bl, K, Wm)
        N, V, rr = bl["N"], bl["V"], bl["r"]
        bl_bytes = 2 * N * V * 4 + rr * V * 2 + N * rr * 2 + N * 4  # base in, logits out, W2, W1 rows, prev
        bl_flops = 2.0 * N * rr * V
        if args.only == "block_logits":
            print(json.dumps({"block_logits_ms": bl_ms, "GBps": bl_bytes / bl_ms / 1e6}))
            return
        result["block_logits"] = dict(ms=bl_ms, bytes=bl_bytes, flops=bl_flops)
        del bl, out
        torch.cuda.empty_cache()

    if args.only in (None, "heads"):
        # gated and recurrent Markov-head samplers at the serving shape: 128
        # requests x 16 steps, V = 151936, rank 256, hidden 4096, greedy
        g = torch.Generator(device=dev).manual_seed(W.SEED_BASE + 60)
        R, G, V, rr, d = 128, 16, 151936, 256, 4096
        base = torch.randn((R, G, V), generator=g, device=dev).mul_(3)
        hid = torch.randn((R, G, d), generator=g, device=dev).to(torch.bfloat16)
        w1h = (torch.randn((V, rr), generator=g, device=dev) * 0.5).to(torch.bfloat16)
        w2h = (torch.randn((rr, V), generator=g, device=dev) * 0.3).to(torch.bfloat16)
        heads = {"gated": (torch.randn((rr, d + rr), generator=g, device=dev) * 1.5 / (d + rr) ** 0.5),
                 "rnn": (torch.randn((3, rr, 2 * rr + d), generator=g, device=dev) * 1.5 / (2 * rr + d) ** 0.5)}
        fp = torch.randint(0, V, (R,), generator=g, device=dev, dtype=torch.int32)
        toks = torch.empty((R, G), dtype=torch.int32, device=dev)
        h_ms = {}
        for kind, wt in heads.items():
            wt = wt.to(torch.bfloat16)
            ws = torch.empty(dsp.markov_head_sample_workspace_bytes(kind, R, G, V, rr), dtype=torch.uint8, device=dev)
            f_h = lambda: dsp.markov_head_sample(kind, base, hid, w1h, w2h, wt, fp, tokens=toks, workspace=ws)
            h_ms[kind] = timed(torch, f_h, K, Wm)
        if args.only == "heads":
            print(json.dumps({"heads_ms": h_ms}))
            return
        result["heads"] = h_ms
        del base, hid, w1h, w2h, heads
        torch.cuda.empty_cache()

    if args.only in (None, "verify"):
        # lossless verify of 128 drafted blocks of 16 tokens, V = 151936, T = 1,
        # draft logits near the target's (about half the drafts kept)
        g = torch.Generator(device=dev).manual_seed(W.SEED_BASE + 70)
        R, Kv, V = 128, 16, 151936
        tl = torch.randn((R, Kv + 1, V), generator=g, device=dev).mul_(2)
        dl = tl[:, :Kv] + torch.randn((R, Kv, V), generator=g, device=dev).mul_(0.3)
        xt = torch.distributions.Categorical(logits=dl).sample().to(torch.int32)
        ws = torch.empty(dsp.verify_workspace_bytes(R, Kv), dtype=torch.uint8, device=dev)
        nv, tv = torch.empty(R, dtype=torch.int32, device=dev), torch.empty(R, dtype=torch.int32, device=dev)
        f_v = lambda: dsp.verify(dl, tl, xt, temperature=1.0, seed=3, n_accepted=nv, next_token=tv, workspace=ws)
        v_ms = timed(torch, f_v, K, Wm)
        v_bytes = (2 * Kv + 1) * R * V * 4 + 2 * R * V * 4  # every position's logits once, the stop row twice
        if args.only == "verify":
            print(json.dumps({"verify_ms": v_ms, "GBps": v_bytes / v_ms / 1e6}))
            return
        result["verify"] = dict(ms=v_ms, bytes=v_bytes, mean_kept=float(nv.float().mean().item()))
        del tl, dl, xt
        torch.cuda.empty_cache()

    if args.only in (None, "schedule"):
        # confidence head + verify-length scheduler at the serving shape: 128
        # blocks of 16 positions, hidden size 4096 (32 heads x 128), Markov
        # input from a rank-256 W1 over V = 151936
        g = torch.Generator(device=dev).manual_seed(W.SEED_BASE + 50)
        hid = torch.randn((128, 1, 16, 4096), generator=g, device=dev).to(torch.bfloat16)
        wh = torch.randn(4096, generator=g, device=dev) / 64
        w1s = torch.randn((151936, 256), generator=g, device=dev).to(torch.bfloat16) * 0.02
        prev = torch.randint(0, 151936, (128, 1, 16), generator=g, device=dev, dtype=torch.int32)
        we = torch.randn(256, generator=g, device=dev)
        sps = torch.linspace(1.0, 0.4, 17, device=dev)
        f_s = lambda: dsp.confidence_schedule(hid, wh, 0.5, sps, w1=w1s, prev=prev, weight_e=we)
        s_ms = timed(torch, f_s, K, Wm)
        if args.only == "schedule":
            print(json.dumps({"schedule_ms": s_ms}))
            return
        result["schedule"] = dict(ms=s_ms)
        del hid, w1s
        torch.cuda.empty_cache()

    if not args.no_cpu:
        result["cpu"] = cpu_baseline(W, round_inp, args.cpu_seconds)
        if "config1" in result:
            # the oracles beside workloads 1 and 3, after every GPU part (idle GPU time between parts
            # lowers the clocks of the next one)
            c1 = config1_part(torch, dsp, W, dev, 0, 0, cpu=True)
            result["config1"].update({k: c1[k] for k in ("cpu", "cpu_1thread")})
        if "config3" in result:
            result["config3"]["cpu"] = config3_part(torch, dsp, W, dev, 1, 0, cpu=True,
                                                    budget_s=args.cpu_seconds / 2)["cpu"]

    r = result["round"]
    attn_gbs = r["attn_bytes"] / r["attn_ms"] / 1e6
    # one launch per round: the step's algorithmic bytes (W2, base slice, W1 rows, keys) times
    # the steps, and separately the least traffic (W2 once)
    mk_bytes = r["markov_step_bytes"] * r["markov_steps"]
    mk_gbs = mk_bytes / r["markov_ms"] / 1e6
    mk_min_gbs = r["markov_min_bytes"] / r["markov_ms"] / 1e6
    if r["attn_ms"] >= r["markov_ms"]:
        k = "block_attn_mfma<128,2,2,2>"
        roof = dict(kernel=k, bound="hbm", achieved=attn_gbs,
                    peak=HBM_PEAK_GBS, unit="GB/s", frac=attn_gbs / HBM_PEAK_GBS,
                    traffic=measured_traffic(k), bytes_per_launch=r["attn_bytes"],
                    launch_ms=r["attn_ms"])
    else:
        k = "markov_round_mfma<false>"
        roof = dict(kernel=k, bound="hbm", achieved=mk_gbs, peak=HBM_PEAK_GBS,
                    unit="GB/s", frac=mk_gbs / HBM_PEAK_GBS, traffic=measured_traffic(k),
                    bytes_per_launch=mk_bytes, launch_ms=r["markov_ms"],
                    min_traffic_bytes=r["markov_min_bytes"], min_traffic_frac=mk_min_gbs / HBM_PEAK_GBS)
    line = {
        "metric": "drafted tokens/s per draft round (attn+Markov)",
        "value": r["tokens"] / (r["ms"] / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": Wm, "ms_per_step": r["ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "serving draft round: 128 requests, context U{1024..8192}, "
                               "one block at the context end, gamma=16, Hq=32/Hkv=8, D=128, "
                               "V=151936, Markov rank 256, greedy",
                   "global_batch": 128, "seq_len": "1024-8192", "gamma": 16},
        "breakdown_ms": {"eval_mask": r["mask_ms"], "block_attention": r["attn_ms"],
                         "markov_sample": r["markov_ms"]},
        "attention": {"GBps": attn_gbs, "hbm_frac": attn_gbs / HBM_PEAK_GBS,
                      "TFLOPs": r["attn_flops"] / r["attn_ms"] / 1e9,
                      "mfma_frac": r["attn_flops"] / r["attn_ms"] / 1e9 / MFMA_BF16_PEAK_TFLOPS},
        "markov": {"kernel": "markov_round_mfma<false> (all 16 steps in one launch)",
                   "algorithmic_GBps": mk_gbs, "hbm_frac": mk_gbs / HBM_PEAK_GBS,
                   "min_traffic_GBps": mk_min_gbs, "min_traffic_frac": mk_min_gbs / HBM_PEAK_GBS,
                   "ms_per_round": r["markov_ms"], "ms_per_step": r["markov_ms"] / r["markov_steps"]},
        "roofline": roof,
    }
    if "accept" in result:
        a = result["accept"]
        gbs = a["bytes"] / a["ms"] / 1e6
        line["accept_rate"] = {"workload": "4 x 512 x 8 rows, V=151936 bf16, with tau",
                               "ms": a["ms"], "GBps": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                               "rows_per_s": 16384 / (a["ms"] / 1e3)}
    if "verify" in result:
        a = result["verify"]
        gbs = a["bytes"] / a["ms"] / 1e6
        line["verify"] = {"workload": "128 drafted blocks of 16 tokens, V=151936, float32 draft and target logits, "
                                      "T=1", "ms": a["ms"], "GBps": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                          "mean_kept": a["mean_kept"]}
    if "heads" in result:
        line["markov_heads"] = {"workload": "gamma = 16 sampling steps for 128 requests, V=151936, rank 256, "
                                            "hidden 4096 bf16, float32 base, greedy",
                                "gated_ms": result["heads"]["gated"], "rnn_ms": result["heads"]["rnn"]}
    if "l1_loss" in result:
        a = result["l1_loss"]
        gbs = a["bytes"] / a["ms"] / 1e6
        ceil = a["bytes"] / a["ceil_ms"] / 1e6
        line["l1_loss"] = {"workload": "4 x 512 x 8 rows, V=151936 bf16, loss + float32 gradient + tau_greedy",
                           "ms": a["ms"], "GBps": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                           "stream_ceiling_GBps": ceil, "ceiling_frac": gbs / ceil}
    if "block_logits" in result:
        a = result["block_logits"]
        gbs = a["bytes"] / a["ms"] / 1e6
        line["block_logits"] = {"workload": "teacher-forced Markov logits, 16384 rows, V=151936, rank 256, "
                                            "float32 base and logits, bf16 W1/W2",
                                "ms": a["ms"], "GBps": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                                "TFLOPs": a["flops"] / a["ms"] / 1e9}
    if "schedule" in result:
        line["confidence_schedule"] = {"workload": "128 blocks x 16 positions, hidden 4096 bf16, Markov input "
                                                   "rank 256, verify-length scan", "ms": result["schedule"]["ms"]}
    if "train_attention" in result:
        a = result["train_attention"]
        tf = a["flops"] / a["ms"] / 1e9
        line["attention_training"] = {"workload": "1 x 4096 context, 512 anchors (472 kept), gamma=8, "
                                                  "Hq=32/Hkv=8, D=128, bf16",
                                      "ms": a["ms"], "TFLOPs": tf, "mfma_frac": tf / MFMA_BF16_PEAK_TFLOPS,
                                      "algorithmic_flops": a["flops"],
                                      "positions_per_s": a["positions"] / (a["ms"] / 1e3)}
    if "config1" in result:
        a = result["config1"]
        line["config1"] = {"workload": "tiny float32 round: 2 x 8 blocks of 8 over context 128, Hq=4/Hkv=2, D=64; "
                                       "Markov 16 rows, V=4096, rank 32, greedy; eval mask",
                           "ms": a["ms"], "tokens_per_s": a["tokens"] / (a["ms"] / 1e3)}
        for k in ("cpu", "cpu_1thread"):
            if k in a:
                line["config1"][k] = a[k]
    if "config3" in result:
        a = result["config3"]
        gbs = a["bytes"] / a["ms"] / 1e6
        line["config3"] = {"workload": "Markov sampling: 64 rows, gamma=16, V=151936, rank 256, bf16 weights, "
                                       "T=1 Gumbel-max", "ms": a["ms"], "tokens_per_s": a["tokens"] / (a["ms"] / 1e3),
                           "GBps": gbs, "hbm_frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": a["bytes"]}
        if "cpu" in a:
            line["config3"]["cpu"] = a["cpu"]
    if "cpu" in result:
        line["cpu_baseline"] = result["cpu"]
    print(json.dumps(line))


if __name__ == "__main__":
    main()
