"""CPU oracle for the DSpark draft-round hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import anything from here.  The
product path (the HIP library and its Python binding) never imports, calls or
links this package, and this package never imports the product path.

Everything here is deliberately plain and slow: float64 arithmetic on the exact
values of the stored inputs, loops or whole-array numpy expressions that follow
the definitions on the pages, and no blocking, fusion or reordering beyond what
each definition states.  Sources, cited per function:

* page 1 — "03 · DSpark 建模：Markov 与 Confidence" (devpress.csdn.net),
  sections 3.1–3.13;
* page 2 — "从 DFlash 到 dLLM Self-Spec（三）" (r00kie-liu.github.io),
  sections 3.4, 3.5, 3.8;
* page 3 — "如何评价 DeepSeek 发布 DSpark？哪些亮点值得关注？" (foosynaptic.github.io
  reading notes), the speculative-decoding primer;
* page 4 — "DSpark 深度解读" (juejin.cn), sections 1.2, 3.2–3.4, 4.1 and 5.1;
* Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
  (SC'11) for the Philox counter-based generator.

Modules:

* ``attention``   — block-masked dual-source attention (page 1 §3.4–3.5).
* ``markov``      — Markov-head step logits and the gamma-step sampler
                    (page 1 §3.7, page 2 §3.4 / §3.8.2).
* ``accept_rate`` — TV accept rate and the tau statistic (page 1 §3.9–3.10,
                    page 2 §3.5).
* ``eval_mask``   — the cumulative-product eval mask (page 1 §3.1, §3.6).
* ``tv_loss``     — teacher-forced Markov block logits, the L1 (TV) loss and
                    its gradient, tau_greedy (page 1 §3.7, §3.9–3.10, §3.12;
                    page 4 §3.3, §4.1).
* ``scheduler``   — confidence head, prefix survival and the causal-greedy
                    verify-length scheduler (page 1 §3.8; page 4 §3.4, §5.1).
* ``markov_heads``— gated and recurrent Markov heads: step embedding,
                    teacher-forced block logits and the stateful sampler
                    (page 1 §3.7; page 4 §3.3).
* ``verify``      — the lossless verify step: rejection sampling of a drafted
                    block against the target (page 3's primer, page 4 §1.2;
                    the published speculative-sampling rule).
* ``philox``      — Philox4x32-10 / 4x64-10 and the Gumbel noise built on it.

Every function here is pinned by a ``-m "not gpu"`` test against something
other than itself (closed forms, brute force, library routines, published
known-answer vectors); there is no "parity unpinned" function.
"""

from . import accept_rate, attention, eval_mask, markov, markov_heads, philox, scheduler, tv_loss, verify  # noqa: F401
