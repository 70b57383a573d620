"""Plain CPU oracle for the GPT training step and greedy decode.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports, calls or links it, and
this package imports nothing from the product package.

Everything here is written in plain numpy (fp64 by default) so that a reader can
check it against the pages by eye: no blocking, fusion or reordering beyond the
textbook definitions.  Sources followed (cited by page title and section):

* "Open Flapping Airplanes ... A100 reproduction" (curiouscaliboi.github.io),
  section "What ran": the 162M GPT (12 layers, width 768, 12 heads), AdamW,
  8 x 512 tokens per step, seeded initial weights.
* "Coppelius training on the RTX 3090" (lsalpha.com), kernel-family table in
  "Where a step's time goes": the step is embedding gather, LayerNorm
  forward/backward/parameter grads, attention forward plus key-side and
  query-side backward, (gated-)GELU forward/backward, RoPE and its inverse,
  cross-entropy forward/backward with target gather, embedding scatter and one
  fused AdamW; "Run" record: the 57.7M RoPE/gated-GELU model; "Loss": mean
  cross-entropy over the rows of the context, ln V for a model that knows
  nothing.
* "How one persistent kernel runs three jobs" (yuxiaoba.github.io review),
  section "How one persistent kernel runs three jobs": serving generates from
  the changing weights, one token releases the next.

Where those pages give no formula the oracle uses the textbook definition; the
readings taken are listed in the module docstrings.

Parity status: every function here is pinned by a ``-m "not gpu"`` test
(closed forms, invariants, finite differences, brute force); none is
"parity unpinned".
"""
