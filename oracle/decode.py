"""Oracle batch-1 greedy decode.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Open Flapping Airplanes ... A100 reproduction", section "What ran": serving is
autoregressive text generation from the changing model; the review "How one
persistent kernel runs three jobs" adds that one token releases the next.  The
pages give no window or sampling rule; the readings used here:

* greedy: the next token is the argmax of the last row's logits, lowest id on
  exact ties;
* window: the context holds at most ``n_ctx`` tokens at positions 0..n-1; when
  appending a token would exceed ``n_ctx`` the context restarts from its most
  recent ``keep`` tokens (the new token included), placed at positions
  0..keep-1.

The oracle recomputes every prediction from the token sequence with a full
causal forward (no cache); row t of ``gpt.sequence_logits`` is exactly the
prediction after tokens 0..t because attention is causal (pinned by a test).
"""

from __future__ import annotations

import numpy as np

from . import gpt


def argmax_lowest(row) -> int:
    """argmax with the lowest index on exact ties (numpy's argmax already does this)."""
    return int(np.argmax(row))


def top2_margin(row) -> float:
    part = np.partition(np.asarray(row), -2)
    return float(part[-1] - part[-2])


def windows(prompt, generated, n_ctx: int, keep: int):
    """Split a decode run into context segments under the window rule.

    Yields (context, rows): ``context`` is one segment's token list placed at
    positions 0..len-1, and each (r, i) in ``rows`` says that generated token i
    is predicted by row r of a causal forward over ``context``.
    """
    ctx = list(prompt)
    seg_rows = []          # (row in ctx, generated index)
    for i, tok in enumerate(generated):
        seg_rows.append((len(ctx) - 1, i))
        ctx.append(int(tok))
        if len(ctx) > n_ctx:
            yield ctx[:-1], seg_rows
            ctx = ctx[-keep:]
            seg_rows = []
    if seg_rows:
        yield ctx, seg_rows


def teacher_forced_logits(s: gpt.Spec, P: dict, prompt, generated, n_ctx: int,
                          keep: int, dtype=np.float64):
    """Logits [n_gen][V] that predict each token of ``generated`` under the window rule.

    The oracle follows the decoder's own token sequence (teacher forcing), so one
    early disagreement does not cascade.
    """
    out = np.zeros((len(generated), s.vocab), dtype=dtype)
    for ctx, rows in windows(prompt, generated, n_ctx, keep):
        z = gpt.sequence_logits(s, P, ctx, dtype=dtype)
        for r, i in rows:
            out[i] = z[r]
    return out


def greedy(s: gpt.Spec, P: dict, prompt, n_new: int, n_ctx: int, keep: int,
           dtype=np.float64):
    """Plain greedy decode by full recomputation of every prefix (small sizes only)."""
    ctx = list(prompt)
    out = []
    for _ in range(n_new):
        z = gpt.sequence_logits(s, P, ctx, dtype=dtype)[-1]
        y = argmax_lowest(z)
        out.append(y)
        ctx.append(y)
        if len(ctx) > n_ctx:
            ctx = ctx[-keep:]
    return out
