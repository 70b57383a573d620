"""Oracle AdamW, learning-rate schedule and training loop.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Open Flapping Airplanes ... A100 reproduction", section "What ran": the 162M
run trains with AdamW from seeded initial weights; section "Reproducibility
needs inputs and an environment record": a 100-step smoke run used the
4,000-step learning-rate schedule, i.e. the schedule is a function of the step
index and of the total step count, not of the run length.  "Coppelius training
on the RTX 3090" ("Where a step's time goes") applies AdamW as one update over
all parameters per step.

Readings (the pages give no formula): decoupled weight decay applied to every
parameter, bias-corrected moments, no gradient clipping; the cosine schedule is
lr_s = lr * (1 + cos(pi * s / total)) / 2 for 0-based step s, no warm-up.
"""

from __future__ import annotations

import math

import numpy as np

from . import gpt


def lr_at(s: gpt.Spec, step: int) -> float:
    """Learning rate of 0-based step ``step``."""
    if s.lr_schedule == "constant":
        return s.lr
    if s.lr_schedule == "cosine":
        return s.lr * 0.5 * (1.0 + math.cos(math.pi * step / s.total_steps))
    raise ValueError(s.lr_schedule)


def adamw_update(p, g, m, v, t, lr, beta1, beta2, eps, wd):
    """One AdamW update in place; t is the 1-based step count.

    p <- p (1 - lr wd);  m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2;
    p <- p - lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
    """
    p *= (1.0 - lr * wd)
    m *= beta1
    m += (1.0 - beta1) * g
    v *= beta2
    v += (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** t)
    vhat = v / (1.0 - beta2 ** t)
    p -= lr * mhat / (np.sqrt(vhat) + eps)


class Trainer:
    """Holds flat parameters and AdamW moments; one ``step`` per token batch."""

    def __init__(self, s: gpt.Spec, flat_init, dtype=np.float64):
        self.s = s
        self.dtype = dtype
        self.flat = np.array(flat_init, dtype=dtype)
        self.m = np.zeros_like(self.flat)
        self.v = np.zeros_like(self.flat)
        self.steps_done = 0

    def params(self) -> dict:
        return gpt.unflatten(self.s, self.flat)

    def grads(self, tokens):
        loss, g = gpt.loss_and_grads(self.s, self.params(), tokens, dtype=self.dtype)
        return loss, gpt.flatten(self.s, g, dtype=self.dtype)

    def step(self, tokens) -> float:
        loss, g = self.grads(tokens)
        s = self.s
        lr = lr_at(s, self.steps_done)
        adamw_update(self.flat, g, self.m, self.v, self.steps_done + 1, lr,
                     s.beta1, s.beta2, s.eps, s.weight_decay)
        self.steps_done += 1
        return float(loss)
