"""Seeded synthetic inputs: token batches, decode prompts and initial weights.

This module holds no model arithmetic; it only draws random inputs.  It is the
one module that both the HIP path's harness and the tests' oracle runs take
their inputs from, so both sides see identical data.

Every draw uses ``numpy.random.default_rng([0, config_id, purpose, step])``:
purpose 0 = initial weights, 1 = the generator's fixed structure (transition
table / permutation), 2 = per-step token batches, 3 = decode prompts.

The pages train on tokenized TinyStories ("Open Flapping Airplanes ... A100
reproduction", "What ran") and on an unnamed text corpus ("Coppelius training
on the RTX 3090", "Run"), neither of which is available; these seeded streams
stand in for them at the same shapes (8 x 512 and 1 x 1024 tokens per step).

* tiny config: first-order Markov chain, each row of the 256 x 256 transition
  table drawn Dirichlet(0.1);
* RoPE config: iid Zipf(1.1) ranks over the vocabulary, token = rank - 1;
* 162M config: order-2 chain x_t = pi[(ha[x_{t-2}] + hb[x_{t-1}] + r - 1) mod V]
  with r ~ Zipf(1.1), pi a seeded permutation and ha, hb in [0, 256)^V.
"""

from __future__ import annotations

import hashlib

import numpy as np

SEED = 0
INIT_STD = 0.02


def rng(config_id: int, purpose: int, step: int = 0) -> np.random.Generator:
    return np.random.default_rng([SEED, int(config_id), int(purpose), int(step)])


# ----------------------------------------------------------------------------
# initial weights
# ----------------------------------------------------------------------------

def init_params(layout, config_id: int) -> np.ndarray:
    """Flat fp32 initial parameters for ``layout`` = [(numel, kind)] in canonical order.

    kind: "normal" -> N(0, 0.02) drawn in fp64 then rounded to fp32; "zeros"; "ones".
    """
    g = rng(config_id, 0)
    parts = []
    for numel, kind in layout:
        if kind == "normal":
            parts.append((g.standard_normal(numel) * INIT_STD).astype(np.float32))
        elif kind == "zeros":
            parts.append(np.zeros(numel, np.float32))
        elif kind == "ones":
            parts.append(np.ones(numel, np.float32))
        else:
            raise ValueError(kind)
    return np.concatenate(parts)


# ----------------------------------------------------------------------------
# token streams
# ----------------------------------------------------------------------------

def _zipf_cdf(V: int, s: float = 1.1) -> np.ndarray:
    k = np.arange(1, V + 1, dtype=np.float64)
    w = k ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def _zipf_ranks(g: np.random.Generator, cdf: np.ndarray, n) -> np.ndarray:
    """Inverse-CDF draw of ranks 1..V."""
    u = g.random(n)
    r = np.searchsorted(cdf, u, side="right") + 1
    return np.minimum(r, cdf.size)


class TokenStream:
    """Seeded token batches [B][T+1] (int32) for one configuration."""

    def __init__(self, kind: str, config_id: int, vocab: int, batch: int, seq: int):
        self.kind, self.cid, self.V, self.B, self.T = kind, config_id, vocab, batch, seq
        g = rng(config_id, 1)
        if kind == "markov1":
            self.table = g.dirichlet(np.full(vocab, 0.1), size=vocab)
            self.cdf = np.cumsum(self.table, axis=1)
            self.cdf /= self.cdf[:, -1:]
        elif kind == "zipf":
            self.zcdf = _zipf_cdf(vocab)
        elif kind == "markov2":
            self.perm = g.permutation(vocab).astype(np.int64)
            self.ha = g.integers(0, 256, size=vocab, dtype=np.int64)
            self.hb = g.integers(0, 256, size=vocab, dtype=np.int64)
            self.zcdf = _zipf_cdf(vocab)
        else:
            raise ValueError(kind)

    def rows(self, purpose: int, step: int, n_rows: int, n_cols: int) -> np.ndarray:
        g = rng(self.cid, purpose, step)
        V = self.V
        out = np.zeros((n_rows, n_cols), np.int64)
        if self.kind == "markov1":
            out[:, 0] = g.integers(0, V, size=n_rows)
            u = g.random((n_rows, n_cols))
            for t in range(1, n_cols):
                c = self.cdf[out[:, t - 1]]
                nxt = (c < u[:, t:t + 1]).sum(axis=1)
                out[:, t] = np.minimum(nxt, V - 1)
        elif self.kind == "zipf":
            out[:] = _zipf_ranks(g, self.zcdf, (n_rows, n_cols)) - 1
        else:
            out[:, :2] = g.integers(0, V, size=(n_rows, 2))
            r = _zipf_ranks(g, self.zcdf, (n_rows, n_cols))
            for t in range(2, n_cols):
                idx = (self.ha[out[:, t - 2]] + self.hb[out[:, t - 1]] + r[:, t] - 1) % V
                out[:, t] = self.perm[idx]
        return out.astype(np.int32)

    def batch(self, step: int) -> np.ndarray:
        """Training batch of step ``step``: [B][T+1] int32."""
        return self.rows(2, step, self.B, self.T + 1)

    def batches(self, first: int, n: int) -> np.ndarray:
        return np.stack([self.batch(first + i) for i in range(n)])

    def prompt(self, length: int) -> np.ndarray:
        """Decode prompt: the first ``length`` tokens of the stream drawn with purpose 3."""
        return self.rows(3, 0, 1, length)[0]

    def prompts(self, n: int, length: int) -> np.ndarray:
        """n decode prompts of ``length`` tokens ([n][length], purpose 3, step 1)."""
        return self.rows(3, 1, n, length)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
