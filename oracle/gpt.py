"""Oracle GPT: forward pass, hand-derived backward pass, loss.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed follows the kernel families of "Coppelius training on the
RTX 3090" ("Where a step's time goes" table: gather, layernorm-forward /
-backward / -parameters, attention-forward, attention-key, attention-query,
qk-rope, inverse-rope-qkv, gated-gelu-forward / -backward, cross-entropy,
cross-entropy-backward, loss-target-gather, embedding-scatter) and the 162M
model of "Open Flapping Airplanes ... A100 reproduction" ("What ran").  The
pages print no formulas; the textbook definitions are written out here.

Readings taken where the pages are silent (each is also listed in the design
notes):

* GELU is the exact erf form u * (1 + erf(u / sqrt 2)) / 2.
* LayerNorm: biased variance over the feature axis, eps = 1e-5, gain and bias.
* Attention: scale 1/sqrt(dh); a query attends to keys at positions <= its own.
* RoPE: rotate-half over the whole head, theta_i = 10000^(-2i/dh), positions
  0..T-1, applied to q and k only.
* Gated MLP: GELU on the gate branch, a = GELU(h W_gate^T) * (h W_up^T).
* Loss: natural-log cross-entropy averaged over all B*T positions; targets are
  the inputs shifted by one.
* Linear weights are stored out x in: y = x W^T (+ b).

All arithmetic is in ``dtype`` (float64 unless the caller asks otherwise).
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
from scipy.special import erf as _erf

LN_EPS = 1e-5
ROPE_BASE = 10000.0


@dataclass(frozen=True)
class Spec:
    n_layer: int
    d_model: int
    n_head: int
    d_ff: int
    vocab: int
    n_pos: int            # learned position table length; 0 means RoPE
    mlp_gated: bool
    tied_head: bool
    has_bias: bool
    batch: int
    seq: int
    lr: float
    beta1: float
    beta2: float
    eps: float
    weight_decay: float
    lr_schedule: str      # "constant" or "cosine"
    total_steps: int

    @property
    def dh(self) -> int:
        return self.d_model // self.n_head

    @property
    def rope(self) -> bool:
        return self.n_pos == 0

    def replace(self, **kw) -> "Spec":
        d = dict(self.__dict__)
        d.update(kw)
        return Spec(**d)


# ----------------------------------------------------------------------------
# parameter layout: canonical order of the flat fp32 parameter vector
# ----------------------------------------------------------------------------

def param_layout(s: Spec):
    """List of (name, shape, init kind) in canonical order.

    init kind: "normal" (N(0, 0.02)), "zeros" or "ones".
    """
    d, F, V = s.d_model, s.d_ff, s.vocab
    out = [("wte", (V, d), "normal")]
    if s.n_pos:
        out.append(("wpe", (s.n_pos, d), "normal"))
    for l in range(s.n_layer):
        p = f"h{l}."
        out.append((p + "ln1.g", (d,), "ones"))
        out.append((p + "ln1.b", (d,), "zeros"))
        out.append((p + "w_qkv", (3 * d, d), "normal"))
        if s.has_bias:
            out.append((p + "b_qkv", (3 * d,), "zeros"))
        out.append((p + "w_o", (d, d), "normal"))
        if s.has_bias:
            out.append((p + "b_o", (d,), "zeros"))
        out.append((p + "ln2.g", (d,), "ones"))
        out.append((p + "ln2.b", (d,), "zeros"))
        if s.mlp_gated:
            out.append((p + "w_gate", (F, d), "normal"))
            out.append((p + "w_up", (F, d), "normal"))
            out.append((p + "w_down", (d, F), "normal"))
        else:
            out.append((p + "w_fc", (F, d), "normal"))
            if s.has_bias:
                out.append((p + "b_fc", (F,), "zeros"))
            out.append((p + "w_proj", (d, F), "normal"))
            if s.has_bias:
                out.append((p + "b_proj", (d,), "zeros"))
    out.append(("lnf.g", (d,), "ones"))
    out.append(("lnf.b", (d,), "zeros"))
    if not s.tied_head:
        out.append(("w_lm", (V, d), "normal"))
    return out


def n_params(s: Spec) -> int:
    return sum(int(np.prod(shape)) for _, shape, _ in param_layout(s))


def unflatten(s: Spec, flat: np.ndarray) -> dict:
    """Views into ``flat`` keyed by parameter name."""
    out, off = {}, 0
    for name, shape, _ in param_layout(s):
        n = int(np.prod(shape))
        out[name] = flat[off:off + n].reshape(shape)
        off += n
    assert off == flat.size, (off, flat.size)
    return out


def flatten(s: Spec, tensors: dict, dtype=np.float64) -> np.ndarray:
    return np.concatenate([np.asarray(tensors[name], dtype=dtype).ravel()
                           for name, _, _ in param_layout(s)])


# ----------------------------------------------------------------------------
# building blocks
# ----------------------------------------------------------------------------

def layer_norm(x, g, b):
    """y = g * (x - mean) / sqrt(var + eps) + b over the last axis (biased var)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + LN_EPS)
    xhat = (x - mu) * rstd
    return xhat * g + b, (xhat, rstd)


def layer_norm_backward(dy, cache, g):
    """Gradient of layer_norm w.r.t. its input, gain and bias.

    With xhat the normalised input and gy = g * dy:
    dx = rstd * (gy - mean(gy) - xhat * mean(gy * xhat)).
    """
    xhat, rstd = cache
    gy = dy * g
    dx = rstd * (gy - gy.mean(axis=-1, keepdims=True)
                 - xhat * (gy * xhat).mean(axis=-1, keepdims=True))
    rows = tuple(range(dy.ndim - 1))
    dg = (dy * xhat).sum(axis=rows)
    db = dy.sum(axis=rows)
    return dx, dg, db


def gelu(u):
    """Exact GELU: u * Phi(u) with Phi the standard normal CDF."""
    return u * 0.5 * (1.0 + _erf(u / math.sqrt(2.0)))


def gelu_grad(u):
    """d/du [u * Phi(u)] = Phi(u) + u * phi(u)."""
    phi = np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)
    return 0.5 * (1.0 + _erf(u / math.sqrt(2.0))) + u * phi


def rope_tables(T: int, dh: int, dtype=np.float64, start: int = 0):
    """cos/sin tables [T][dh/2] for positions start..start+T-1."""
    half = dh // 2
    i = np.arange(half, dtype=np.float64)
    theta = ROPE_BASE ** (-2.0 * i / dh)
    ang = np.arange(start, start + T, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope(x, cos, sin):
    """Rotate-half RoPE on the last axis: pair (i, i + dh/2) turned by pos*theta_i."""
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], axis=-1)


def rope_inverse(x, cos, sin):
    """Transpose (= inverse) of the rotation applied by ``rope``."""
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos + x2 * sin, -x1 * sin + x2 * cos], axis=-1)


def causal_attention(q, k, v):
    """q, k, v: [..., T, dh].  Returns o and the probabilities P."""
    T, dh = q.shape[-2], q.shape[-1]
    s = (q @ np.swapaxes(k, -1, -2)) / math.sqrt(dh)
    future = np.triu(np.ones((T, T), dtype=bool), k=1)   # key position > query
    s = np.where(future, -np.inf, s)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return p @ v, p


def causal_attention_backward(do, q, k, v, p):
    """Gradients of o = softmax(q k^T / sqrt(dh), causal) v."""
    dh = q.shape[-1]
    dv = np.swapaxes(p, -1, -2) @ do
    dp = do @ np.swapaxes(v, -1, -2)
    ds = p * (dp - (dp * p).sum(axis=-1, keepdims=True))
    scale = 1.0 / math.sqrt(dh)
    dq = (ds @ k) * scale
    dk = (np.swapaxes(ds, -1, -2) @ q) * scale
    return dq, dk, dv


def prediction_entropy(z):
    """Entropy in nats of softmax(z) over the last axis: -sum_i p_i log p_i.

    "Coppelius training on the RTX 3090", "Prediction entropy": the next-token
    entropy of a row, ln V when every token is equally likely.
    """
    logp, _ = log_softmax_rows(z)
    return -(np.exp(logp) * logp).sum(axis=-1)


def log_softmax_rows(z):
    m = z.max(axis=-1, keepdims=True)
    lse = m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True))
    return z - lse, lse[..., 0]


# ----------------------------------------------------------------------------
# model
# ----------------------------------------------------------------------------

def _heads(x, B, T, H, dh):
    """[B*T, H*dh] -> [B, H, T, dh]"""
    return x.reshape(B, T, H, dh).transpose(0, 2, 1, 3)


def _unheads(x):
    B, H, T, dh = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B * T, H * dh)


def embed(s: Spec, P: dict, ids, positions):
    x = P["wte"][ids]
    if s.n_pos:
        x = x + P["wpe"][positions]
    return x


def forward(s: Spec, P: dict, tokens, dtype=np.float64, keep=True):
    """Full forward of a [B][T+1] token batch; returns (loss, cache).

    inputs = tokens[:, :T], targets = tokens[:, 1:].
    """
    tokens = np.asarray(tokens)
    B, T1 = tokens.shape
    T = T1 - 1
    d, H, dh = s.d_model, s.n_head, s.dh
    P = {k: np.asarray(v, dtype=dtype) for k, v in P.items()}
    ids, tgt = tokens[:, :T], tokens[:, 1:]
    x = embed(s, P, ids, np.arange(T)).reshape(B * T, d)
    cos = sin = None
    if s.rope:
        cos, sin = rope_tables(T, dh, dtype)
    layers = []
    for l in range(s.n_layer):
        p = f"h{l}."
        c = {"x_in": x}
        h, c["ln1"] = layer_norm(x, P[p + "ln1.g"], P[p + "ln1.b"])
        c["h"] = h
        qkv = h @ P[p + "w_qkv"].T
        if s.has_bias:
            qkv = qkv + P[p + "b_qkv"]
        q = _heads(qkv[:, :d], B, T, H, dh)
        k = _heads(qkv[:, d:2 * d], B, T, H, dh)
        v = _heads(qkv[:, 2 * d:], B, T, H, dh)
        if s.rope:
            q, k = rope(q, cos, sin), rope(k, cos, sin)
        o, pr = causal_attention(q, k, v)
        c.update(q=q, k=k, v=v, p=pr)
        o = _unheads(o)
        c["o"] = o
        y = o @ P[p + "w_o"].T
        if s.has_bias:
            y = y + P[p + "b_o"]
        x = x + y
        c["x_mid"] = x
        h2, c["ln2"] = layer_norm(x, P[p + "ln2.g"], P[p + "ln2.b"])
        c["h2"] = h2
        if s.mlp_gated:
            g = h2 @ P[p + "w_gate"].T
            up = h2 @ P[p + "w_up"].T
            a = gelu(g) * up
            c.update(g=g, up=up, a=a)
            y = a @ P[p + "w_down"].T
        else:
            u = h2 @ P[p + "w_fc"].T
            if s.has_bias:
                u = u + P[p + "b_fc"]
            a = gelu(u)
            c.update(u=u, a=a)
            y = a @ P[p + "w_proj"].T
            if s.has_bias:
                y = y + P[p + "b_proj"]
        x = x + y
        layers.append(c if keep else None)
    hf, lnf = layer_norm(x, P["lnf.g"], P["lnf.b"])
    w_lm = P["wte"] if s.tied_head else P["w_lm"]
    z = hf @ w_lm.T
    logp, lse = log_softmax_rows(z)
    y_flat = tgt.reshape(-1)
    nll = -logp[np.arange(B * T), y_flat]
    loss = nll.mean()
    cache = dict(B=B, T=T, ids=ids, tgt=y_flat, layers=layers, x_final=x,
                 hf=hf, lnf=lnf, z=z, logp=logp, nll=nll, cos=cos, sin=sin, P=P)
    return loss, cache


def backward(s: Spec, cache: dict) -> dict:
    """Hand-derived gradient of the mean loss w.r.t. every parameter."""
    P = cache["P"]
    B, T = cache["B"], cache["T"]
    BT = B * T
    d, H, dh = s.d_model, s.n_head, s.dh
    grads = {name: np.zeros(shape, dtype=P["wte"].dtype) for name, shape, _ in param_layout(s)}

    # softmax cross-entropy: dz = (softmax(z) - onehot(y)) / BT
    dz = np.exp(cache["logp"])
    dz[np.arange(BT), cache["tgt"]] -= 1.0
    dz /= BT
    hf = cache["hf"]
    if s.tied_head:
        grads["wte"] += dz.T @ hf
        dhf = dz @ P["wte"]
    else:
        grads["w_lm"] = dz.T @ hf
        dhf = dz @ P["w_lm"]
    dx, grads["lnf.g"], grads["lnf.b"] = layer_norm_backward(dhf, cache["lnf"], P["lnf.g"])

    for l in reversed(range(s.n_layer)):
        p = f"h{l}."
        c = cache["layers"][l]
        # MLP branch: x_out = x_mid + mlp(LN2(x_mid))
        if s.mlp_gated:
            grads[p + "w_down"] = dx.T @ c["a"]
            da = dx @ P[p + "w_down"]
            dg = da * c["up"] * gelu_grad(c["g"])
            dup = da * gelu(c["g"])
            grads[p + "w_gate"] = dg.T @ c["h2"]
            grads[p + "w_up"] = dup.T @ c["h2"]
            dh2 = dg @ P[p + "w_gate"] + dup @ P[p + "w_up"]
        else:
            if s.has_bias:
                grads[p + "b_proj"] = dx.sum(axis=0)
            grads[p + "w_proj"] = dx.T @ c["a"]
            da = dx @ P[p + "w_proj"]
            du = da * gelu_grad(c["u"])
            if s.has_bias:
                grads[p + "b_fc"] = du.sum(axis=0)
            grads[p + "w_fc"] = du.T @ c["h2"]
            dh2 = du @ P[p + "w_fc"]
        dln, grads[p + "ln2.g"], grads[p + "ln2.b"] = layer_norm_backward(dh2, c["ln2"], P[p + "ln2.g"])
        dx = dx + dln
        # attention branch: x_mid = x_in + attn(LN1(x_in))
        if s.has_bias:
            grads[p + "b_o"] = dx.sum(axis=0)
        grads[p + "w_o"] = dx.T @ c["o"]
        do = _heads(dx @ P[p + "w_o"], B, T, H, dh)
        dq, dk, dv = causal_attention_backward(do, c["q"], c["k"], c["v"], c["p"])
        if s.rope:
            dq = rope_inverse(dq, cache["cos"], cache["sin"])
            dk = rope_inverse(dk, cache["cos"], cache["sin"])
        dqkv = np.concatenate([_unheads(dq), _unheads(dk), _unheads(dv)], axis=1)
        if s.has_bias:
            grads[p + "b_qkv"] = dqkv.sum(axis=0)
        grads[p + "w_qkv"] = dqkv.T @ c["h"]
        dh1 = dqkv @ P[p + "w_qkv"]
        dln, grads[p + "ln1.g"], grads[p + "ln1.b"] = layer_norm_backward(dh1, c["ln1"], P[p + "ln1.g"])
        dx = dx + dln

    # embedding: scatter-add rows of dx into the token table; sum over batch for positions
    dx3 = dx.reshape(B, T, d)
    np.add.at(grads["wte"], cache["ids"].reshape(-1), dx)
    if s.n_pos:
        grads["wpe"][:T] += dx3.sum(axis=0)
    return grads


def loss_and_grads(s: Spec, P: dict, tokens, dtype=np.float64):
    loss, cache = forward(s, P, tokens, dtype=dtype)
    return loss, backward(s, cache)


# ----------------------------------------------------------------------------
# single-sequence logits (used by the decode oracle)
# ----------------------------------------------------------------------------

def sequence_logits(s: Spec, P: dict, seq_tokens, dtype=np.float64):
    """Logits [n][V] for every position of one sequence placed at positions 0..n-1.

    Because attention is causal, row t depends only on tokens 0..t, so row t is
    exactly the next-token logits a decoder computes after seeing tokens 0..t.
    """
    seq_tokens = np.asarray(seq_tokens).reshape(1, -1)
    padded = np.concatenate([seq_tokens, seq_tokens[:, -1:]], axis=1)  # dummy target
    _, cache = forward(s, P, padded, dtype=dtype, keep=False)
    return cache["z"]
