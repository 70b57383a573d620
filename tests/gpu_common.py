"""Helpers shared by the GPU parity tests (imported by tests only)."""

from __future__ import annotations

import sys

import numpy as np

from oracle import gpt
from persistent_transformer_train_amd import configs, synth


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def spec_from_cfg(c: dict) -> gpt.Spec:
    return gpt.Spec(n_layer=c["n_layer"], d_model=c["d_model"], n_head=c["n_head"], d_ff=c["d_ff"],
                    vocab=c["vocab"], n_pos=c["n_pos"], mlp_gated=bool(c["mlp_gated"]),
                    tied_head=bool(c["tied_head"]), has_bias=bool(c["has_bias"]), batch=c["batch"],
                    seq=c["seq"], lr=c["lr"], beta1=c["beta1"], beta2=c["beta2"], eps=c["eps"],
                    weight_decay=c["weight_decay"],
                    lr_schedule="cosine" if c["lr_schedule"] == configs.LR_COSINE else "constant",
                    total_steps=c["total_steps"])


# small bf16 models with every feature and ragged sizes (rows, columns and K
# not multiples of the 128-wide tiles)
MINI = {
    # RoPE + gated GELU + tied head, no biases
    "m2": configs._cfg(n_layer=2, d_model=128, n_head=2, d_ff=344, vocab=1000, n_pos=0, mlp_gated=1,
                       tied_head=1, has_bias=0, batch=1, seq=200, precision=configs.BF16, lr=6e-4,
                       lr_schedule=configs.LR_COSINE, total_steps=2000, decode_window=96, prompt_len=16),
    # learned positions + GELU + untied head + biases
    "m3": configs._cfg(n_layer=2, d_model=128, n_head=2, d_ff=512, vocab=1000, n_pos=128, mlp_gated=0,
                       tied_head=0, has_bias=1, batch=2, seq=100, precision=configs.BF16, lr=6e-4,
                       lr_schedule=configs.LR_COSINE, total_steps=4000, decode_window=128, prompt_len=16),
}
# learned positions with batch*seq a multiple of 64: every GEMM (weight gradients
# included) takes the pipelined tile; vocabulary still ragged against the tiles
MINI["m3b"] = dict(MINI["m3"], seq=128)
STREAM_OF = {"m2": ("zipf", 12), "m3": ("markov2", 13), "m3b": ("markov2", 14)}


def cfg_of(name: str, **kw) -> dict:
    if name in MINI:
        d = dict(MINI[name])
        d.update(kw)
        return d
    return configs.get(name, **kw)


def stream_of(name: str, cfg: dict) -> synth.TokenStream:
    kind, cid = STREAM_OF.get(name) or configs.STREAMS[name]
    return synth.TokenStream(kind, cid, cfg["vocab"], cfg["batch"], cfg["seq"])


def init_of(name: str, cfg: dict):
    from persistent_transformer_train_amd import ofa
    lay = ofa.layout(ofa.make_config(cfg))
    cid = (STREAM_OF.get(name) or configs.STREAMS[name])[1]
    return synth.init_params([(n, k) for _, _, n, k in lay], cid)


def cosine(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-300))


def rel_err(a, b) -> float:
    """||a - b|| / ||b|| in float64 (0 when both are zero)."""
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def per_tensor_rel_err(layout, g_gpu, g_or):
    """{tensor name: relative error} over the canonical layout."""
    return {n: rel_err(g_gpu[o:o + k], g_or[o:o + k]) for n, o, k, _ in layout}
