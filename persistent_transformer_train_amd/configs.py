"""Registry of the five workload configurations (plain values for ofa_config).

c1  tiny GPT, fp32 (correctness case)
c2  57.7M RoPE + gated-GELU GPT, tied head, bf16 with fp32 master weights, 1 x 1024 tokens
    ("Coppelius training on the RTX 3090", "Run": 16 blocks, width 512, 8 heads,
    context 1024, FFN 1408, vocab 12288)
c3  162M GPT-2-small shape, bf16 with fp32 master weights, 8 x 512 tokens
    ("Open Flapping Airplanes ... A100 reproduction", "What ran": 12 layers, width 768,
    12 heads, 8 sequences of 512 tokens)
c4  batch-1 greedy decode of the c3 model (frozen seeded weights), 32-token prompt,
    512 generated tokens, 48 of 256 CUs
c5  c3 training and c4 decode co-resident in one persistent kernel (208 + 48 CUs)
"""

from __future__ import annotations

import copy

FP32, BF16 = 0, 1
LR_CONSTANT, LR_COSINE = 0, 1
EXEC_PERSISTENT, EXEC_LAUNCH_PER_PHASE = 0, 1

_BASE = dict(
    n_layer=0, d_model=0, n_head=0, d_ff=0, vocab=0, n_pos=0,
    mlp_gated=0, tied_head=0, has_bias=1, batch=1, seq=1, precision=FP32,
    lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1,
    lr_schedule=LR_CONSTANT, total_steps=1,
    train_cus=0, serve_cus=0, decode_window=0, prompt_len=0, restart_every=0,
    exec_mode=EXEC_PERSISTENT, debug_counter_base=0, debug_flags=0, decode_batch=0,
)


def _cfg(**kw):
    d = dict(_BASE)
    d.update(kw)
    return d


CONFIGS = {
    "c1": _cfg(n_layer=2, d_model=64, n_head=4, d_ff=256, vocab=256, n_pos=64,
               batch=4, seq=64, precision=FP32, lr=1e-3, lr_schedule=LR_CONSTANT, total_steps=10,
               decode_window=64, prompt_len=8),
    "c2": _cfg(n_layer=16, d_model=512, n_head=8, d_ff=1408, vocab=12288, n_pos=0,
               mlp_gated=1, tied_head=1, has_bias=0, batch=1, seq=1024, precision=BF16,
               lr=6e-4, lr_schedule=LR_COSINE, total_steps=2000, decode_window=1024, prompt_len=32),
    "c3": _cfg(n_layer=12, d_model=768, n_head=12, d_ff=3072, vocab=50304, n_pos=512,
               batch=8, seq=512, precision=BF16, lr=6e-4, lr_schedule=LR_COSINE, total_steps=4000,
               decode_window=512, prompt_len=32),
}
CONFIGS["c4"] = _cfg(**{**CONFIGS["c3"], "serve_cus": 48})
CONFIGS["c5"] = _cfg(**{**CONFIGS["c3"], "train_cus": 208, "serve_cus": 48, "restart_every": 512})

# token-stream kind and id per configuration (see synth.py)
STREAMS = {"c1": ("markov1", 1), "c2": ("zipf", 2), "c3": ("markov2", 3), "c4": ("markov2", 3), "c5": ("markov2", 3)}

DECODE = {"c4": dict(prompt_len=32, n_new=512), "c5": dict(prompt_len=32, n_new=512)}


def get(name: str, **overrides) -> dict:
    d = copy.deepcopy(CONFIGS[name])
    d.update(overrides)
    return d
