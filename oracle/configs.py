"""The oracle's own table of the five workload configurations.

Kept separate from the product's registry on purpose: a test asserts the two
agree, so a typo in either one is caught.

Shapes follow "Open Flapping Airplanes ... A100 reproduction", section "What
ran" (12 layers, width 768, 12 heads, 8 x 512 tokens per step) and
"Coppelius training on the RTX 3090", section "Run" (16 blocks, width 512,
8 heads, context 1024, FFN 1408, vocab 12288).  The tiny fp32 configuration is
a correctness case of the same architecture.
"""

from .gpt import Spec

ORACLE_CONFIGS = {
    # tiny GPT, fp32: the case the oracle finishes in well under a second
    "c1": Spec(n_layer=2, d_model=64, n_head=4, d_ff=256, vocab=256, n_pos=64,
               mlp_gated=False, tied_head=False, has_bias=True,
               batch=4, seq=64, lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8,
               weight_decay=0.1, lr_schedule="constant", total_steps=10),
    # 57.7M RoPE + gated-GELU GPT, tied head, no biases, one 1024-token context
    "c2": Spec(n_layer=16, d_model=512, n_head=8, d_ff=1408, vocab=12288, n_pos=0,
               mlp_gated=True, tied_head=True, has_bias=False,
               batch=1, seq=1024, lr=6e-4, beta1=0.9, beta2=0.95, eps=1e-8,
               weight_decay=0.1, lr_schedule="cosine", total_steps=2000),
    # 162M GPT-2-small shape, learned positions, untied head
    "c3": Spec(n_layer=12, d_model=768, n_head=12, d_ff=3072, vocab=50304, n_pos=512,
               mlp_gated=False, tied_head=False, has_bias=True,
               batch=8, seq=512, lr=6e-4, beta1=0.9, beta2=0.95, eps=1e-8,
               weight_decay=0.1, lr_schedule="cosine", total_steps=4000),
}
