"""Writes the oracle's own free-running fp32 loss trajectories of the full-size
bf16 workloads, the expected values of the free-running parity test.

Calls only ``oracle/`` and the seeded input generators (``synth``), never the
HIP library.  For each workload the oracle starts from the seeded fp32 initial
weights, trains ``--steps`` steps in float32 on the seeded token batches of
steps 0, 1, 2, ... (a fresh batch every step) and records each step's mean
cross-entropy.  The GPU runs the same inputs in bf16 mode and must stay within
2e-2 of this trajectory at every step (reading A19: the oracle follows its own
trajectory, it is not synced to the GPU's weights).

    python tests/golden/make_free_running.py c2 c3 [--steps 100]
    python tests/golden/make_free_running.py c3 --steps 66 --bf16-init

Output: tests/golden/<name>_fp32_free_running.txt, one "step loss" line per
step after a header recording the input fingerprints (SHA-256 of the initial
weights and of the first token batch).

With --bf16-init the same fp32 training starts from the initial weights
rounded to bf16 (nearest even), a change of the order of one rounding of the
bf16 path; the output, <name>_fp32_bf16init_free_running.txt, shows how far the
trajectory itself moves under such a change (the free-running bar's limit).
"""

from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import gpt, optim                      # noqa: E402
from oracle.configs import ORACLE_CONFIGS          # noqa: E402
from persistent_transformer_train_amd import synth  # noqa: E402  (seeded inputs only)

# token stream kind and id of each workload (the same ids the input module documents)
STREAMS = {"c2": ("zipf", 2), "c3": ("markov2", 3)}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 (ties to even), as fp32."""
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return r.astype(np.uint32).view(np.float32)


def run(name: str, steps: int, bf16_init: bool = False) -> None:
    spec = ORACLE_CONFIGS[name]
    kind, cid = STREAMS[name]
    layout = [(int(np.prod(shape)), k) for _, shape, k in gpt.param_layout(spec)]
    init = synth.init_params(layout, cid)
    if bf16_init:
        init = round_bf16(init)
    stream = synth.TokenStream(kind, cid, spec.vocab, spec.batch, spec.seq)
    tr = optim.Trainer(spec, init, dtype=np.float32)
    path = os.path.join(HERE, f"{name}_fp32_{'bf16init_' if bf16_init else ''}free_running.txt")
    tmp = path + ".partial"
    with open(tmp, "w") as f:
        f.write(f"# oracle fp32 free-running loss trajectory of {name} ({steps} steps)"
                f"{' from the bf16-rounded initial weights' if bf16_init else ''}\n")
        f.write(f"# written by tests/golden/make_free_running.py (oracle + seeded inputs only)\n")
        f.write(f"# init sha256 {synth.sha256(init)}\n")
        f.write(f"# batch0 sha256 {synth.sha256(stream.batch(0))}\n")
        for s in range(steps):
            t0 = time.perf_counter()
            loss = tr.step(stream.batch(s))
            f.write(f"{s} {loss:.9g}\n")
            f.flush()
            print(f"{name} step {s}: loss {loss:.6f} ({time.perf_counter() - t0:.1f} s)", flush=True)
    os.replace(tmp, path)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("names", nargs="+", choices=sorted(STREAMS))
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--bf16-init", action="store_true", help="start from the initial weights rounded to bf16")
    a = ap.parse_args()
    for n in a.names:
        run(n, a.steps, a.bf16_init)


if __name__ == "__main__":
    main()
