"""Benchmark: training tokens/s of the 162M GPT step (forward, backward, AdamW)
on one MI355X, plus batch-1 greedy decode tokens/s of the same model.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--exec-mode persistent|per_phase]

Prints ONE JSON line.  Workload: the 162M GPT-2-small-shaped model (12 layers,
width 768, 12 heads, MLP 3072, learned positions 512, vocabulary 50,304, untied
head) on 8 x 512 = 4,096 synthetic tokens per step (seeded order-2 Markov
chain), bf16 operands with fp32 master weights -- the shape of the 162M run on
the "Open Flapping Airplanes ... A100 reproduction" page ("What ran").  Inputs
are resident in HBM before the timed region starts.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15   # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12    # MI355X HBM3E, bytes/s


def model_flops_per_step(c: dict) -> dict:
    """Algorithmic FLOPs of one training step: 6 * matmul params * tokens + causal attention."""
    d, F, V, L, B, T, H = c["d_model"], c["d_ff"], c["vocab"], c["n_layer"], c["batch"], c["seq"], c["n_head"]
    mlp = (3 if c["mlp_gated"] else 2) * d * F
    matmul_params = L * (4 * d * d + mlp) + V * d
    tokens = B * T
    gemm = 6.0 * matmul_params * tokens
    dh = d // H
    attn_fwd = L * B * H * 2.0 * T * T * dh   # QK^T and PV over the causal half
    return {"gemm": gemm, "attention": 3.0 * attn_fwd, "total": gemm + 3.0 * attn_fwd,
            "matmul_params": matmul_params}


def decode_bytes_per_token(c: dict, ctx: float) -> float:
    """Weights read per decoded token (bf16) + KV cache read at context length ctx."""
    d, F, V, L = c["d_model"], c["d_ff"], c["vocab"], c["n_layer"]
    per_layer = (3 * d * d + 3 * d) + (d * d + d) + 2 * d + (2 * d * F + F + d) + 2 * d
    weights = L * per_layer + V * d + 2 * d + (c["n_pos"] and d)   # blocks + head + lnf + one wte/wpe row
    kv = L * 2 * d * ctx
    return 2.0 * (weights + kv)


def kernel_sources_sha256() -> str:
    import hashlib
    src = os.path.join(ROOT, "persistent_transformer_train_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(src)):
        if name.endswith((".h", ".hip", ".cpp")):
            with open(os.path.join(src, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(profile: str):
    """HBM-side bytes per training step of the persistent kernel, from the
    FETCH_SIZE / WRITE_SIZE passes recorded in the committed profile summary,
    scaled by the same counters' reading for a plain copy of known size.  None
    when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", profile)
    try:
        with open(path) as f:
            for line in f:
                if line.startswith("traffic: "):
                    rec = json.loads(line[len("traffic: "):])
                    if rec.get("sources_sha256") == kernel_sources_sha256():
                        return rec["bytes_per_step"]
    except (OSError, ValueError, KeyError):
        pass
    return None


def oracle_spec(cfg: dict):
    """The oracle's description of the benchmarked model (test infrastructure: used
    only by the CPU baselines)."""
    from oracle import gpt
    from persistent_transformer_train_amd import configs
    return gpt.Spec(n_layer=cfg["n_layer"], d_model=cfg["d_model"], n_head=cfg["n_head"], d_ff=cfg["d_ff"],
                    vocab=cfg["vocab"], n_pos=cfg["n_pos"], mlp_gated=bool(cfg["mlp_gated"]),
                    tied_head=bool(cfg["tied_head"]), has_bias=bool(cfg["has_bias"]), batch=cfg["batch"],
                    seq=cfg["seq"], lr=cfg["lr"], beta1=cfg["beta1"], beta2=cfg["beta2"], eps=cfg["eps"],
                    weight_decay=cfg["weight_decay"],
                    lr_schedule="cosine" if cfg["lr_schedule"] == configs.LR_COSINE else "constant",
                    total_steps=cfg["total_steps"])


def cpu_baseline(cfg: dict) -> dict:
    """The oracle (numpy, untuned) on one full training step of the same workload:
    the 162M model on all 8 x 512 = 4,096 tokens of a step (forward, hand-derived
    backward, AdamW), in float32 as the parity runs use it, on the host's cores."""
    from oracle import gpt, optim
    from persistent_transformer_train_amd import synth
    spec = oracle_spec(cfg)
    lay = gpt.param_layout(spec)
    init = synth.init_params([(int(np.prod(sh)), k) for _, sh, k in lay], 3)
    stream = synth.TokenStream("markov2", 3, cfg["vocab"], cfg["batch"], cfg["seq"])
    tr = optim.Trainer(spec, init, dtype=np.float32)
    t0 = time.perf_counter()
    tr.step(stream.batch(0))
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    tokens = cfg["batch"] * cfg["seq"]
    return {"value": round(tokens / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"one float32 training step (forward, backward, AdamW) of the 162M model on the full "
                      f"{cfg['batch']} x {cfg['seq']} = {tokens}-token batch: {dt:.2f} s; numpy BLAS threads = "
                      f"the {cores} cores of the process's affinity"}


def cpu_baseline_decode(cfg: dict, init, stream, n_tok: int = 4) -> dict:
    """The oracle's batch-1 greedy decode of the same model: every token by a full
    causal forward of its whole context (the oracle keeps no KV cache), float32,
    on the host's cores; n_tok tokens from a context of the decode run's average
    length ((prompt + window) / 2 = 272 tokens of the seeded prompt chain)."""
    from oracle import decode, gpt
    from persistent_transformer_train_amd import configs
    spec = oracle_spec(cfg)
    P = gpt.unflatten(spec, np.asarray(init, np.float32))
    dcfg = configs.get("c4")
    n_ctx = (dcfg["prompt_len"] + dcfg["decode_window"]) // 2
    ctx = stream.prompt(n_ctx)
    t0 = time.perf_counter()
    decode.greedy(spec, P, ctx, n_tok, dcfg["decode_window"], dcfg["prompt_len"], dtype=np.float32)
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    return {"value": round(n_tok / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_tok} greedy tokens from a {n_ctx}-token context (the decode run's average), each by a "
                      f"full float32 forward of its context (no KV cache): {dt:.2f} s; numpy BLAS threads = the "
                      f"{cores} cores"}


def bench_decode(init, stream, args) -> dict:
    """Batch-1 greedy decode of the frozen seeded weights (version 0, published at
    create) on the serve CUs: a 32-token prompt, then decode_tokens tokens; the
    first call (prompt prefill + first token) is not timed."""
    import torch
    from persistent_transformer_train_amd import configs, ofa
    dcfg = configs.get("c4", exec_mode=0 if args.exec_mode == "persistent" else 1)
    h = ofa.Handle(dcfg, init)
    prompt = torch.from_numpy(stream.prompt(dcfg["prompt_len"])).cuda()
    n = args.decode_tokens
    toks = torch.zeros(n, dtype=torch.int32, device="cuda")
    h.decode(prompt, 1, toks)
    h.sync()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    h.decode(None, n - 1, toks[1:])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    st = h.sync()
    h.close()
    rate = (n - 1) / dt
    avg_ctx = (dcfg["prompt_len"] + dcfg["decode_window"]) / 2
    bpt = decode_bytes_per_token(dcfg, avg_ctx)
    ceiling = read_ceiling(dcfg["serve_cus"], bpt)
    return {"metric": "batch-1 greedy decode tokens/s", "value": round(rate, 1), "unit": "tokens/s",
            "tokens": n - 1, "prompt": dcfg["prompt_len"], "window": dcfg["decode_window"],
            "cus": dcfg["serve_cus"] if args.exec_mode == "persistent" else "all (launch per phase)",
            "kernel_ms": round(st.last_call_ms, 3),
            "roofline": {"bound": "hbm", "achieved": round(bpt * rate / 1e9, 1), "peak": PEAK_HBM / 1e9,
                         "unit": "GB/s", "frac": round(bpt * rate / PEAK_HBM, 4), "bytes_per_token": bpt},
            "read_ceiling": dict(ceiling, frac=round(bpt * rate / 1e9 / ceiling["GBps"], 4))}


def read_ceiling(n_wg: int, nbytes: float) -> dict:
    """The streaming-read ceiling of the decode weight stream on n_wg workgroups
    (ofa_read_ceiling): a buffer of the token's bytes, copied through LDS as the
    GEMV tickets copy their weights."""
    import torch
    from persistent_transformer_train_amd import ofa
    buf = torch.zeros(int(nbytes) // 16 * 16, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(n_wg, dtype=torch.int32, device="cuda")
    gbps, us = ofa.read_ceiling(n_wg, buf, sink, reps=5)
    del buf
    return {"workgroups": n_wg, "bytes": int(nbytes), "GBps": round(gbps, 1), "best_us": round(us, 1),
            "tokens_per_s_at_ceiling": round(gbps * 1e9 / nbytes, 1)}


def bench_decode_batch(init, stream, args, nseq: int = 8) -> dict:
    """Serving variant: nseq prompts of 32 tokens decoded together on the 48 serve
    CUs (each weight tile streamed once per position for all sequences); the
    first call (prefill + first token) is not timed.  Aggregate tokens/s."""
    import torch
    from persistent_transformer_train_amd import configs, ofa
    dcfg = configs.get("c4", decode_batch=nseq, exec_mode=0 if args.exec_mode == "persistent" else 1)
    h = ofa.Handle(dcfg, init)
    prompts = torch.from_numpy(stream.prompts(nseq, dcfg["prompt_len"])).cuda().contiguous()
    n = args.decode_tokens
    toks = torch.zeros(n, nseq, dtype=torch.int32, device="cuda")
    h.decode(prompts, 1, toks)
    h.sync()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    h.decode(None, n - 1, toks[1:])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    st = h.sync()
    h.close()
    avg_ctx = (dcfg["prompt_len"] + dcfg["decode_window"]) / 2
    one = decode_bytes_per_token(dcfg, avg_ctx)
    kv = 2.0 * dcfg["n_layer"] * 2 * dcfg["d_model"] * avg_ctx
    bytes_per_position = one + (nseq - 1) * kv   # weights once, every sequence's KV
    return {"metric": f"batch-{nseq} greedy decode tokens/s (all sequences)", "value": round(nseq * (n - 1) / dt, 1),
            "unit": "tokens/s", "sequences": nseq, "positions": n - 1, "kernel_ms": round(st.last_call_ms, 3),
            "roofline": {"bound": "hbm", "achieved": round(bytes_per_position * (n - 1) / dt / 1e9, 1),
                         "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                         "frac": round(bytes_per_position * (n - 1) / dt / PEAK_HBM, 4)}}


def bench_doorbell(init, stream, args, n_new: int = 64) -> dict:
    """Host doorbell to wake-up: a batch-1 decode of the c4 model on the 48 serve CUs
    in which the host rings for every token; per token, the host clock's ring-to-token
    time and the device clock's wake-to-token time (their difference: the doorbell's
    trip to the device plus the progress word's trip back)."""
    import torch
    from persistent_transformer_train_amd import configs, ofa
    dcfg = configs.get("c4")
    h = ofa.Handle(dcfg, init)
    prompt = torch.from_numpy(stream.prompt(dcfg["prompt_len"])).cuda()
    toks = torch.zeros(n_new, dtype=torch.int32, device="cuda")
    host_us, dev_us = h.decode_doorbell(prompt, n_new, toks)
    h.close()
    host_us, dev_us = np.array(host_us[1:]), np.array(dev_us[1:])   # the first token includes the prefill
    trip = host_us - dev_us
    return {"metric": "host doorbell to token (batch-1 decode, c4 model, 48 CUs)", "tokens": n_new - 1,
            "ring_to_token_us": {"median": round(float(np.median(host_us)), 1), "max": round(float(host_us.max()), 1)},
            "device_wake_to_token_us": {"median": round(float(np.median(dev_us)), 1), "max": round(float(dev_us.max()), 1)},
            "doorbell_round_trip_us": {"median": round(float(np.median(trip)), 1), "max": round(float(trip.max()), 1)}}


def bench_coresident(init, stream, args) -> dict:
    """c5: the training step on 208 CUs and batch-1 decode on 48 CUs in one
    persistent launch; decode restarts from the seeded prompt every 512 tokens
    and reads the weights each AdamW step publishes.  Both rates over the call."""
    import torch
    from persistent_transformer_train_amd import configs, ofa
    cfg = configs.get("c5")
    h = ofa.Handle(cfg, init)
    BT = cfg["batch"] * cfg["seq"]
    n = args.co_steps
    toks = torch.from_numpy(stream.batches(0, n)).cuda()
    losses = torch.zeros(n, dtype=torch.float32, device="cuda")
    prompt = torch.from_numpy(stream.prompt(cfg["prompt_len"])).cuda()
    ring = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    vers = torch.zeros(1 << 16, dtype=torch.int64, device="cuda")
    n_gen = torch.zeros(1, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    h.train_and_serve(toks, losses, prompt, ring, vers, n_gen)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    st = h.sync()
    g = int(n_gen.item())
    v = vers[:min(g, ring.numel())].cpu().numpy()
    ls = losses.cpu().numpy()
    h.close()
    return {"metric": "co-resident train tokens/s and decode tokens/s in one persistent launch",
            "train_value": round(n * BT / dt, 1), "decode_value": round(g / dt, 1), "unit": "tokens/s",
            "steps": n, "tokens_generated": g, "seconds": round(dt, 4), "kernel_ms": round(st.last_call_ms, 3),
            "train_cus": cfg["train_cus"], "serve_cus": cfg["serve_cus"], "restart_every": cfg["restart_every"],
            "versions_read": [int(v.min()), int(v.max()), int(len(np.unique(v)))] if g else None,
            "losses": [float(ls[0]), float(ls[-1])]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--exec-mode", choices=["persistent", "per_phase"], default="persistent")
    ap.add_argument("--decode-tokens", type=int, default=512)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--co-steps", type=int, default=40, help="co-resident (c5) training steps; 0 = skip")
    ap.add_argument("--dump-phases", default="", help="write the training program's phase names (launch order) here")
    ap.add_argument("--debug-flags", type=int, default=0, help="OFA_DEBUG_* bits for the training handle (experiments)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(collectives and sharding are design-only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from persistent_transformer_train_amd import configs, ofa, synth

    cfg = configs.get("c3", exec_mode=0 if args.exec_mode == "persistent" else 1, debug_flags=args.debug_flags)
    lay = ofa.layout(ofa.make_config(cfg))
    init = synth.init_params([(n, k) for _, _, n, k in lay], 3)
    stream = synth.TokenStream("markov2", 3, cfg["vocab"], cfg["batch"], cfg["seq"])
    h = ofa.Handle(cfg, init)
    BT = cfg["batch"] * cfg["seq"]
    W, K = args.warmup, args.steps
    toks_w = torch.from_numpy(stream.batches(0, max(W, 1))).cuda()
    toks_k = torch.from_numpy(stream.batches(W, K)).cuda()
    losses = torch.zeros(max(W, K, 1), dtype=torch.float32, device="cuda")
    if W:
        h.train_step(toks_w, losses)
        h.sync()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    h.train_step(toks_k, losses)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    st = h.sync()
    kernel_ms = st.last_call_ms   # HIP events around the launch(es) on the handle's stream
    if args.dump_phases:
        with open(args.dump_phases, "w") as f:
            json.dump([nm for nm, _, _ in h.phase_times()], f)
    ls = losses[:K].cpu().numpy()
    assert np.all(np.isfinite(ls)), ls

    fl = model_flops_per_step(cfg)
    value = K * BT / elapsed
    achieved = fl["total"] * K / (kernel_ms / 1e3)
    out = {
        "metric": "train tokens/s for 162M GPT step (fwd+bwd+AdamW); batch-1 decode tokens/s",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(elapsed * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / 24772.0, 3),
        "baseline_ref": "24,772 tokens/s: A100 SXM4 40 GB, 85 training SMs (A100 reproduction page, "
                        "'Measured results' table); context only, another machine",
        "dtype": "bf16",
        "data": "synthetic (seeded order-2 Markov chain, Zipf(1.1) transitions); random N(0,0.02) init",
        "config": {"workload": "162M GPT-2-small-shaped training step: 12 layers, width 768, 12 heads, "
                               "MLP 3072 GELU, 512 learned positions, vocab 50304, untied head; bf16 operands, "
                               "fp32 master weights and AdamW state",
                   "global_batch": cfg["batch"], "seq_len": cfg["seq"], "tokens_per_step": BT,
                   "executor": args.exec_mode, "params": int(ofa.ofa_param_count(ofa.make_config(cfg)))},
        "roofline": {"bound": "mfma", "kernel": "persistent_kernel" if args.exec_mode == "persistent"
                     else "all phase kernels", "achieved": round(achieved / 1e12, 2), "peak": PEAK_BF16 / 1e12,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16, 4),
                     "traffic": measured_traffic("persistent_kernel_c3_train.md") if args.exec_mode == "persistent" else None,
                     "flops_per_step": fl["total"], "kernel_ms_per_step": round(kernel_ms / K, 4)},
        "losses": [float(ls[0]), float(ls[-1])],
    }

    h.close()
    if not args.no_decode and args.decode_tokens > 1:
        out["decode"] = bench_decode(init, stream, args)
        out["decode_batch"] = bench_decode_batch(init, stream, args)
        if args.exec_mode == "persistent":
            out["doorbell"] = bench_doorbell(init, stream, args)
    if args.co_steps > 0 and args.exec_mode == "persistent":
        out["coresident"] = bench_coresident(init, stream, args)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
        if "decode" in out:
            out["decode"]["cpu_baseline"] = cpu_baseline_decode(cfg, init, stream)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
