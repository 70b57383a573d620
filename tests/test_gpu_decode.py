"""GPU parity of batch-1 greedy decode against the oracle's full recomputation.

Teacher forcing: the oracle recomputes the logits along the GPU's own token
sequence; the GPU token must equal the oracle argmax wherever the oracle's
top-2 margin exceeds 1e-2.  Small windows force the context-restart rule.
"""

import numpy as np
import pytest

from gpu_common import cfg_of, init_of, log, spec_from_cfg, stream_of
from oracle import decode, gpt

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def run_decode(name, n_new, exec_mode=1, publish=True, **kw):
    from persistent_transformer_train_amd import ofa
    cfg = cfg_of(name, exec_mode=exec_mode, **kw)
    init = init_of(name, cfg)
    h = ofa.Handle(cfg, init)
    if publish:
        v = h.publish()
        assert v == 1
    stream = stream_of(name, cfg)
    keep = cfg["prompt_len"]
    prompt = stream.prompt(keep)
    toks = torch.zeros(n_new, dtype=torch.int32, device="cuda")
    logits = torch.zeros(n_new, cfg["vocab"], dtype=torch.float32, device="cuda")
    vers = torch.zeros(n_new, dtype=torch.int64, device="cuda")
    h.decode(torch.from_numpy(prompt).cuda(), n_new, toks, logits, vers)
    h.sync()
    return h, cfg, init, prompt, toks.cpu().numpy(), logits.cpu().numpy(), vers.cpu().numpy()


def check_against_oracle(cfg, params_flat, prompt, toks, logits, dtype, logit_tol):
    s = spec_from_cfg(cfg)
    P = gpt.unflatten(s, np.asarray(params_flat, np.float64))
    win = cfg["decode_window"]
    keep = cfg["prompt_len"]
    z = decode.teacher_forced_logits(s, P, prompt, toks, win, keep, dtype=dtype)
    checked = 0
    for i in range(len(toks)):
        if decode.top2_margin(z[i]) > 1e-2:
            assert toks[i] == decode.argmax_lowest(z[i]), (i, toks[i], decode.argmax_lowest(z[i]))
            checked += 1
    err = np.abs(logits - z).max()
    log(f"decode: {checked}/{len(toks)} tokens checked, max |logit err| {err:.3g}")
    assert err <= logit_tol
    return checked


MODES = pytest.mark.parametrize("exec_mode", [1, 0], ids=["per_phase", "persistent"])


@MODES
@pytest.mark.parametrize("window", [64, 24])
def test_c1_fp32_decode(window, exec_mode):
    n_new = 60
    h, cfg, init, prompt, toks, logits, vers = run_decode("c1", n_new, exec_mode, decode_window=window)
    assert np.all(vers == 1)
    checked = check_against_oracle(cfg, init, prompt, toks, logits, np.float64, 1e-4)
    assert checked >= n_new // 2
    # continuing the context gives the same tokens as one longer call
    h.close()


@MODES
def test_c1_decode_continue_matches_single_call(exec_mode):
    from persistent_transformer_train_amd import ofa
    cfg = cfg_of("c1", exec_mode=exec_mode, decode_window=24)
    h = ofa.Handle(cfg, init_of("c1", cfg))
    prompt = torch.from_numpy(stream_of("c1", cfg).prompt(cfg["prompt_len"])).cuda()
    a = torch.zeros(40, dtype=torch.int32, device="cuda")
    h.decode(prompt, 40, a)
    b1 = torch.zeros(17, dtype=torch.int32, device="cuda")
    b2 = torch.zeros(23, dtype=torch.int32, device="cuda")
    h.decode(prompt, 17, b1)
    h.decode(None, 23, b2)
    h.sync()
    assert np.array_equal(a.cpu().numpy(), np.concatenate([b1.cpu().numpy(), b2.cpu().numpy()]))
    h.close()


@MODES
@pytest.mark.parametrize("name", ["m2", "m3"])
def test_bf16_mini_decode(name, exec_mode):
    # bf16 weights and KV cache: the oracle uses the same bf16-rounded weights
    n_new = 100
    h, cfg, init, prompt, toks, logits, vers = run_decode(name, n_new, exec_mode)
    w_bf16 = torch.tensor(init).to(torch.bfloat16).to(torch.float32).numpy()
    checked = check_against_oracle(cfg, w_bf16, prompt, toks, logits, np.float64, 5e-2)
    assert checked >= n_new // 4
    h.close()


def test_decode_after_training_reads_published_weights():
    from persistent_transformer_train_amd import ofa
    cfg = cfg_of("c1", exec_mode=0, decode_window=32)
    h = ofa.Handle(cfg, init_of("c1", cfg))
    stream = stream_of("c1", cfg)
    losses = torch.zeros(3, dtype=torch.float32, device="cuda")
    h.train_step(torch.from_numpy(stream.batches(0, 3)).cuda(), losses)
    v = h.publish()
    assert v == 1
    trained = h.get_params().cpu().numpy()
    h.train_step(torch.from_numpy(stream.batches(3, 2)).cuda(), losses)   # not published
    prompt = stream.prompt(cfg["prompt_len"])
    toks = torch.zeros(30, dtype=torch.int32, device="cuda")
    logits = torch.zeros(30, cfg["vocab"], dtype=torch.float32, device="cuda")
    vers = torch.zeros(30, dtype=torch.int64, device="cuda")
    h.decode(torch.from_numpy(prompt).cuda(), 30, toks, logits, vers)
    h.sync()
    assert np.all(vers.cpu().numpy() == 1)
    check_against_oracle(cfg, trained, prompt, toks.cpu().numpy(), logits.cpu().numpy(), np.float64, 1e-4)
    h.close()


@pytest.mark.parametrize("name", ["c4", "c2"])
def test_full_size_decode(name):
    # Full-size models, one persistent launch on 48 CUs, all 512 tokens after a
    # 32-token prompt: c4 is the decode workload the benchmark times (the 162M
    # model, 512-token window: after 480 generated tokens the context restarts
    # from its last 32 tokens, so the re-prefill and 32 tokens after it are
    # checked too); c2 takes the rotary, gated-MLP, tied-head path.  The oracle
    # recomputes the logits along the GPU's tokens (bf16 weights).
    n_new = 512
    h, cfg, init, prompt, toks, logits, vers = run_decode(name, n_new, exec_mode=0, serve_cus=48)
    assert np.all(vers == 1)
    w_bf16 = torch.tensor(init).to(torch.bfloat16).to(torch.float32).numpy()
    checked = check_against_oracle(cfg, w_bf16, prompt, toks, logits, np.float64, 2e-2)
    assert checked >= n_new // 2
    if name == "c4":
        # tokens after the window restart were checked as well: the first context
        # predicts 481 tokens (32 prompt tokens grow to 512 positions), the
        # restarted one the remaining 31
        segs = list(decode.windows(prompt, toks, cfg["decode_window"], cfg["prompt_len"]))
        assert len(segs) == 2 and len(segs[1][1]) == n_new - (cfg["decode_window"] - cfg["prompt_len"] + 1)
    h.close()


def test_read_ceiling_helper():
    """ofa_read_ceiling streams whole decode tiles on the given workgroups and
    rejects arguments it cannot use."""
    from persistent_transformer_train_amd import ofa
    buf = torch.zeros(48 * 24576 * 8 + 1000, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(48, dtype=torch.int32, device="cuda")
    gbps, us = ofa.read_ceiling(48, buf, sink, reps=2)
    log(f"read ceiling on 48 workgroups over {buf.numel()} bytes: {gbps:.1f} GB/s ({us:.1f} us)")
    assert gbps > 0 and us > 0
    small = torch.zeros(1000, dtype=torch.uint8, device="cuda")
    with pytest.raises(ofa.OfaError) as e:
        ofa.read_ceiling(48, small, sink, reps=1)
    assert e.value.code == ofa.OFA_E_ARG
    with pytest.raises(ofa.OfaError) as e:
        ofa.read_ceiling(0, buf, sink, reps=1)
    assert e.value.code == ofa.OFA_E_ARG
