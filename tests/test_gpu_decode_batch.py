"""Batch > 1 decode: several prompts of one length decoded together, each weight
tile streamed once per position for all of them (a serving variant: the news
page's "What happened" compares batch-one serving, the review page's "Fewer
launches do not guarantee fastest training" weighs one request at a time).

Each sequence's arithmetic is that of a batch-1 decode (same tiles, lanes and
reduction order), so a batch must reproduce, bit for bit, the tokens and
logits of decoding its prompts one at a time; the oracle checks each sequence
by teacher forcing."""

import numpy as np
import pytest

from gpu_common import cfg_of, init_of, log, spec_from_cfg, stream_of
from oracle import decode, gpt

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def decode_batch(name, nseq, n_new, exec_mode, **kw):
    from persistent_transformer_train_amd import ofa
    cfg = cfg_of(name, exec_mode=exec_mode, decode_batch=nseq, **kw)
    init = init_of(name, cfg)
    prompts = stream_of(name, cfg).prompts(nseq, cfg["prompt_len"])
    h = ofa.Handle(cfg, init)
    toks = torch.zeros(n_new, nseq, dtype=torch.int32, device="cuda")
    logits = torch.zeros(n_new, nseq, cfg["vocab"], dtype=torch.float32, device="cuda")
    vers = torch.zeros(n_new, dtype=torch.int64, device="cuda")
    h.decode(torch.from_numpy(prompts).cuda().contiguous(), n_new, toks, logits, vers)
    st = h.sync()
    h.close()
    return cfg, init, prompts, toks.cpu().numpy(), logits.cpu().numpy(), vers.cpu().numpy(), st


def decode_one(name, prompt, n_new, exec_mode, **kw):
    from persistent_transformer_train_amd import ofa
    cfg = cfg_of(name, exec_mode=exec_mode, **kw)
    h = ofa.Handle(cfg, init_of(name, cfg))
    toks = torch.zeros(n_new, dtype=torch.int32, device="cuda")
    logits = torch.zeros(n_new, cfg["vocab"], dtype=torch.float32, device="cuda")
    h.decode(torch.from_numpy(np.ascontiguousarray(prompt)).cuda(), n_new, toks, logits)
    h.sync()
    h.close()
    return toks.cpu().numpy(), logits.cpu().numpy()


@pytest.mark.parametrize("exec_mode", [1, 0], ids=["per_phase", "persistent"])
@pytest.mark.parametrize("name,nseq,window", [("c1", 4, 24), ("m3", 3, 40), ("m2", 2, 96)])
def test_batch_decode_equals_sequences_one_at_a_time(name, nseq, window, exec_mode):
    n_new = 50
    cfg, init, prompts, toks, logits, vers, _ = decode_batch(name, nseq, n_new, exec_mode, decode_window=window)
    assert np.all(vers == 0)
    for q in range(nseq):
        t1, l1 = decode_one(name, prompts[q], n_new, exec_mode, decode_window=window)
        assert np.array_equal(toks[:, q], t1), q
        assert logits[:, q].tobytes() == l1.tobytes(), q
    log(f"{name}: {nseq} sequences x {n_new} tokens equal to one-at-a-time decoding")


@pytest.mark.parametrize("name,nseq", [("c1", 4), ("m3", 3)])
def test_batch_decode_against_oracle(name, nseq):
    n_new = 40
    cfg, init, prompts, toks, logits, vers, _ = decode_batch(name, nseq, n_new, 0, decode_window=24)
    s = spec_from_cfg(cfg)
    w = np.asarray(init, np.float64)
    if cfg["precision"] == 1:   # bf16 weights
        w = torch.tensor(np.asarray(init, np.float32)).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    P = gpt.unflatten(s, w)
    tol, margin = (1e-4, 1e-4) if cfg["precision"] == 0 else (5e-2, 1e-2)
    checked = 0
    for q in range(nseq):
        z = decode.teacher_forced_logits(s, P, prompts[q], toks[:, q], cfg["decode_window"], cfg["prompt_len"])
        assert np.abs(logits[:, q] - z).max() <= tol
        for i in range(n_new):
            if decode.top2_margin(z[i]) > margin:
                assert toks[i, q] == decode.argmax_lowest(z[i]), (q, i)
                checked += 1
    log(f"{name}: {checked} of {nseq * n_new} tokens checked")
    assert checked >= nseq * n_new // 4


def test_full_size_batch_decode_c4():
    """The 162M model on 48 CUs, 8 prompts decoded together for 64 tokens: the
    first and last sequences equal their batch-1 decodes bit for bit, and every
    sequence matches the oracle (bf16 weights) wherever its margin is clear."""
    nseq, n_new = 8, 64
    cfg, init, prompts, toks, logits, vers, st = decode_batch("c4", nseq, n_new, 0)
    for q in (0, nseq - 1):
        t1, l1 = decode_one("c4", prompts[q], n_new, 0)
        assert np.array_equal(toks[:, q], t1), q
        assert logits[:, q].tobytes() == l1.tobytes(), q
    s = spec_from_cfg(cfg)
    w = torch.tensor(np.asarray(init, np.float32)).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    P = gpt.unflatten(s, w)
    checked = 0
    for q in range(nseq):
        z = decode.teacher_forced_logits(s, P, prompts[q], toks[:, q], cfg["decode_window"], cfg["prompt_len"])
        assert np.abs(logits[:, q] - z).max() <= 2e-2
        for i in range(n_new):
            if decode.top2_margin(z[i]) > 1e-2:
                assert toks[i, q] == decode.argmax_lowest(z[i]), (q, i)
                checked += 1
    log(f"c4 batch {nseq}: {checked} tokens checked; {st.last_call_ms:.1f} ms for {n_new} positions")
    assert checked >= nseq * n_new // 2
