"""Co-resident training and decoding in one persistent launch (the c5 mode),
through ofa_train_and_serve.

Training runs on its own CU partition with the same arithmetic as step mode, so
its losses and weights must equal a step-mode run bit for bit.  Decoding reads
the weights each training step publishes: versions never decrease, and every
token whose whole context (prompt prefill included) was computed under one
version must equal the oracle's greedy choice for that version's bf16 weights
wherever the oracle's top-2 margin exceeds 1e-2.
"""

import numpy as np
import pytest

from gpu_common import cfg_of, init_of, log, spec_from_cfg, stream_of
from oracle import decode, gpt

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

CO = dict(train_cus=32, serve_cus=16, restart_every=6, exec_mode=0)


def run_coresident(name, n_steps, ring=4096, **kw):
    from persistent_transformer_train_amd import ofa
    cfg = cfg_of(name, **dict(CO, **kw))
    stream = stream_of(name, cfg)
    init = init_of(name, cfg)
    h = ofa.Handle(cfg, init)
    toks = torch.from_numpy(stream.batches(0, n_steps)).cuda()
    losses = torch.zeros(n_steps, dtype=torch.float32, device="cuda")
    prompt = torch.from_numpy(stream.prompt(cfg["prompt_len"])).cuda()
    ring_t = torch.full((ring,), -1, dtype=torch.int32, device="cuda")
    ring_v = torch.zeros(ring, dtype=torch.int64, device="cuda")
    n_gen = torch.zeros(1, dtype=torch.int64, device="cuda")
    h.train_and_serve(toks, losses, prompt, ring_t, ring_v, n_gen)
    h.sync()
    out = dict(losses=losses.cpu().numpy(), params=h.get_params().cpu().numpy(), n_gen=int(n_gen.item()),
               tokens=ring_t.cpu().numpy(), versions=ring_v.cpu().numpy(), prompt=prompt.cpu().numpy(),
               version=h.publish())
    h.close()
    return cfg, stream, init, out


def step_mode_snapshots(name, n_steps, cfg, keep=None):
    """Step-mode training of the same model: losses and the fp32 weights after every
    step (only after the steps in `keep`, when given; other entries are None)."""
    from persistent_transformer_train_amd import ofa
    stream = stream_of(name, cfg)
    init = init_of(name, cfg)
    # the co-resident launch runs one workgroup per CU: the step-mode reference too
    h = ofa.Handle(dict(cfg, train_cus=0, serve_cus=0, debug_flags=cfg.get("debug_flags", 0) | ofa.OFA_DEBUG_OCC1),
                   init)
    snaps = [np.asarray(init, np.float32)]
    losses = torch.zeros(1, dtype=torch.float32, device="cuda")
    out = []
    for s in range(n_steps):
        h.train_step(torch.from_numpy(stream.batches(s, 1)).cuda(), losses)
        h.sync()
        out.append(float(losses.item()))
        snaps.append(h.get_params().cpu().numpy() if keep is None or s + 1 in keep else None)
    h.close()
    return np.array(out, np.float32), snaps


def test_coresident_training_equals_step_mode_and_decode_reads_live_weights():
    n_steps = 20
    log("co-resident m3: 32 train CUs, 16 serve CUs, 20 steps")
    cfg, stream, init, co = run_coresident("m3", n_steps)
    ref_losses, snaps = step_mode_snapshots("m3", n_steps, cfg)
    log("losses co-resident", co["losses"][[0, -1]], "step mode", ref_losses[[0, -1]])
    assert co["losses"].tobytes() == ref_losses.tobytes()
    assert co["params"].tobytes() == snaps[-1].tobytes()
    assert co["version"] == n_steps
    n = co["n_gen"]
    log(f"decode: {n} tokens, versions {co['versions'][:min(n, 4096)].min() if n else None}.."
        f"{co['versions'][:min(n, 4096)].max() if n else None}")
    assert 1 <= n <= 4096
    toks, vers = co["tokens"][:n], co["versions"][:n]
    assert np.all((toks >= 0) & (toks < cfg["vocab"]))
    assert np.all(np.diff(vers) >= 0)
    assert vers.min() >= 0 and vers.max() <= n_steps
    # oracle check of tokens whose whole restart period so far read one version
    s = spec_from_cfg(cfg)
    per = cfg["restart_every"]
    checked = 0
    for k in range(0, (n + per - 1) // per):
        tk, vk = toks[k * per:(k + 1) * per], vers[k * per:(k + 1) * per]
        same = int(np.argmax(vk != vk[0])) if np.any(vk != vk[0]) else len(vk)
        if same == 0:
            continue
        w = torch.tensor(snaps[int(vk[0])]).to(torch.bfloat16).to(torch.float32).numpy()
        P = gpt.unflatten(s, np.asarray(w, np.float64))
        z = decode.teacher_forced_logits(s, P, co["prompt"], tk[:same], cfg["decode_window"], cfg["prompt_len"])
        for i in range(same):
            if decode.top2_margin(z[i]) > 1e-2:
                assert tk[i] == decode.argmax_lowest(z[i]), (k, i, tk[i], decode.argmax_lowest(z[i]))
                checked += 1
    log(f"decode: {checked} tokens checked against the oracle at their version, "
        f"{len(np.unique(vers))} distinct versions read")
    # every period starts with one version (its prompt prefill and first token read the
    # version acquired at the restart), so at least its first token is checkable
    n_periods = (n + per - 1) // per
    assert checked >= max(3, n_periods // 2)


def test_coresident_publish_without_serving():
    """A co-resident configuration trained in step mode publishes every step (the
    slot guard does not wait when no decoder runs)."""
    from persistent_transformer_train_amd import ofa
    cfg = cfg_of("m3", **CO)
    stream = stream_of("m3", cfg)
    h = ofa.Handle(cfg, init_of("m3", cfg))
    losses = torch.zeros(3, dtype=torch.float32, device="cuda")
    h.train_step(torch.from_numpy(stream.batches(0, 3)).cuda(), losses)
    h.sync()
    assert h.publish() == 3
    # step-mode decode now reads version 3
    toks = torch.zeros(4, dtype=torch.int32, device="cuda")
    vers = torch.zeros(4, dtype=torch.int64, device="cuda")
    h.decode(torch.from_numpy(stream.prompt(cfg["prompt_len"])).cuda(), 4, toks, None, vers)
    h.sync()
    assert np.all(vers.cpu().numpy() == 3)
    h.close()


def test_full_size_coresident_c5():
    """The co-resident launch the benchmark times (the 162M model, 208 training and
    48 serving CUs, decode restarting from the prompt every 512 tokens), long enough
    for one restart: training equals step mode bit for bit, versions never decrease,
    and the tokens of each restart period that read the period's first version match
    the oracle on that version's weights."""
    n_steps = 70
    log("co-resident c5: 208 train CUs, 48 serve CUs, 70 steps, restart every 512 tokens")
    cfg, stream, init, co = run_coresident("c5", n_steps, train_cus=208, serve_cus=48, restart_every=512)
    n = co["n_gen"]
    toks, vers = co["tokens"][:n], co["versions"][:n]
    per = cfg["restart_every"]
    log(f"decode: {n} tokens, versions {vers.min()}..{vers.max()}")
    assert n > per, "no restart happened"
    starts = {int(vers[k * per]) for k in range((n + per - 1) // per)}
    ref_losses, snaps = step_mode_snapshots("c5", n_steps, cfg, keep=starts | {n_steps})
    assert co["losses"].tobytes() == ref_losses.tobytes()
    assert co["params"].tobytes() == snaps[-1].tobytes()
    assert co["version"] == n_steps
    assert np.all((toks >= 0) & (toks < cfg["vocab"]))
    assert np.all(np.diff(vers) >= 0)
    s = spec_from_cfg(cfg)
    checked = 0
    for k in range((n + per - 1) // per):
        tk, vk = toks[k * per:(k + 1) * per], vers[k * per:(k + 1) * per]
        same = int(np.argmax(vk != vk[0])) if np.any(vk != vk[0]) else len(vk)
        snap = snaps[int(vk[0])] if int(vk[0]) > 0 else np.asarray(init, np.float32)
        w = torch.tensor(snap).to(torch.bfloat16).to(torch.float32).numpy()
        P = gpt.unflatten(s, np.asarray(w, np.float64))
        z = decode.teacher_forced_logits(s, P, co["prompt"], tk[:same], cfg["decode_window"], cfg["prompt_len"])
        for i in range(same):
            if decode.top2_margin(z[i]) > 1e-2:
                assert tk[i] == decode.argmax_lowest(z[i]), (k, i, tk[i], decode.argmax_lowest(z[i]))
                checked += 1
        log(f"period {k}: version {int(vk[0])} for its first {same} tokens")
    log(f"decode: {checked} tokens checked against the oracle at their version")
    assert checked >= 2


def test_coresident_set_params_then_publish_makes_a_new_version():
    """In a co-resident configuration, weights set from outside become a new
    published version: publish copies them into the next weight slot, and a
    step-mode decode then reads that version and decodes the new weights."""
    from persistent_transformer_train_amd import ofa
    cfg = cfg_of("m3", **CO)
    stream = stream_of("m3", cfg)
    init = np.asarray(init_of("m3", cfg), np.float32)
    h = ofa.Handle(cfg, init)
    losses = torch.zeros(2, dtype=torch.float32, device="cuda")
    h.train_step(torch.from_numpy(stream.batches(0, 2)).cuda(), losses)
    h.sync()
    assert h.publish() == 2            # the steps published themselves
    new_w = (init * 1.5).astype(np.float32)
    h.set_params(torch.from_numpy(new_w))
    assert h.publish() == 3            # a new version, in slot 3 & 1
    n_new = 12
    prompt = stream.prompt(cfg["prompt_len"])
    toks = torch.zeros(n_new, dtype=torch.int32, device="cuda")
    logits = torch.zeros(n_new, cfg["vocab"], dtype=torch.float32, device="cuda")
    vers = torch.zeros(n_new, dtype=torch.int64, device="cuda")
    h.decode(torch.from_numpy(prompt).cuda(), n_new, toks, logits, vers)
    h.sync()
    assert np.all(vers.cpu().numpy() == 3)
    s = spec_from_cfg(cfg)
    w = torch.tensor(new_w).to(torch.bfloat16).to(torch.float32).numpy()
    z = decode.teacher_forced_logits(s, gpt.unflatten(s, np.asarray(w, np.float64)), prompt, toks.cpu().numpy(),
                                     cfg["decode_window"], cfg["prompt_len"])
    assert np.abs(logits.cpu().numpy() - z).max() <= 5e-2
    # training continues from the new weights and publishes version 4 next
    h.train_step(torch.from_numpy(stream.batches(2, 1)).cuda(), losses)
    h.sync()
    assert h.publish() == 4
    h.close()
