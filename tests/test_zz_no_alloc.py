"""ofa_create_static: the entry point for callers that cannot allocate device
memory.  Its handle (workspace = the library's static per-device array) must
give the same results as a handle from ofa_create, on two creations in a row,
the second with a smaller model; a model too large for the array is rejected."""

import ctypes as C

import numpy as np
import pytest

from gpu_common import cfg_of, init_of, log, stream_of

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def run(cfg, static, n_steps=3, n_tok=8):
    from persistent_transformer_train_amd import ofa
    name = "c1"
    stream = stream_of(name, cfg)
    h = ofa.Handle(cfg, init_of(name, cfg), static=static)
    losses = torch.zeros(n_steps, dtype=torch.float32, device="cuda")
    h.train_step(torch.from_numpy(stream.batches(0, n_steps)).cuda(), losses)
    h.publish()
    toks = torch.zeros(n_tok, dtype=torch.int32, device="cuda")
    logits = torch.zeros(n_tok, cfg["vocab"], dtype=torch.float32, device="cuda")
    h.decode(torch.from_numpy(stream.prompt(cfg["prompt_len"])).cuda(), n_tok, toks, logits)
    h.sync()
    out = dict(losses=losses.cpu().numpy(), params=h.get_params().cpu().numpy(), grads=h.get_grads().cpu().numpy(),
               toks=toks.cpu().numpy(), logits=logits.cpu().numpy(), handle=h.h.value)
    return h, out


@pytest.mark.parametrize("exec_mode", [0, 1], ids=["persistent", "per_phase"])
def test_static_workspace_matches_caller_workspace(exec_mode):
    from persistent_transformer_train_amd import ofa
    big = cfg_of("c1", exec_mode=exec_mode)
    small = cfg_of("c1", exec_mode=exec_mode, batch=2, n_layer=1)   # the second, smaller model
    handles = []
    for cfg in (big, small):
        hr, ref = run(cfg, static=False)
        hs, got = run(cfg, static=True)
        log(f"{cfg['batch']}x{cfg['seq']}, {cfg['n_layer']} layers: losses {got['losses']} vs {ref['losses']}")
        for k in ("losses", "params", "grads", "toks", "logits"):
            assert got[k].tobytes() == ref[k].tobytes(), k
        handles.append(got["handle"])
        hr.close()
    # one static handle per device, re-created by each call
    assert handles[0] == handles[1]
    raw = hs.h
    assert ofa.ofa_destroy(raw) == ofa.OFA_OK
    toks = torch.zeros(1, 2, 65, dtype=torch.int32, device="cuda")
    losses = torch.zeros(1, dtype=torch.float32, device="cuda")
    assert ofa.ofa_train_step(raw, toks.data_ptr(), 1, losses.data_ptr()) == ofa.OFA_E_STATE
    hs.h = ofa._H()


def test_static_workspace_rejects_a_model_too_large():
    from persistent_transformer_train_amd import ofa
    cfg = cfg_of("c3")
    assert ofa.ofa_workspace_bytes(C.byref(ofa.make_config(cfg))) > (64 << 20)
    init = torch.zeros(ofa.ofa_param_count(C.byref(ofa.make_config(cfg))), dtype=torch.float32, device="cuda")
    h = ofa._H()
    rc = ofa.ofa_create_static(C.byref(ofa.make_config(cfg)), init.data_ptr(),
                               torch.cuda.current_stream().cuda_stream, C.byref(h))
    assert rc == ofa.OFA_E_ARG
    msg = ofa.ofa_last_error(h).decode()
    log(msg)
    assert "static" in msg
